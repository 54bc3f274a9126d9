/*
 * attn_probe.h — measured ceilings of the GPU the attention library runs on
 * (libattn_probe.so, built beside libattn_fwd.so; not part of the attention
 * path).  The roofline of the fused forward is set by the matrix-core rate at
 * the clock the chip sustains under load, and, for the online softmax, by the
 * issue cost of its vector instructions (the exponential, the scaling FMA,
 * the row-sum add, the row max, the conversions that pack the probabilities
 * for the second product).  The "Fused attention kernel" page (section "When
 * to use which") gives no such figures; they are measured here.
 *
 * attn_probe_ceilings(r, n): runs every probe on the current device,
 * synchronously, and writes n >= ATTN_PROBE_NUM doubles to the host array r,
 * indexed by the constants below.  It allocates a few MB of device memory for
 * its own outputs and frees them.  Returns 0, or 1 on any HIP error.
 *
 * Rates are chip-wide per second with every CU busy (8 waves per SIMD for the
 * vector and matrix rates).  *_LANE_OPS: instructions x 64 lanes per second
 * (one wave64 instruction counts 64).  The clock is the shader-clock counter
 * (s_memtime) against the 100 MHz real-time counter over the bf16 matrix run.
 * The *_MS entries are the durations (ms) of the overlap probes: ONE_WAVE: one
 * wave per SIMD issuing 4096 rounds of two bf16 32x32x16 products (MFMA), 16
 * exponentials (EXP16), or both in one stream with 8 or 16 exponentials per
 * round (MIX8, MIX16); TWO_WAVES: two waves per SIMD, one issuing 4096 rounds
 * of four products and one 8192 rounds of 8 exponentials, alone or together
 * (BOTH).
 */
#ifndef ATTN_PROBE_MI355X_H
#define ATTN_PROBE_MI355X_H

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ATTN_PROBE_EXP_LANE_OPS = 0,
    ATTN_PROBE_FMA_LANE_OPS,
    ATTN_PROBE_ADD_LANE_OPS,
    ATTN_PROBE_MAX3_LANE_OPS,
    ATTN_PROBE_CVT_FP8_LANE_OPS,
    ATTN_PROBE_CVT_BF16_LANE_OPS,
    ATTN_PROBE_RCP_LANE_OPS,
    ATTN_PROBE_MFMA_BF16_FLOPS,
    ATTN_PROBE_MFMA_FP8_FLOPS,
    ATTN_PROBE_MFMA_I8_OPS,
    ATTN_PROBE_CLOCK_GHZ,
    ATTN_PROBE_ONE_WAVE_MFMA_MS,
    ATTN_PROBE_ONE_WAVE_EXP16_MS,
    ATTN_PROBE_ONE_WAVE_MIX8_MS,
    ATTN_PROBE_ONE_WAVE_MIX16_MS,
    ATTN_PROBE_TWO_WAVES_MFMA_MS,
    ATTN_PROBE_TWO_WAVES_EXP_MS,
    ATTN_PROBE_TWO_WAVES_BOTH_MS,
    ATTN_PROBE_CUS,
    ATTN_PROBE_NUM
};

int attn_probe_ceilings(double* r, int n);

/*
 * attn_probe_cycles(r, n): shader-clock cycles counted inside each wave
 * (s_memtime around the loop; one workgroup per CU).  LAT_*: cycles per
 * instruction of one dependent chain (CVT_FP8_ROUNDTRIP: one packing
 * conversion plus one byte-to-float conversion).  BF16_* / FP8_*: one wave
 * per SIMD, cycles per round of one matrix product (bf16 32x32x16 or fp8
 * 32x32x64) plus N independent fma or exp instructions (MFMA: none).
 * PAIR_*: two waves per SIMD, one issuing 1024 rounds of four products, the
 * other 512 rounds of 16 independent exps or fmas; four entries each: the
 * product wave's cycles alone, the vector wave's alone, then both while they
 * run together.  SNOP15: counter ticks per `s_nop 15` (16 cycles of the
 * shader clock), which calibrates the counter.  WAVE_SIMDS: the SIMD of each
 * of the 8 waves of one pair workgroup, as 8 hexadecimal digits (wave 0
 * first).  FMA_Wk / EXP_Wk: SIMD cycles per fma / exp instruction with k
 * waves per SIMD issuing 16 independent chains each.  MFMA_PLUS_2FMA /
 * MFMA_PLUS_2EXP: the same with three waves per SIMD, one of them issuing
 * bf16 products instead (four accumulators); the _MFMA entry after each is
 * that wave's cycles per product.  PAIR_*_AGPR: the pair probes with the
 * products' accumulators in AGPRs (the _AGPR-less entries use VGPRs).
 * LDS_B128_Wk / LDS_TR16_Wk: bytes read from LDS per CU per cycle with k
 * waves per SIMD issuing independent conflict-free reads of 16 bytes per lane
 * (ds_read_b128) or 8 bytes per lane through the transposing read
 * (ds_read_b64_tr_b16; LDS_TR8_Wk: ds_read_b64_tr_b8).  DMA_L2 / DMA_HBM:
 * asynchronous global -> LDS copies (buffer_load_dwordx4 ... lds, 1 KB per
 * wave instruction) with two waves per SIMD, each wave issuing 8 copies and
 * waiting for them, from a 256 KB source every CU shares (L2) or from 4 MB
 * per CU (HBM); DMA_L2_ONE_WAVE: the L2 case with one wave per CU; three
 * entries each: bytes per CU per cycle, cycles a wave spends issuing one copy
 * instruction, and chip-wide GB/s.
 */
enum {
    ATTN_PROBE_CYC_LAT_EXP = 0,
    ATTN_PROBE_CYC_LAT_FMA,
    ATTN_PROBE_CYC_LAT_MAX3,
    ATTN_PROBE_CYC_LAT_CVT_FP8_ROUNDTRIP,
    ATTN_PROBE_CYC_BF16_MFMA,
    ATTN_PROBE_CYC_BF16_FMA8,
    ATTN_PROBE_CYC_BF16_FMA16,
    ATTN_PROBE_CYC_BF16_EXP4,
    ATTN_PROBE_CYC_BF16_EXP8,
    ATTN_PROBE_CYC_FP8_MFMA,
    ATTN_PROBE_CYC_FP8_FMA16,
    ATTN_PROBE_CYC_FP8_FMA32,
    ATTN_PROBE_CYC_FP8_EXP8,
    ATTN_PROBE_CYC_FP8_EXP16,
    ATTN_PROBE_CYC_PAIR_BF16_EXP,
    ATTN_PROBE_CYC_PAIR_BF16_FMA = ATTN_PROBE_CYC_PAIR_BF16_EXP + 4,
    ATTN_PROBE_CYC_PAIR_FP8_EXP = ATTN_PROBE_CYC_PAIR_BF16_FMA + 4,
    ATTN_PROBE_CYC_SNOP15 = ATTN_PROBE_CYC_PAIR_FP8_EXP + 4,
    ATTN_PROBE_CYC_WAVE_SIMDS,
    ATTN_PROBE_CYC_FMA_W1,
    ATTN_PROBE_CYC_FMA_W2,
    ATTN_PROBE_CYC_FMA_W3,
    ATTN_PROBE_CYC_FMA_W4,
    ATTN_PROBE_CYC_EXP_W1,
    ATTN_PROBE_CYC_EXP_W2,
    ATTN_PROBE_CYC_EXP_W3,
    ATTN_PROBE_CYC_EXP_W4,
    ATTN_PROBE_CYC_MFMA_PLUS_2FMA,
    ATTN_PROBE_CYC_MFMA_PLUS_2FMA_MFMA,
    ATTN_PROBE_CYC_MFMA_PLUS_2EXP,
    ATTN_PROBE_CYC_MFMA_PLUS_2EXP_MFMA,
    ATTN_PROBE_CYC_PAIR_BF16_FMA_AGPR,
    ATTN_PROBE_CYC_PAIR_FP8_FMA_AGPR = ATTN_PROBE_CYC_PAIR_BF16_FMA_AGPR + 4,
    ATTN_PROBE_CYC_PAIR_FP8_FMA = ATTN_PROBE_CYC_PAIR_FP8_FMA_AGPR + 4,
    ATTN_PROBE_CYC_LDS_B128_W1 = ATTN_PROBE_CYC_PAIR_FP8_FMA + 4,
    ATTN_PROBE_CYC_LDS_B128_W2,
    ATTN_PROBE_CYC_LDS_B128_W4,
    ATTN_PROBE_CYC_LDS_TR16_W1,
    ATTN_PROBE_CYC_LDS_TR16_W2,
    ATTN_PROBE_CYC_LDS_TR16_W4,
    ATTN_PROBE_CYC_LDS_TR8_W1,
    ATTN_PROBE_CYC_LDS_TR8_W2,
    ATTN_PROBE_CYC_LDS_TR8_W4,
    ATTN_PROBE_CYC_DMA_L2,
    ATTN_PROBE_CYC_DMA_HBM = ATTN_PROBE_CYC_DMA_L2 + 3,
    ATTN_PROBE_CYC_DMA_L2_ONE_WAVE = ATTN_PROBE_CYC_DMA_HBM + 3,
    ATTN_PROBE_CYC_NUM = ATTN_PROBE_CYC_DMA_L2_ONE_WAVE + 3
};

int attn_probe_cycles(double* r, int n);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_MI355X_H */
