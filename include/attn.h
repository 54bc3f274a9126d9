/*
 * attn.h — C ABI of the fused scaled-dot-product attention forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (the "Fused attention kernel" page, Overview and
 * Implementation sketch): for every batch b, head h and query row i,
 *
 *     s_ij   = softmax_scale * <q_i, k_j>            for keys j in A_i
 *     O_i    = sum_j exp(s_ij) v_j / sum_j exp(s_ij)
 *     LSE_i  = ln sum_j exp(s_ij)
 *
 * one key block at a time with a running row maximum and row sum, so that the
 * score and probability matrices never reach device memory.  A_i is every key
 * of the sequence, intersected with {j <= i + Lk - Lq} when causal (masking is
 * aligned to the bottom-right corner; identical to j <= i when Lq == Lk).  A
 * row whose A_i is empty gets O_i = 0 and LSE_i = -inf.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing, keeps no per-call state and is safe to call
 *    from several host threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on that stream; nothing inside the library
 *    synchronises.  The caller keeps every buffer alive until the stream has
 *    run the work.
 *  - Element strides are given in ELEMENTS, as int64 triples
 *    {batch, seq, head}; the head_dim stride is always 1.
 *  - Arguments are validated on the host before anything is launched: on any
 *    error nothing is written.  Sizes of zero (batch, heads or sequence) are a
 *    no-op returning ATTN_OK.  Device-resident index arrays (cu_seqlens,
 *    block tables) are trusted: they must satisfy the stated invariants.
 *  - Accumulation is float32; O is rounded to nearest-even into its storage
 *    type; LSE is float32 in natural-log units.
 */
#ifndef ATTN_FWD_MI355X_H
#define ATTN_FWD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,      /* a null pointer, a negative size, a bad stride, a non-finite scale ... */
    ATTN_ERR_UNSUPPORTED = 2,  /* a valid request this build does not implement (e.g. head_dim 96) */
    ATTN_ERR_HIP = 3           /* the HIP runtime refused a launch */
} attn_status_t;

typedef enum {
    ATTN_BF16 = 0,
    ATTN_FP16 = 1
} attn_dtype_t;

/*
 * attn_fwd — 16-bit fused forward.
 * ("Fused attention kernel" page: Overview, Implementation sketch; the
 * FlashAttention-3 summary page: FP16 forward.)
 *
 * q: [B, Sq, H, D], k and v: [B, Sk, H, D], o: [B, Sq, H, D], all of `dtype`,
 * addressed as base + b*s[0] + i*s[1] + h*s[2] + d with s the stride triple.
 * lse: float32 [B, H, Sq] contiguous, or NULL to skip it.
 * D must be 64, 128 or 256 (ATTN_ERR_UNSUPPORTED otherwise); strides must be
 * multiples of 8 elements and pointers 16-byte aligned; the k and v sequence
 * strides must be at least D (rows may not overlap) and at most 2^24 elements
 * (ATTN_ERR_UNSUPPORTED above).
 * softmax_scale must be finite and > 0 (1/sqrt(D) is the usual choice).
 * causal: 0 or 1.
 */
attn_status_t attn_fwd(int dtype,
                       const void* q, const int64_t q_strides[3],
                       const void* k, const int64_t k_strides[3],
                       const void* v, const int64_t v_strides[3],
                       void* o, const int64_t o_strides[3],
                       float* lse,
                       int B, int H, int Sq, int Sk, int D,
                       float softmax_scale, int causal, void* stream);

/*
 * attn_fwd_ws — attn_fwd with a workspace, which lets the non-causal forward
 * at head dim 128 (4096 keys or more) split the last, partial round of its
 * grid by keys.
 * (The "Fused attention kernel" page's implementation sketch keeps a running
 * row max and row sum per query, so the partial results of key ranges merge
 * exactly through their logsumexps, as for attn_fwd_splitkv.)
 *
 * That forward runs in 256-row workgroups, one per compute unit.  When their
 * number is not a multiple of the device's compute units, the last round
 * would leave most of them idle; with a workspace, the work items of that
 * round instead run as up to 8 key ranges each, over the whole device, and a
 * merge combines them (two extra fp32 roundings of those rows' outputs).
 *
 * Arguments as for attn_fwd, plus:
 * workspace: device memory of at least attn_fwd_workspace_bytes(...) bytes
 *   for the same sizes, on the current device, 16-byte aligned, owned by the
 *   caller, free for this call only (it holds fp32 partial outputs and
 *   logsumexps).  workspace_bytes is its size; a smaller non-NULL workspace is
 *   an error.  NULL runs the schedule that needs none: attn_fwd itself.
 */
attn_status_t attn_fwd_ws(int dtype,
                          const void* q, const int64_t q_strides[3],
                          const void* k, const int64_t k_strides[3],
                          const void* v, const int64_t v_strides[3],
                          void* o, const int64_t o_strides[3],
                          float* lse,
                          int B, int H, int Sq, int Sk, int D,
                          float softmax_scale, int causal,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace attn_fwd_ws uses for these sizes on the current device (it
 * depends on the device's compute-unit count): 0 when the problem has no
 * split tail (causal, head dim 256, fewer than 4096 keys, a grid
 * of whole rounds, a last round more than half full, or invalid sizes), else
 * splits * tail_items * 256 * (D + 1) * 4 bytes. */
size_t attn_fwd_workspace_bytes(int dtype, int B, int H, int Sq, int Sk, int D, int causal);

/*
 * attn_fwd_bias — attn_fwd with an additive score bias: s = scale <q, k> +
 * bias[b, h, i, j] before the causal mask and the softmax (Bias is among the
 * features the StreamHPC case study, section "Our approach", adds to its
 * fused kernel).  -inf entries
 * exclude a key; a row whose keys are all excluded gets O = 0, LSE = -inf.
 *
 * bias: same dtype as q, element (b, h, i, j) at
 *   bias + b*bias_strides[0] + h*bias_strides[1] + i*bias_strides[2] + j
 *   (keys contiguous; a stride of 0 broadcasts over that index).  The strides
 *   must be multiples of 8 elements and the pointer 16-byte aligned; every
 *   row, the last one included, must be readable up to Sk rounded up to a
 *   multiple of 8 elements (padding values are never used); one (b, h) plane
 *   must span less than 2^31 bytes.
 * D must be 64 or 128 (ATTN_ERR_UNSUPPORTED otherwise).  Other arguments as
 * for attn_fwd.
 */
attn_status_t attn_fwd_bias(int dtype,
                            const void* q, const int64_t q_strides[3],
                            const void* k, const int64_t k_strides[3],
                            const void* v, const int64_t v_strides[3],
                            const void* bias, const int64_t bias_strides[3],
                            void* o, const int64_t o_strides[3], float* lse,
                            int B, int H, int Sq, int Sk, int D,
                            float softmax_scale, int causal, void* stream);

/*
 * attn_fp8_quantize — the 8-bit prologue for one tensor.
 * ("Fused attention kernel" page, section "8-bit forward pass": e4m3 format,
 * block quantisation, incoherent processing with a random-sign Hadamard
 * rotation.)
 *
 * x: bf16 [B, S, H, D] with stride triple x_strides.
 * signs: NULL, or int8 [D] of +-1 on the device: then every row is first
 *   rotated, x' = (x * signs) H_D / sqrt(D) with H_D the Sylvester Hadamard
 *   matrix (computed in float32 as a fast Walsh-Hadamard transform).
 * block_rows: 128 -> one scale per (b, h, block of 128 consecutive rows),
 *   scales float32 [B, H, ceil(S/128)];  0 -> one scale for the whole tensor,
 *   scales float32 [1].
 * Each scale is amax / 448 in float32 (1 for an all-zero block); each code is
 * e4m3fn(x' / scale) rounded to nearest-even and saturated to +-448.
 * x8: uint8 e4m3fn (OCP E4M3FN encoding) [B, S, H, D], contiguous.
 * Per-tensor mode uses `scales[0]` as its reduction cell; it is overwritten.
 */
attn_status_t attn_fp8_quantize(const void* x, const int64_t x_strides[3],
                                uint8_t* x8, float* scales,
                                int B, int H, int S, int D,
                                int block_rows, const int8_t* signs, void* stream);

/*
 * attn_fp8_quantize_pow2 — the 8-bit prologue with power-of-two block scales,
 * the input form of attn_fwd_fp8_pow2.  ("Fused attention kernel" page,
 * section "8-bit forward pass": one scale per block, whose format the section
 * leaves open; a power of two is a shared exponent, the block-scale form the
 * gfx950 matrix cores apply inside their products.)
 *
 * Arguments as for attn_fp8_quantize, plus
 * premul: finite and > 0; every (rotated) value is multiplied by it in
 *   float32, x'' = x' * premul, before the amax and the coding.  Pass 1 for K
 *   and V, and softmax_scale * log2(e) for Q: attn_fwd_fp8_pow2 takes the
 *   softmax scale from the Q codes (its scores are then base-2 exponents).
 * Each scale is a power of two: the smallest one at or above amax / 448 (the
 * quotient rounded to float32; amax of |x''| over the block), and at least
 * 2^-126; 1 for an all-zero block.  Each code is e4m3fn(x'' / scale) (an
 * exact division) rounded to nearest-even and saturated to +-448.
 */
attn_status_t attn_fp8_quantize_pow2(const void* x, const int64_t x_strides[3],
                                     uint8_t* x8, float* scales,
                                     int B, int H, int S, int D,
                                     int block_rows, const int8_t* signs, float premul,
                                     void* stream);

/*
 * attn_fwd_fp8 — 8-bit fused forward on quantised inputs.
 * ("Fused attention kernel" page, section "8-bit forward pass": both GEMMs in
 * e4m3, V tiles transposed on chip rather than in a global pass, per-block
 * scales.)
 *
 * q8: e4m3 [B, Sq, H, D] and k8, v8: e4m3 [B, Sk, H, D], contiguous, as
 * written by attn_fp8_quantize (with the same `signs` for q and k, none for v).
 * q_scale, k_scale, v_scale: float32, [B, H, ceil(S/128)] when block_rows is
 * 128, [1] when block_rows is 0.  The attention probabilities are also
 * rounded to e4m3 for the second GEMM.
 * o: bf16 [B, Sq, H, D] contiguous; lse: float32 [B, H, Sq] or NULL.
 * D must be 128.
 */
attn_status_t attn_fwd_fp8(const uint8_t* q8, const float* q_scale,
                           const uint8_t* k8, const float* k_scale,
                           const uint8_t* v8, const float* v_scale,
                           int block_rows,
                           void* o, float* lse,
                           int B, int H, int Sq, int Sk, int D,
                           float softmax_scale, int causal, void* stream);

/*
 * attn_fwd_fp8_pow2 — attn_fwd_fp8 on the power-of-two form: the block scales
 * enter the matrix-core products as their exponents, and the score products
 * return the exp2 argument directly (no multiply-add per score).
 *
 * q8, k8, v8 and their scales as written by attn_fp8_quantize_pow2: q with
 * premul = softmax_scale * log2(e), k and v with premul = 1 (the same `signs`
 * for q and k, none for v).  There is no softmax_scale argument: the Q codes
 * carry it.  Every scale must be a power of two in [2^-126, 2^127] (the kernel
 * reads a scale's exponent bits only).  Other arguments, outputs (lse: natural
 * log of the row sum of exp(softmax_scale q.k)) and errors as for
 * attn_fwd_fp8.
 */
attn_status_t attn_fwd_fp8_pow2(const uint8_t* q8, const float* q_scale,
                                const uint8_t* k8, const float* k_scale,
                                const uint8_t* v8, const float* v_scale,
                                int block_rows,
                                void* o, float* lse,
                                int B, int H, int Sq, int Sk, int D,
                                int causal, void* stream);

/*
 * attn_int8_quantize — the int8 prologue for Q or K.
 * (The StreamHPC case study lists an int8 path beside the fp8 one; the
 * "Fused attention kernel" page, section "8-bit forward pass", gives the block
 * quantisation and the random-sign Hadamard rotation it shares.)
 *
 * Arguments as for attn_fp8_quantize, except:
 * x8: int8 [B, S, H, D] contiguous; each scale is amax / 127 in float32 (1 for
 *   an all-zero block) and each code is x' / scale (a correctly rounded
 *   float32 division) rounded to nearest-even and clamped to [-127, 127].
 */
attn_status_t attn_int8_quantize(const void* x, const int64_t x_strides[3],
                                 int8_t* x8, float* scales,
                                 int B, int H, int S, int D,
                                 int block_rows, const int8_t* signs, void* stream);

/*
 * attn_fwd_int8 — fused forward with int8 scores.
 * (StreamHPC case study, "Our approach": an int8 path of the fused kernel;
 * the block scales and the rotation are those of the "Fused attention kernel"
 * page's 8-bit section.)  Q K^T runs on the int8 matrix cores and sums exactly
 * in int32; V and the probabilities keep the e4m3 format of attn_fwd_fp8
 * (a fixed-point int8 probability would round every key below 1/254 of the
 * row maximum to zero).
 *
 * q8: int8 [B, Sq, H, D], k8: int8 [B, Sk, H, D], both from
 *   attn_int8_quantize with the same `signs` (or none for both);
 * v8: e4m3 [B, Sk, H, D] from attn_fp8_quantize without rotation;
 * all contiguous, with scales as for attn_fwd_fp8 (all three with the same
 * block_rows).  Outputs, errors and D = 128 as for attn_fwd_fp8.
 */
attn_status_t attn_fwd_int8(const int8_t* q8, const float* q_scale,
                            const int8_t* k8, const float* k_scale,
                            const uint8_t* v8, const float* v_scale,
                            int block_rows,
                            void* o, float* lse,
                            int B, int H, int Sq, int Sk, int D,
                            float softmax_scale, int causal, void* stream);

/*
 * attn_fwd_varlen — packed variable-length batch, optionally with a paged KV
 * cache.  (The StreamHPC case study lists Paged Attention and Varlen Attention
 * among the features of its fused kernel.)
 *
 * q, o: [total_q, H, D] contiguous of `dtype`; cu_seqlens_q: int32 [B+1]
 * prefix sums, cu_seqlens_q[0] = 0, non-decreasing; sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and has Lk[b] = cu_seqlens_k[b+1] -
 * cu_seqlens_k[b] keys.
 * block_table == NULL: k, v are packed [total_k, H, D] contiguous, sequence b
 *   owning rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.
 * block_table != NULL: k, v are paged caches [num_pages, page_size, H, D]
 *   contiguous; key t of sequence b lives in page
 *   block_table[b * max_pages_per_seq + t / page_size] at slot t % page_size.
 *   page_size must be a power of two >= 16.  Only the entries a sequence needs
 *   are read, and slots past Lk[b] in its last page are never read.
 * lse: float32 [H, total_q] or NULL, total_q = cu_seqlens_q[B] (the caller
 * states it; it is the row count of q and o).  max_seqlen_q / max_seqlen_k
 * bound every sequence's lengths.
 */
attn_status_t attn_fwd_varlen(int dtype,
                              const void* q, const int32_t* cu_seqlens_q,
                              const void* k, const void* v,
                              const int32_t* cu_seqlens_k,
                              const int32_t* block_table, int max_pages_per_seq, int page_size,
                              void* o, float* lse,
                              int B, int H, int D, int total_q, int max_seqlen_q, int max_seqlen_k,
                              float softmax_scale, int causal, void* stream);

/*
 * attn_fwd_splitkv — attn_fwd_varlen with every sequence's keys cut into
 * num_splits ranges that run as separate work items, followed by a merge.
 * (The "Fused attention kernel" page's implementation sketch keeps a running
 * row max and row sum per query; the partial results of two key ranges merge
 * exactly through their logsumexps, L = ln(e^L1 + e^L2) and
 * O = e^(L1-L) O1 + e^(L2-L) O2.  The FlashAttention-3 summary page names
 * LLM inference as future work; short queries over long, paged key caches are
 * that case.)
 *
 * Arguments as for attn_fwd_varlen, plus:
 * num_splits >= 1: ranges of ceil(ceil(max_seqlen_k / 64) / num_splits) key
 *   tiles of 64 keys each; sequences shorter than max_seqlen_k leave their last
 *   ranges empty.  num_splits == 1 is attn_fwd_varlen itself and needs no
 *   workspace.
 * workspace: device memory of at least
 *   attn_fwd_splitkv_workspace_bytes(total_q, H, D, num_splits) bytes, 16-byte
 *   aligned, owned by the caller, free for this call only (it holds the
 *   partial outputs and logsumexps in fp32).  workspace_bytes is its size;
 *   a smaller workspace is an error.
 * The result is the same attention as attn_fwd_varlen up to floating-point
 * rounding (two extra fp32 roundings of the partial outputs).
 * Decoding (max_seqlen_q == 1) with B * H * num_splits >= 512 runs a streaming
 * kernel, one wave per (sequence, key range, head), at every head dim and page
 * size (attn_fwd_varlen takes it too when B * H >= 512); it reads K and V near
 * the device's streaming rate from about 1024 such items, so num_splits of
 * about 1024 / (B * H), with ranges of at least two tiles, suits it.
 */
attn_status_t attn_fwd_splitkv(int dtype,
                               const void* q, const int32_t* cu_seqlens_q,
                               const void* k, const void* v,
                               const int32_t* cu_seqlens_k,
                               const int32_t* block_table, int max_pages_per_seq, int page_size,
                               void* o, float* lse,
                               int B, int H, int D, int total_q, int max_seqlen_q, int max_seqlen_k,
                               float softmax_scale, int causal, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace attn_fwd_splitkv needs: num_splits * total_q * H * (D + 1) * 4
 * bytes (0 for num_splits <= 1 or an empty problem). */
size_t attn_fwd_splitkv_workspace_bytes(int total_q, int H, int D, int num_splits);

/* Size of the scratch attn_fwd_splitkv_noalloc keeps on each device. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * attn_fwd_splitkv_noalloc — attn_fwd_splitkv for callers that cannot
 * allocate device memory at call time: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as attn_fwd_splitkv without the workspace: the partial outputs
 * and logsumexps go to a scratch array of ATTN_NOALLOC_SCRATCH_BYTES (32 MiB)
 * that the library holds on each device it runs on until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); on its first call on a device it looks up that device's scratch
 * address (the current device, which must own `stream`).
 *
 * Limit: num_splits * total_q * H * (D + 1) * 4 bytes (what
 * attn_fwd_splitkv_workspace_bytes reports) must not exceed
 * ATTN_NOALLOC_SCRATCH_BYTES; a larger request returns ATTN_ERR_INVALID and
 * launches nothing.  num_splits == 1 uses no scratch.
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (other streams, other host threads) race and must be
 * serialised by the caller.  No part of the scratch needs to start at zero
 * (every partial result the merge reads is written by the same call).
 */
attn_status_t attn_fwd_splitkv_noalloc(int dtype,
                                       const void* q, const int32_t* cu_seqlens_q,
                                       const void* k, const void* v,
                                       const int32_t* cu_seqlens_k,
                                       const int32_t* block_table, int max_pages_per_seq, int page_size,
                                       void* o, float* lse,
                                       int B, int H, int D, int total_q, int max_seqlen_q, int max_seqlen_k,
                                       float softmax_scale, int causal, int num_splits, void* stream);

/*
 * attn_bwd — gradients of attn_fwd with respect to q, k and v.
 * (The FlashAttention-3 summary page reports a backward pass beside the
 * forward one; the "Fused attention kernel" page's "When to use which" says it
 * follows the same pattern.  The pages do not write it out: this is the chain
 * rule through O = softmax(scale q k^T [+ causal mask]) v.)
 *
 * With P recomputed from the forward's logsumexp, P = exp(scale q k^T - lse):
 *   dv = P^T dout,  dS = P * (dout v^T - delta),  delta_i = <dout_i, o_i>,
 *   dq = scale dS k,  dk = scale dS^T q.
 * q, o, dout, dq: [B, Sq, H, D]; k, v, dk, dv: [B, Sk, H, D]; all contiguous
 * of `dtype` (bf16 or fp16).  o and lse (float32 [B, H, Sq]) are the outputs of
 * attn_fwd on the same q, k, v, scale and mask.
 * workspace: float32 [2, B, H, Sq] scratch owned by the caller, 16-byte
 *   aligned, overwritten (delta, then lse * log2(e)).
 * D must be 64 or 128.  Masks as for attn_fwd (causal: bottom-right); rows
 * with no allowed key pass no gradient; with Sq = 0, dk and dv are zero.
 * The gradients are written once, with no atomics (run-to-run identical).
 */
attn_status_t attn_bwd(int dtype,
                       const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, float* workspace,
                       int B, int H, int Sq, int Sk, int D,
                       float softmax_scale, int causal, void* stream);

/*
 * attn_set_index_checks — debug switch for the device-resident index arrays
 * of attn_fwd_varlen, attn_fwd_splitkv and attn_fwd_splitkv_noalloc, which
 * are otherwise trusted.  With enable != 0 (process-wide; off by default)
 * each of those calls first copies cu_seqlens_q, cu_seqlens_k and the block
 * table to host memory on its stream, waits for the stream, and returns
 * ATTN_ERR_INVALID (launching nothing) unless attn_check_indices_host
 * accepts them.  The checked calls synchronise and use host memory.
 */
void attn_set_index_checks(int enable);

/*
 * attn_check_indices_host — the invariants of the index arrays, on HOST
 * copies: cu_seqlens_q[0] == 0 and cu_seqlens_k[0] >= 0, both non-decreasing,
 * every sequence's query and key counts within max_seqlen_q / max_seqlen_k,
 * cu_seqlens_q[B] == total_q, and (block_table != NULL) every sequence's
 * ceil(Lk / page_size) pages within max_pages_per_seq with non-negative
 * entries.  (Page ids above the cache's page count cannot be checked: the
 * library is not told that count.)  Returns ATTN_OK or ATTN_ERR_INVALID with
 * the first violation in attn_last_error().
 */
attn_status_t attn_check_indices_host(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      const int32_t* block_table, int max_pages_per_seq, int page_size,
                                      int B, int total_q, int max_seqlen_q, int max_seqlen_k);

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(int status);

/* Message describing the last error returned on the calling host thread. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_MI355X_H */
