// Measured ceilings of one MI355X (gfx950) for the attention kernels: the
// sustained shader clock under matrix load, the dense MFMA rates of the three
// operand types the forward uses, the issue cost of the vector instructions
// of the online softmax (exp2, fma, add, max3, the packing conversions), and
// whether exponentials run beside matrix products, from one wave or from two
// waves of one SIMD.  None of this is on the attention path: it bounds it.
//
// Every kernel runs a fixed count of independent instructions per lane and is
// timed with HIP events; the figures are per chip (all 256 CUs busy).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <vector>

#include "../../include/attn_probe.h"

namespace probe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

enum ValuOp { kExp = 0, kFma, kAdd, kMax3, kCvtFp8, kCvtBf16, kRcp, kNumValu };

// Eight independent registers per lane, `iters` rounds of one instruction on
// each: a throughput figure (the chains are 8 instructions apart).
template <int OP>
__global__ void __launch_bounds__(256) valu_kernel(float* out, int iters, float seed) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = seed + 0.01f * (threadIdx.x + i);
  const float a = 0.999f, b = 1e-3f;
  uint32_t u[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (OP == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
      else if constexpr (OP == kFma) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
      else if constexpr (OP == kAdd) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x[i]) : "v"(b));
      else if constexpr (OP == kMax3) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
      else if constexpr (OP == kCvtFp8) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "+v"(u[i]) : "v"(x[i]), "v"(a));
      else if constexpr (OP == kCvtBf16) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "+v"(u[i]) : "v"(x[i]), "v"(a));
      else asm volatile("v_rcp_f32 %0, %0" : "+v"(x[i]));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + (float)u[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

enum MfmaKind { kBf16 = 0, kFp8, kI8, kNumMfma };

// Four independent accumulators per wave, `iters` rounds of one product on
// each.  Thread 0 of every workgroup records the shader-clock and real-time
// (100 MHz) counters around its loop.
template <int KIND>
__global__ void __launch_bounds__(256) mfma_kernel(float* out, uint64_t* clk, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[4] = {};
  i32x16 iacc[4] = {};
  i32x8 a8, b8;
  i32x4 a4, b4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a8[i] = 0x38383838 ^ (lane << i);
    b8[i] = 0x30303030 + i;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a4[i] = a8[i];
    b4[i] = b8[i];
  }
  const bf16x8 ab = __builtin_bit_cast(bf16x8, a4), bb = __builtin_bit_cast(bf16x8, b4);
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (KIND == kBf16) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[j], 0, 0, 0);
      else if constexpr (KIND == kFp8)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 0, 0, 0, 127, 0, 127);
      else iacc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, iacc[j], 0, 0, 0);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r] + (float)iacc[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Matrix products and exponentials together.  One workgroup of 4 waves per CU
// (its LDS request keeps a second one off the CU), so every SIMD holds ONE
// wave: per round two independent bf16 products and 2 * NEXP exponentials on
// independent registers, issued in program order.  NEXP = 0 is the products
// alone; MFMA = false drops the products.
template <int NEXP, bool MFMA>
__global__ void __launch_bounds__(256) mix_one_wave_kernel(float* out, int iters) {
  extern __shared__ float lds_hold[];
  const int lane = threadIdx.x & 63;
  f32x16 acc0 = {}, acc1 = {};
  i32x4 a4 = {0x3f803f80 ^ lane, 0x3f003f00, 0x3e803e80, 0x3f803f80};
  const bf16x8 ab = __builtin_bit_cast(bf16x8, a4);
  float x[NEXP > 0 ? 2 * NEXP : 1];
#pragma unroll
  for (int i = 0; i < (NEXP > 0 ? 2 * NEXP : 1); ++i) x[i] = 0.01f * (lane + i);
  for (int it = 0; it < iters; ++it) {
    if constexpr (MFMA) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
    if constexpr (MFMA) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc1, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[NEXP + i]));
  }
  float s = lds_hold[0] * 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r];
#pragma unroll
  for (int i = 0; i < (NEXP > 0 ? 2 * NEXP : 1); ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Two waves on every SIMD: one workgroup of 8 waves per CU; waves 0-3 (one per
// SIMD) issue only bf16 products, waves 4-7 only exponentials (MODE 1 =
// products only, 2 = exponentials only, 3 = both).
template <int MODE>
__global__ void __launch_bounds__(512) mix_two_waves_kernel(float* out, int iters) {
  extern __shared__ float lds_hold[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float s = lds_hold[0] * 0.f;
  if (wave < 4) {
    if constexpr ((MODE & 1) != 0) {
      f32x16 acc[4] = {};
      i32x4 a4 = {0x3f803f80 ^ lane, 0x3f003f00, 0x3e803e80, 0x3f803f80};
      const bf16x8 ab = __builtin_bit_cast(bf16x8, a4);
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    }
  } else if constexpr ((MODE & 2) != 0) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.01f * (lane + i);
    // 16 exponentials per product round of the other wave (4 products)
    for (int it = 0; it < 2 * iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ---- cycle-counted probes (s_memtime around the loop, per wave) ------------
// One workgroup per CU (its LDS request keeps others off), 4 or 8 waves: with
// 8, waves w and w + 4 share SIMD w % 4.  Every wave records its own cycles.
//
// Latency: one dependent chain of `iters` instructions.
template <int OP>
__global__ void __launch_bounds__(256) latency_kernel(float* out, uint64_t* cyc, int iters) {
  extern __shared__ float lds_hold[];
  float x = 0.001f * threadIdx.x + lds_hold[0] * 0.f;
  uint32_t u = 0;
  const float a = 0.999f, b = 1e-3f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (OP == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(x));
      else if constexpr (OP == kFma) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
      else if constexpr (OP == kCvtFp8) {
        // the packed bytes feed the next conversion's input
        asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "+v"(u) : "v"(x), "v"(a));
        asm volatile("v_cvt_f32_ubyte0 %0, %1" : "=v"(x) : "v"(u));
      } else if constexpr (OP == kMax3) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
      else asm volatile("s_nop 15");  // 16 cycles, no data: calibrates the counter
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = x + (float)u;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

// One wave per SIMD: every round one matrix product (bf16 32x32x16, or fp8
// 32x32x64 when FP8) on one of two accumulators, then NV vector instructions
// (exp when EXP, else fma) on independent registers.
template <bool FP8, bool EXP, int NV>
__global__ void __launch_bounds__(256) mix_cycles_kernel(float* out, uint64_t* cyc, int iters) {
  extern __shared__ float lds_hold[];
  const int lane = threadIdx.x & 63;
  f32x16 acc0 = {}, acc1 = {};
  i32x8 a8;
#pragma unroll
  for (int i = 0; i < 8; ++i) a8[i] = 0x38383838 ^ (lane << i);
  const i32x4 a4 = {a8[0], a8[1], a8[2], a8[3]};
  const bf16x8 ab = __builtin_bit_cast(bf16x8, a4);
  float x[NV > 0 ? NV : 1];
#pragma unroll
  for (int i = 0; i < (NV > 0 ? NV : 1); ++i) x[i] = 0.01f * (lane + i) + lds_hold[0] * 0.f;
  const float a = 0.999f, b = 1e-3f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  auto vec = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if constexpr (EXP) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
      else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
    }
  };
  for (int it = 0; it < iters; it += 2) {
    if constexpr (FP8) acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, acc0, 0, 0, 0, 127, 0, 127);
    else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc0, 0, 0, 0);
    vec();
    if constexpr (FP8) acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, acc1, 0, 0, 0, 127, 0, 127);
    else acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc1, 0, 0, 0);
    vec();
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r];
#pragma unroll
  for (int i = 0; i < (NV > 0 ? NV : 1); ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 4 + threadIdx.x / 64] = t1 - t0;
}

// Two waves per SIMD (8-wave workgroup, one per CU): waves 0-3 issue matrix
// products only (four accumulators, bf16 or fp8), waves 4-7 vector
// instructions only (16 independent exps or fmas per round).  MODE 1 =
// products alone, 2 = vector alone, 3 = both.  Each wave reports its cycles.
template <bool FP8, bool EXP, int MODE, bool AGPR = false>
__global__ void __launch_bounds__(512) pair_cycles_kernel(float* out, uint64_t* cyc, int m_iters, int v_iters) {
  extern __shared__ float lds_hold[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float s = lds_hold[0] * 0.f;
  uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (wave < 4) {
    if constexpr ((MODE & 1) != 0) {
      f32x16 acc[4] = {};
      i32x8 a8;
#pragma unroll
      for (int i = 0; i < 8; ++i) a8[i] = 0x38383838 ^ (lane << i);
      const i32x4 a4 = {a8[0], a8[1], a8[2], a8[3]};
      const bf16x8 ab = __builtin_bit_cast(bf16x8, a4);
      t0 = __builtin_amdgcn_s_memtime();
      for (int it = 0; it < m_iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (AGPR) {
            // accumulators held in AGPRs
            if constexpr (FP8)
              asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a8), "v"(a8));
            else
              asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(ab), "v"(ab));
          } else if constexpr (FP8) {
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, acc[j], 0, 0, 0, 127, 0, 127);
          } else {
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc[j], 0, 0, 0);
          }
        }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    }
  } else if constexpr ((MODE & 2) != 0) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.01f * (lane + i);
    const float a = 0.999f, b = 1e-3f;
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < v_iters; ++it)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (EXP) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
        else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 8 + wave] = t1 - t0;
  // HW_ID (hardware register 4): the SIMD this wave runs on is bits 5:4
  if (lane == 0 && blockIdx.x == 0) cyc[(size_t)gridDim.x * 8 + wave] = __builtin_amdgcn_s_getreg((31 << 11) | 4);
}

// Vector throughput against waves per SIMD: one workgroup of 4 K waves per
// CU (K waves on every SIMD), each wave 16 independent chains.  With MFMA,
// wave 0 of each SIMD issues bf16 products instead (four accumulators).
template <int OP, bool MFMA>
__global__ void __launch_bounds__(1024) waves_kernel(float* out, uint64_t* cyc, int iters) {
  extern __shared__ float lds_hold[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float s = lds_hold[0] * 0.f;
  uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (MFMA && wave < 4) {
    f32x16 acc[4] = {};
    i32x4 a4 = {0x3f803f80 ^ lane, 0x3f003f00, 0x3e803e80, 0x3f803f80};
    const bf16x8 ab = __builtin_bit_cast(bf16x8, a4);
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < 4 * iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[j][r];
  } else {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.01f * (lane + i);
    const float a = 0.999f, b = 1e-3f;
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (OP == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i]));
        else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b));
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 16 + wave] = t1 - t0;
}


// LDS read bandwidth: one workgroup of 4 K waves per CU, each wave `iters`
// rounds of 16 independent reads of 16 bytes per lane (ds_read_b128, TR = 0)
// or of 8 bytes per lane through a transposing read (ds_read_b64_tr_b16, TR
// = 1; ds_read_b64_tr_b8, TR = 2), consecutive lanes at consecutive addresses
// (no bank conflicts); the values are folded with xor so that no read is dead.
template <int TR>
__global__ void __launch_bounds__(1024) lds_read_kernel(uint32_t* out, uint64_t* cyc, int iters) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];  // 64 KiB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int base = (wave & 3) * 4096;  // words: each wave reads its own 16 KiB
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (TR == 1) {
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const uint32_t* p = buf + base + ((i * 128 + 2 * lane + 2 * it) & 4094);  // 8-byte aligned
        const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
        const u32x2 u = __builtin_bit_cast(u32x2, v);
        acc[0] ^= u[0];
        acc[1] ^= u[1];
      } else if constexpr (TR == 2) {
        typedef int v2i __attribute__((vector_size(8)));
        typedef __attribute__((address_space(3))) v2i lds_v2i;
        const uint32_t* p = buf + base + ((i * 128 + 2 * lane + 2 * it) & 4094);  // 8-byte aligned
        const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
        const u32x2 u = __builtin_bit_cast(u32x2, v);
        acc[0] ^= u[0];
        acc[1] ^= u[1];
      } else {
        const u32x4 v = *(const u32x4*)(buf + base + ((i * 256 + 4 * lane + 4 * it) & 4095));
        acc ^= v;
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (lane == 0) cyc[blockIdx.x * 16 + wave] = t1 - t0;
}


// Asynchronous global -> LDS copies (buffer_load_dwordx4 ... lds, 16 bytes
// per lane, 1 KB per wave instruction): one workgroup of up to 8 waves per CU,
// each wave `iters` rounds of 8 copies into its own 8 KB of LDS, then a wait
// for them.  The source is one buffer resource of `bytes` per workgroup at
// `stride` bytes from the previous workgroup's (stride 0: every CU copies the
// same bytes, which then come from L2; a stride past the data: HBM); a wave
// walks its slice round by round, wrapping inside the resource, so every copy
// stays in bounds.  Per wave: the cycles of the whole loop (cyc[.. + 0]) and
// of the copy instructions' issue alone (cyc[.. + 16]).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ void buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
                                int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__global__ void __launch_bounds__(512) lds_dma_kernel(const uint8_t* src, uint32_t bytes, uint32_t stride,
                                                       uint64_t* cyc, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lbuf[8 * 8192];  // 8 KB per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint64_t base = (uint64_t)(src + (uint64_t)blockIdx.x * stride);
  const i32x4 rsrc = {(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), (int)bytes, 0x00020000};
  const uint32_t slice = bytes / 8192u;  // 8 KB slices in the resource
  uint64_t issue = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const uint32_t off0 = ((uint32_t)(wave + 8 * it) % slice) * 8192u + 16u * (uint32_t)lane;
    __builtin_amdgcn_sched_barrier(0);
    const uint64_t a = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lbuf + wave * 8192 + i * 1024), 16,
                      (int)(off0 + 1024u * (uint32_t)i), 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    const uint64_t b = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_sched_barrier(0);
    issue += b - a;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    cyc[blockIdx.x * 32 + wave] = t1 - t0;
    cyc[blockIdx.x * 32 + 16 + wave] = issue;
  }
}

}  // namespace probe

namespace {

struct Timer {
  hipEvent_t a, b;
  Timer() {
    (void)hipEventCreate(&a);
    (void)hipEventCreate(&b);
  }
  ~Timer() {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
  }
};

template <class F>
int timed(F launch, double* ms) {
  Timer t;
  launch();  // warm-up
  if (hipDeviceSynchronize() != hipSuccess) return 1;
  if (hipEventRecord(t.a, 0) != hipSuccess) return 1;
  launch();
  if (hipEventRecord(t.b, 0) != hipSuccess) return 1;
  if (hipEventSynchronize(t.b) != hipSuccess) return 1;
  float f = 0.f;
  if (hipEventElapsedTime(&f, t.a, t.b) != hipSuccess) return 1;
  *ms = f;
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

namespace {

// mean of the first `per` counters of each of `n` workgroups, starting at `first`
double mean_cycles(const uint64_t* d_cyc, int n, int stride, int first, int per, int* err) {
  std::vector<uint64_t> h((size_t)n * stride);
  if (hipMemcpy(h.data(), d_cyc, sizeof(uint64_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess) {
    *err = 1;
    return 0.0;
  }
  double s = 0.0;
  for (int b = 0; b < n; ++b)
    for (int w = first; w < first + per; ++w) s += (double)h[(size_t)b * stride + w];
  return s / ((double)n * per);
}

}  // namespace

extern "C" int attn_probe_cycles(double* r, int n) {
  using namespace probe;
  if (r == nullptr || n < ATTN_PROBE_CYC_NUM) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 1;
  float* out = nullptr;
  uint64_t* cyc = nullptr;
  if (hipMalloc(&out, sizeof(float) * (size_t)cus * 1024) != hipSuccess) return 1;
  if (hipMalloc(&cyc, sizeof(uint64_t) * ((size_t)cus * 32 + 8)) != hipSuccess) {
    (void)hipFree(out);
    return 1;
  }
  int err = 0;
  double ms = 0.0;
  const size_t hold = 96 * 1024;  // one workgroup per CU
  const int it = 2048;
  auto lat = [&](auto op, int slot) {
    constexpr int OP = decltype(op)::value;
    err |= timed([&] { hipLaunchKernelGGL((latency_kernel<OP>), dim3(cus), dim3(256), hold, 0, out, cyc, it); }, &ms);
    r[slot] = mean_cycles(cyc, cus, 4, 0, 4, &err) / (16.0 * it);
  };
  lat(std::integral_constant<int, kExp>{}, ATTN_PROBE_CYC_LAT_EXP);
  lat(std::integral_constant<int, kFma>{}, ATTN_PROBE_CYC_LAT_FMA);
  lat(std::integral_constant<int, kMax3>{}, ATTN_PROBE_CYC_LAT_MAX3);
  lat(std::integral_constant<int, kCvtFp8>{}, ATTN_PROBE_CYC_LAT_CVT_FP8_ROUNDTRIP);
  lat(std::integral_constant<int, kNumValu>{}, ATTN_PROBE_CYC_SNOP15);
  // one wave per SIMD, one product plus NV vector instructions per round
  auto mix = [&](auto fp8, auto exp, auto nv, int slot) {
    constexpr bool F = decltype(fp8)::value, E = decltype(exp)::value;
    constexpr int NV = decltype(nv)::value;
    err |= timed([&] { hipLaunchKernelGGL((mix_cycles_kernel<F, E, NV>), dim3(cus), dim3(256), hold, 0, out, cyc, it); }, &ms);
    r[slot] = mean_cycles(cyc, cus, 4, 0, 4, &err) / it;
  };
  using T = std::true_type;
  using Fa = std::false_type;
  mix(Fa{}, Fa{}, std::integral_constant<int, 0>{}, ATTN_PROBE_CYC_BF16_MFMA);
  mix(Fa{}, Fa{}, std::integral_constant<int, 8>{}, ATTN_PROBE_CYC_BF16_FMA8);
  mix(Fa{}, Fa{}, std::integral_constant<int, 16>{}, ATTN_PROBE_CYC_BF16_FMA16);
  mix(Fa{}, T{}, std::integral_constant<int, 4>{}, ATTN_PROBE_CYC_BF16_EXP4);
  mix(Fa{}, T{}, std::integral_constant<int, 8>{}, ATTN_PROBE_CYC_BF16_EXP8);
  mix(T{}, Fa{}, std::integral_constant<int, 0>{}, ATTN_PROBE_CYC_FP8_MFMA);
  mix(T{}, Fa{}, std::integral_constant<int, 16>{}, ATTN_PROBE_CYC_FP8_FMA16);
  mix(T{}, Fa{}, std::integral_constant<int, 32>{}, ATTN_PROBE_CYC_FP8_FMA32);
  mix(T{}, T{}, std::integral_constant<int, 8>{}, ATTN_PROBE_CYC_FP8_EXP8);
  mix(T{}, T{}, std::integral_constant<int, 16>{}, ATTN_PROBE_CYC_FP8_EXP16);
  // two waves per SIMD: products beside vector instructions
  auto pair = [&](auto fp8, auto exp, int slot, auto agpr) {
    constexpr bool F = decltype(fp8)::value, E = decltype(exp)::value, G = decltype(agpr)::value;
    const int mi = 1024, vi = 512;
    double m_alone, v_alone;
    err |= timed([&] { hipLaunchKernelGGL((pair_cycles_kernel<F, E, 1, G>), dim3(cus), dim3(512), hold, 0, out, cyc, mi, vi); }, &ms);
    m_alone = mean_cycles(cyc, cus, 8, 0, 4, &err);
    err |= timed([&] { hipLaunchKernelGGL((pair_cycles_kernel<F, E, 2, G>), dim3(cus), dim3(512), hold, 0, out, cyc, mi, vi); }, &ms);
    v_alone = mean_cycles(cyc, cus, 8, 4, 4, &err);
    err |= timed([&] { hipLaunchKernelGGL((pair_cycles_kernel<F, E, 3, G>), dim3(cus), dim3(512), hold, 0, out, cyc, mi, vi); }, &ms);
    r[slot] = m_alone;
    r[slot + 1] = v_alone;
    r[slot + 2] = mean_cycles(cyc, cus, 8, 0, 4, &err);
    r[slot + 3] = mean_cycles(cyc, cus, 8, 4, 4, &err);
    // SIMD of each of the 8 waves of workgroup 0, as 8 hex digits
    uint64_t ids[8];
    err |= hipMemcpy(ids, cyc + (size_t)cus * 8, sizeof ids, hipMemcpyDeviceToHost) != hipSuccess;
    double code = 0.0;
    for (int w = 0; w < 8; ++w) code = code * 16.0 + (double)((ids[w] >> 4) & 3);
    r[ATTN_PROBE_CYC_WAVE_SIMDS] = code;
  };
  // vector instructions per SIMD per cycle-block against waves per SIMD
  auto waves = [&](auto op, auto mfma, int k, int slot) {
    constexpr int OP = decltype(op)::value;
    constexpr bool M = decltype(mfma)::value;
    const int vi = 512;
    err |= timed([&] { hipLaunchKernelGGL((waves_kernel<OP, M>), dim3(cus), dim3(256 * k), hold, 0, out, cyc, vi); }, &ms);
    // cycles of the vector waves; SIMD cycles per vector instruction
    const int first = M ? 4 : 0, nvec = 4 * k - first;
    const double c = mean_cycles(cyc, cus, 16, first, nvec, &err);
    r[slot] = c / (16.0 * vi * (nvec / 4.0));
    if (M) r[slot + 1] = mean_cycles(cyc, cus, 16, 0, 4, &err) / (4.0 * 4 * vi);  // cycles per product
  };
  for (int k = 1; k <= 4; ++k) {
    waves(std::integral_constant<int, kFma>{}, Fa{}, k, ATTN_PROBE_CYC_FMA_W1 + k - 1);
    waves(std::integral_constant<int, kExp>{}, Fa{}, k, ATTN_PROBE_CYC_EXP_W1 + k - 1);
  }
  // LDS bytes read per CU per cycle (over the mean wave's cycle count)
  auto lds = [&](auto tr, int k, int slot) {
    constexpr int TR = decltype(tr)::value;
    const int li = 256;
    err |= timed([&] { hipLaunchKernelGGL((lds_read_kernel<TR>), dim3(cus), dim3(256 * k), 0, 0, (uint32_t*)out, cyc, li); }, &ms);
    const double c = mean_cycles(cyc, cus, 16, 0, 4 * k, &err);
    r[slot] = (double)(4 * k) * li * 16 * 64 * (TR ? 8 : 16) / c;
  };
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  lds(M0{}, 1, ATTN_PROBE_CYC_LDS_B128_W1);
  lds(M0{}, 2, ATTN_PROBE_CYC_LDS_B128_W2);
  lds(M0{}, 4, ATTN_PROBE_CYC_LDS_B128_W4);
  lds(M1{}, 1, ATTN_PROBE_CYC_LDS_TR16_W1);
  lds(M1{}, 2, ATTN_PROBE_CYC_LDS_TR16_W2);
  lds(M1{}, 4, ATTN_PROBE_CYC_LDS_TR16_W4);
  lds(M2{}, 1, ATTN_PROBE_CYC_LDS_TR8_W1);
  lds(M2{}, 2, ATTN_PROBE_CYC_LDS_TR8_W2);
  lds(M2{}, 4, ATTN_PROBE_CYC_LDS_TR8_W4);
  // global -> LDS copies, 2 waves per SIMD: from L2 (every CU copies the same
  // 256 KB) and streaming from HBM (each CU its own 4 MB, 1 GB in all)
  {
    const uint32_t l2_bytes = 256u << 10, hbm_bytes = 4u << 20;
    uint8_t* src = nullptr;
    const size_t total = (size_t)cus * hbm_bytes;
    if (hipMalloc(&src, total) != hipSuccess) {
      err = 1;
    } else {
      err |= hipMemset(src, 0, total) != hipSuccess;
      auto dma = [&](uint32_t bytes, uint32_t stride, int waves, int slot) {
        const int di = 256;
        err |= timed([&] { hipLaunchKernelGGL(lds_dma_kernel, dim3(cus), dim3(64 * waves), 0, 0, src, bytes, stride, cyc, di); }, &ms);
        const double c = mean_cycles(cyc, cus, 32, 0, waves, &err), iss = mean_cycles(cyc, cus, 32, 16, waves, &err);
        r[slot] = (double)waves * di * 8 * 1024 / c;  // bytes per CU per cycle
        r[slot + 1] = iss / (8.0 * di);               // issue cycles per copy instruction
        r[slot + 2] = (double)cus * waves * di * 8 * 1024 / (ms * 1e-3) / 1e9;  // GB/s, whole chip
      };
      dma(l2_bytes, 0, 8, ATTN_PROBE_CYC_DMA_L2);
      dma(hbm_bytes, hbm_bytes, 8, ATTN_PROBE_CYC_DMA_HBM);
      dma(l2_bytes, 0, 1, ATTN_PROBE_CYC_DMA_L2_ONE_WAVE);
      (void)hipFree(src);
    }
  }
  waves(std::integral_constant<int, kFma>{}, T{}, 3, ATTN_PROBE_CYC_MFMA_PLUS_2FMA);
  waves(std::integral_constant<int, kExp>{}, T{}, 3, ATTN_PROBE_CYC_MFMA_PLUS_2EXP);
  pair(Fa{}, T{}, ATTN_PROBE_CYC_PAIR_BF16_EXP, Fa{});
  pair(Fa{}, Fa{}, ATTN_PROBE_CYC_PAIR_BF16_FMA, Fa{});
  pair(T{}, T{}, ATTN_PROBE_CYC_PAIR_FP8_EXP, Fa{});
  pair(Fa{}, Fa{}, ATTN_PROBE_CYC_PAIR_BF16_FMA_AGPR, T{});
  pair(T{}, Fa{}, ATTN_PROBE_CYC_PAIR_FP8_FMA_AGPR, T{});
  pair(T{}, Fa{}, ATTN_PROBE_CYC_PAIR_FP8_FMA, Fa{});
  (void)hipFree(out);
  (void)hipFree(cyc);
  return err ? 1 : 0;
}

extern "C" int attn_probe_ceilings(double* r, int n) {
  using namespace probe;
  if (r == nullptr || n < ATTN_PROBE_NUM) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 1;
  const int grid = cus * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  float* out = nullptr;
  uint64_t* clk = nullptr;
  if (hipMalloc(&out, sizeof(float) * (size_t)grid * 512) != hipSuccess) return 1;
  if (hipMalloc(&clk, sizeof(uint64_t) * 2 * (size_t)grid) != hipSuccess) {
    (void)hipFree(out);
    return 1;
  }
  int err = 0;
  double ms = 0.0;
  // vector instructions: lane-ops per second
  const int vit = 4096;
  auto valu = [&](auto op, int slot) {
    constexpr int OP = decltype(op)::value;
    err |= timed([&] { hipLaunchKernelGGL((valu_kernel<OP>), dim3(grid), dim3(256), 0, 0, out, vit, 0.5f); }, &ms);
    r[slot] = (double)grid * 256 * vit * 8 / (ms * 1e-3);
  };
  valu(std::integral_constant<int, kExp>{}, ATTN_PROBE_EXP_LANE_OPS);
  valu(std::integral_constant<int, kFma>{}, ATTN_PROBE_FMA_LANE_OPS);
  valu(std::integral_constant<int, kAdd>{}, ATTN_PROBE_ADD_LANE_OPS);
  valu(std::integral_constant<int, kMax3>{}, ATTN_PROBE_MAX3_LANE_OPS);
  valu(std::integral_constant<int, kCvtFp8>{}, ATTN_PROBE_CVT_FP8_LANE_OPS);
  valu(std::integral_constant<int, kCvtBf16>{}, ATTN_PROBE_CVT_BF16_LANE_OPS);
  valu(std::integral_constant<int, kRcp>{}, ATTN_PROBE_RCP_LANE_OPS);
  // matrix products: flops (or int ops) per second, and the clock
  const int mit = 2048;
  auto mfma = [&](auto kind, int slot, double flops_per) {
    constexpr int K = decltype(kind)::value;
    err |= timed([&] { hipLaunchKernelGGL((mfma_kernel<K>), dim3(grid), dim3(256), 0, 0, out, clk, mit); }, &ms);
    r[slot] = (double)grid * 4 * mit * 4 * flops_per / (ms * 1e-3);
  };
  mfma(std::integral_constant<int, kFp8>{}, ATTN_PROBE_MFMA_FP8_FLOPS, 32.0 * 32 * 64 * 2);
  mfma(std::integral_constant<int, kI8>{}, ATTN_PROBE_MFMA_I8_OPS, 32.0 * 32 * 32 * 2);
  mfma(std::integral_constant<int, kBf16>{}, ATTN_PROBE_MFMA_BF16_FLOPS, 32.0 * 32 * 16 * 2);
  {
    // shader clock from the last run: counter cycles over 100 MHz real time
    uint64_t* h = new uint64_t[2 * (size_t)grid];
    err |= hipMemcpy(h, clk, sizeof(uint64_t) * 2 * grid, hipMemcpyDeviceToHost) != hipSuccess;
    double c = 0.0, t = 0.0;
    for (int i = 0; i < grid; ++i) {
      c += (double)h[2 * i];
      t += (double)h[2 * i + 1];
    }
    delete[] h;
    r[ATTN_PROBE_CLOCK_GHZ] = t > 0.0 ? c / t * 0.1 : 0.0;
  }
  // one wave per SIMD: products, exponentials, and both in one instruction stream
  const int xit = 4096;
  const size_t hold = 96 * 1024;  // LDS per workgroup: one workgroup per CU
  double t_mfma = 0, t_exp8 = 0, t_mix4 = 0, t_mix8 = 0;
  err |= timed([&] { hipLaunchKernelGGL((mix_one_wave_kernel<0, true>), dim3(cus), dim3(256), hold, 0, out, xit); }, &t_mfma);
  err |= timed([&] { hipLaunchKernelGGL((mix_one_wave_kernel<8, false>), dim3(cus), dim3(256), hold, 0, out, xit); }, &t_exp8);
  err |= timed([&] { hipLaunchKernelGGL((mix_one_wave_kernel<4, true>), dim3(cus), dim3(256), hold, 0, out, xit); }, &t_mix4);
  err |= timed([&] { hipLaunchKernelGGL((mix_one_wave_kernel<8, true>), dim3(cus), dim3(256), hold, 0, out, xit); }, &t_mix8);
  r[ATTN_PROBE_ONE_WAVE_MFMA_MS] = t_mfma;
  r[ATTN_PROBE_ONE_WAVE_EXP16_MS] = t_exp8;
  r[ATTN_PROBE_ONE_WAVE_MIX8_MS] = t_mix4;
  r[ATTN_PROBE_ONE_WAVE_MIX16_MS] = t_mix8;
  // two waves per SIMD, one of each kind
  double t2m = 0, t2e = 0, t2b = 0;
  err |= timed([&] { hipLaunchKernelGGL((mix_two_waves_kernel<1>), dim3(cus), dim3(512), hold, 0, out, xit); }, &t2m);
  err |= timed([&] { hipLaunchKernelGGL((mix_two_waves_kernel<2>), dim3(cus), dim3(512), hold, 0, out, xit); }, &t2e);
  err |= timed([&] { hipLaunchKernelGGL((mix_two_waves_kernel<3>), dim3(cus), dim3(512), hold, 0, out, xit); }, &t2b);
  r[ATTN_PROBE_TWO_WAVES_MFMA_MS] = t2m;
  r[ATTN_PROBE_TWO_WAVES_EXP_MS] = t2e;
  r[ATTN_PROBE_TWO_WAVES_BOTH_MS] = t2b;
  r[ATTN_PROBE_CUS] = cus;
  (void)hipFree(out);
  (void)hipFree(clk);
  return err ? 1 : 0;
}
