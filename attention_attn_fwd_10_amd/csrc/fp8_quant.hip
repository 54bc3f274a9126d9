// The 8-bit prologue ("Fused attention kernel" page, section "8-bit forward
// pass"): optional incoherent processing — every row multiplied by
// diag(signs) H_D / sqrt(D), evaluated as a fast Walsh-Hadamard transform in
// float32 — then block quantisation to e4m3: one scale per (b, h, 128 rows)
// (or one per tensor for the baseline), scale = amax / 448, code =
// e4m3fn(x / scale) with round-to-nearest-even and saturation.
//
// The int8 form (the case study's int8 path) quantises symmetrically instead:
// scale = amax / 127, code = x / scale rounded to nearest-even and clamped to
// [-127, 127].
//
// This step streams every element once from HBM and writes a byte back, so it
// is bandwidth bound; a workgroup owns one 128-row block of one head, holds
// the whole block in registers (16 values per lane), reduces the block amax
// through LDS and writes 16 codes per lane with one 16-byte store.
#include "common.hpp"

namespace attn {

// float32 (already divided by the scale) -> int8 code: nearest-even, clamped
// to [-127, 127], returned as its byte
__device__ __forceinline__ uint32_t int8_encode(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.f), 127.f);
  return (uint32_t)(int32_t)r & 0xffu;
}

enum QuantMode { kQuantBlock = 0, kAmaxOnly = 1, kQuantGlobal = 2 };
enum QuantFormat { kE4M3 = 0, kInt8 = 1 };

template <int FMT>
constexpr float code_max() { return FMT == kInt8 ? 127.f : 448.f; }

template <int D, int MODE, int FMT>
__global__ void __launch_bounds__(256) fp8_quant_kernel(QuantArgs a) {
  constexpr int LPR = D / 16;          // lanes per row (16 values per lane)
  constexpr int RP = 256 / LPR;        // rows per pass
  constexpr int NP = 128 / RP;         // passes over a 128-row block
  __shared__ float red[4];

  const int tid = threadIdx.x;
  const int nblk = (a.S + 127) / 128;
  const int w = blockIdx.x;
  const int bh = w / nblk, blk = w - bh * nblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int seg = tid % LPR;
  const int r_in = tid / LPR;

  float x[NP][16];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = blk * 128 + p * RP + r_in;
    if (row < a.S) {
      const uint16_t* src = a.x + b * a.x_sb + (int64_t)row * a.x_ss + h * a.x_sh + 16 * seg;
      const u32x4 lo = *(const u32x4*)src;
      const u32x4 hi = *(const u32x4*)(src + 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[p][2 * e] = __uint_as_float(lo[e] << 16);
        x[p][2 * e + 1] = __uint_as_float(lo[e] & 0xffff0000u);
        x[p][8 + 2 * e] = __uint_as_float(hi[e] << 16);
        x[p][8 + 2 * e + 1] = __uint_as_float(hi[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[p][e] = 0.f;
    }
    if (a.signs != nullptr) {
      // x <- (x * signs) H_D: butterflies of span 1..8 inside the lane, then
      // span 16..D/2 across the LPR lanes of the row (lane xor span/16)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[p][e] *= (float)a.signs[16 * seg + e];
#pragma unroll
      for (int span = 1; span < 16; span <<= 1)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e & span) == 0) {
            const float u = x[p][e], v = x[p][e + span];
            x[p][e] = u + v;
            x[p][e + span] = u - v;
          }
#pragma unroll
      for (int s = 1; s < LPR; s <<= 1) {
        const bool upper = (seg & s) != 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float other = __shfl_xor(x[p][e], s);
          x[p][e] = upper ? other - x[p][e] : x[p][e] + other;
        }
      }
      const float norm = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[p][e] *= norm;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[p][e]));
  }

  if constexpr (MODE != kQuantGlobal) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  if constexpr (MODE == kAmaxOnly) {
    // non-negative floats order like their bit patterns
    if (tid == 0) atomicMax((unsigned int*)a.scales, __float_as_uint(amax));
    return;
  }
  if constexpr (MODE == kQuantGlobal) amax = a.scales[0];
  const float scale = amax > 0.f ? __fdiv_rn(amax, code_max<FMT>()) : 1.f;
  if constexpr (MODE == kQuantBlock)
    if (tid == 0) a.scales[(int64_t)bh * nblk + blk] = scale;

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = blk * 128 + p * RP + r_in;
    if (row < a.S) {
      u32x4 out;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float y[4];
#pragma unroll
        for (int by = 0; by < 4; ++by) y[by] = __fdiv_rn(x[p][4 * wd + by], scale);
        if constexpr (FMT == kInt8) {
          uint32_t v = 0;
#pragma unroll
          for (int by = 0; by < 4; ++by) v |= int8_encode(y[by]) << (8 * by);
          out[wd] = v;
        } else {
          // the hardware converter rounds to nearest-even into e4m3fn but does
          // not saturate: clamp to +-448 first (one v_med3 per value)
#pragma unroll
          for (int by = 0; by < 4; ++by) y[by] = __builtin_amdgcn_fmed3f(y[by], -448.f, 448.f);
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          out[wd] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        }
      }
      *(u32x4*)(a.x8 + (((int64_t)b * a.S + row) * a.H + h) * D + 16 * seg) = out;
    }
  }
}

// per-tensor mode helpers: clear the reduction cell, then turn amax into the scale
__global__ void fp8_fill_kernel(float* p, float v) { *p = v; }
__global__ void fp8_finalize_scale_kernel(float* p, float code_max) {
  const float amax = *p;
  *p = amax > 0.f ? __fdiv_rn(amax, code_max) : 1.f;
}

template <int D, int FMT>
hipError_t launch_quant_d(const QuantArgs& a, hipStream_t s) {
  const int nblk = (a.S + 127) / 128;
  const dim3 grid(a.B * a.H * nblk), block(256);
  if (a.block_rows == 128) {
    hipLaunchKernelGGL((fp8_quant_kernel<D, kQuantBlock, FMT>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fp8_fill_kernel, dim3(1), dim3(1), 0, s, a.scales, 0.f);
  hipLaunchKernelGGL((fp8_quant_kernel<D, kAmaxOnly, FMT>), grid, block, 0, s, a);
  hipLaunchKernelGGL((fp8_quant_kernel<D, kQuantGlobal, FMT>), grid, block, 0, s, a);
  hipLaunchKernelGGL(fp8_finalize_scale_kernel, dim3(1), dim3(1), 0, s, a.scales, code_max<FMT>());
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_quant(const QuantArgs& a, int D, hipStream_t s) {
  if (D == 64) return launch_quant_d<64, FMT>(a, s);
  if (D == 128) return launch_quant_d<128, FMT>(a, s);
  return launch_quant_d<256, FMT>(a, s);
}

hipError_t launch_fp8_quantize(const QuantArgs& a, int D, hipStream_t s) { return launch_quant<kE4M3>(a, D, s); }
hipError_t launch_int8_quantize(const QuantArgs& a, int D, hipStream_t s) { return launch_quant<kInt8>(a, D, s); }

}  // namespace attn
