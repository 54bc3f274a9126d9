// The 8-bit prologue ("Fused attention kernel" page, section "8-bit forward
// pass"): optional incoherent processing — every row multiplied by
// diag(signs) H_D / sqrt(D) — then block quantisation to e4m3: one scale per
// (b, h, 128 rows) (or one per tensor for the baseline), scale = amax / 448,
// code = e4m3fn(x / scale) with round-to-nearest-even and saturation.
//
// The power-of-two form (kE4M3Pow2) multiplies every value by a factor
// `premul` first (float32; the softmax scale times log2(e) for Q, 1 for K and
// V) and takes as scale the smallest power of two at or above amax / 448 (at
// least 2^-126): the division is then exact, and the scale is what the matrix
// cores' block-scale operands take (an 8-bit exponent), so the matching
// forward applies the scales inside its MFMAs.
//
// The int8 form (the case study's int8 path) quantises symmetrically instead:
// scale = amax / 127, code = x / scale rounded to nearest-even and clamped to
// [-127, 127].
//
// This step streams every element once from HBM and writes a byte back; a
// workgroup owns one 128-row block of one head and holds it in registers,
// reduces the block amax through LDS and writes the codes.  What each element
// costs on the vector units decides whether the pass reaches the bandwidth
// bound, so:
//  * the rotation runs on the matrix cores: (x * signs) H_D is a product with
//    a +-1 matrix, exact in bf16 operands (the signs flip sign bits of the bf16
//    inputs; H_D's entries are generated in registers from the parity of the
//    row and column indices) with float32 accumulation;
//  * amax / 448 and int8: the quotient x / scale, which decides the code, is
//    correctly rounded float32 without a division per element: r = 1 / scale
//    once per block, q = x r, then two residual corrections
//    q += fma(-q, scale, x) r (with r
//    within half an ulp of 1 / scale each residual is exact and the corrected
//    quotient is the correctly rounded one).  Blocks whose scale is below
//    2^-60 are first multiplied by 2^64 (exact), so no residual falls in the
//    subnormal range where that fails; elsewhere a subnormal x gives a
//    quotient below 2^-66, which codes as a zero of x's sign either way.
#include "common.hpp"

namespace attn {

// float32 (already divided by the scale) -> int8 code: nearest-even, clamped
// to [-127, 127], returned as its byte
__device__ __forceinline__ uint32_t int8_encode(float y) {
  const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(y), -127.f, 127.f);
  return (uint32_t)(int32_t)r & 0xffu;
}

enum QuantMode { kQuantBlock = 0, kAmaxOnly = 1, kQuantGlobal = 2 };
enum QuantFormat { kE4M3 = 0, kInt8 = 1, kE4M3Pow2 = 2 };

template <int FMT>
constexpr float code_max() { return FMT == kInt8 ? 127.f : 448.f; }

// The correctly rounded float32 quotient x / s from r = RN(1 / s): one
// product and two fma residual corrections; the sign of a zero quotient is
// taken from x.
struct QuotientRN {
  float s, r, pre;  // scale (pre-multiplied), its reciprocal, the factor applied to x
  __device__ __forceinline__ explicit QuotientRN(float scale) {
    pre = scale < 0x1p-60f ? 0x1p64f : 1.f;
    s = scale * pre;
    r = __fdiv_rn(1.f, s);
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float q0 = x * r;
    const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
    return __builtin_copysignf(fmaf(fmaf(-q1, s, x), r, q1), x);
  }
};

// four quotients -> four code bytes (byte i = value i)
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float y0, float y1, float y2, float y3) {
  if constexpr (FMT == kInt8) {
    return int8_encode(y0) | int8_encode(y1) << 8 | int8_encode(y2) << 16 | int8_encode(y3) << 24;
  } else {
    // the hardware converter rounds to nearest-even into e4m3fn but does not
    // saturate: clamp to +-448 first (one v_med3 per value)
    y0 = __builtin_amdgcn_fmed3f(y0, -448.f, 448.f);
    y1 = __builtin_amdgcn_fmed3f(y1, -448.f, 448.f);
    y2 = __builtin_amdgcn_fmed3f(y2, -448.f, 448.f);
    y3 = __builtin_amdgcn_fmed3f(y3, -448.f, 448.f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
  }
}

// amax of the workgroup (4 waves) through LDS
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// scale of a block (or of the tensor) from its amax: amax / 448 or amax /
// 127 (correctly rounded); for kE4M3Pow2 the smallest power of two at or above
// amax / 448 (the quotient rounded to float32), and at least 2^-126, the
// smallest normal float; 1 for an all-zero block
template <int FMT>
__device__ __forceinline__ float scale_of(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const float t = __fdiv_rn(amax, code_max<FMT>());
  if constexpr (FMT != kE4M3Pow2) {
    return t;
  } else {
    uint32_t u = __float_as_uint(t);
    if (u < 0x00800000u) return 0x1p-126f;
    if (u & 0x007fffffu) u = (u & 0x7f800000u) + 0x00800000u;
    return __uint_as_float(u);
  }
}

// x / scale: correctly rounded (QuotientRN), or for the power-of-two scales
// exact, one multiply by the exact reciprocal
template <int FMT>
struct Divider : QuotientRN {
  __device__ __forceinline__ explicit Divider(float scale) : QuotientRN(scale) {}
};
template <>
struct Divider<kE4M3Pow2> {
  float r;
  static constexpr float pre = 1.f;
  __device__ __forceinline__ explicit Divider(float scale) : r(1.f / scale) {}
  __device__ __forceinline__ float operator()(float x) const { return x * r; }
};

// ---------------------------------------------------------------------------
// Without rotation: D/16 lanes per row, 16 consecutive values per lane.
// ---------------------------------------------------------------------------
template <int D, int MODE, int FMT>
__global__ void __launch_bounds__(256) quant_plain_kernel(QuantArgs a) {
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
      if constexpr (FMT == kE4M3Pow2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[p][e] *= a.premul;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[p][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[p][e]));
  }

  if constexpr (MODE == kAmaxOnly) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    // non-negative floats order like their bit patterns
    if ((tid & 63) == 0) atomicMax((unsigned int*)a.scales, __float_as_uint(amax));
    return;
  }
  float scale;
  if constexpr (MODE == kQuantGlobal) {
    scale = a.scales[0];
  } else {
    scale = scale_of<FMT>(block_max(amax, red));
    if (tid == 0) a.scales[(int64_t)bh * nblk + blk] = scale;
  }
  const Divider<FMT> div(scale);
  if (div.pre != 1.f) {  // uniform: a block of tiny values
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[p][e] *= div.pre;
  }

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = blk * 128 + p * RP + r_in;
    if (row < a.S) {
      u32x4 out;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
        out[wd] = encode4<FMT>(div(x[p][4 * wd]), div(x[p][4 * wd + 1]), div(x[p][4 * wd + 2]), div(x[p][4 * wd + 3]));
      *(u32x4*)(a.x8 + (((int64_t)b * a.S + row) * a.H + h) * D + 16 * seg) = out;
    }
  }
}

// ---------------------------------------------------------------------------
// With rotation: y = (x * signs) H_D on the matrix cores, then y / sqrt(D).
// Wave w owns rows 32w .. 32w+31 of the block.  Y^T = H_D^T (x * signs)^T is
// computed 32 output columns (tile jt) x 32 rows at a time with
// v_mfma_f32_32x32x16_bf16: the A operand is a 32 x 16 tile of H_D^T, whose
// row m stands for output column 32 jt + swz23(m), so that accumulator
// register r of lane-half hh holds output column 32 jt + 16 (r / 8) + 8 hh +
// r % 8 of data row (lane % 32): runs of 8 consecutive codes per lane.  The B
// operand is the lane's 8 inputs x[row][16 kk + 8 hh .. +7] (one 16-byte
// load each), their sign bits flipped where signs are negative.
// ---------------------------------------------------------------------------
template <int D, int MODE, int FMT>
__global__ void __launch_bounds__(256) quant_rot_kernel(QuantArgs a) {
  constexpr int NK = D / 16, NJ = D / 32;
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint32_t smask[D / 2];  // sign-bit masks of bf16 pairs (k, k + 1)

  const int tid = threadIdx.x;
  const int nblk = (a.S + 127) / 128;
  const int w = blockIdx.x;
  const int bh = w / nblk, blk = w - bh * nblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int row = blk * 128 + 32 * wave + l32;
  const bool valid = row < a.S;

  // inputs, as B operands
  u32x4 xb[NK];
  {
    const uint16_t* src = a.x + b * a.x_sb + (int64_t)(valid ? row : 0) * a.x_ss + h * a.x_sh + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) xb[kk] = valid ? *(const u32x4*)(src + 16 * kk) : u32x4{0, 0, 0, 0};
  }
  for (int p = tid; p < D / 2; p += 256)
    smask[p] = (a.signs[2 * p] < 0 ? 0x8000u : 0u) | (a.signs[2 * p + 1] < 0 ? 0x80000000u : 0u);
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) xb[kk] ^= *(const u32x4*)&smask[(16 * kk + 8 * hh) / 2];

  // A operands.  H_D[k][j] = (-1)^popcount(k & j); with k = 16 kk + 8 hh + e
  // and j = 32 jt + jl, jl = swz23(m):
  //   popcount(k & j) = popcount(e & jl & 7) + hh * jl[3] + kk[0] * jl[4]
  //                     + popcount((kk >> 1) & jt),
  // so every tile is one per-lane vector (the first two terms) with its sign
  // flipped by a per-lane bit (kk odd and jl[4]) and by a compile-time bit.
  const int jl = swz23(l32);
  u32x4 h00;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint32_t v = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int e = 2 * e2 + t;
      const int par = (__builtin_popcount(e & jl & 7) + (hh & (jl >> 3))) & 1;
      v |= (par ? 0xBF80u : 0x3F80u) << (16 * t);
    }
    h00[e2] = v;
  }
  const uint32_t lane_flip = ((jl >> 4) & 1) ? 0x80008000u : 0u;
  const u32x4 h01 = h00 ^ 0x80008000u, h10 = h00 ^ lane_flip, h11 = h10 ^ 0x80008000u;

  f32x16 acc[NJ];
  const f32x16 zero16 = {};
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bool odd = kk & 1, ct = __builtin_popcount((kk >> 1) & jt) & 1;
      const u32x4 hop = odd ? (ct ? h11 : h10) : (ct ? h01 : h00);
      acc[jt] = mfma32<kBF16>(hop, xb[kk], kk == 0 ? zero16 : acc[jt]);
    }

  const float norm = 1.0f / __builtin_sqrtf((float)D);
  float amax = 0.f;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[jt][r] *= norm;
      if constexpr (FMT == kE4M3Pow2) acc[jt][r] *= a.premul;
      amax = fmaxf(amax, fabsf(acc[jt][r]));
    }

  if constexpr (MODE == kAmaxOnly) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    if (lane == 0) atomicMax((unsigned int*)a.scales, __float_as_uint(amax));
    return;
  }
  float scale;
  if constexpr (MODE == kQuantGlobal) {
    scale = a.scales[0];
  } else {
    scale = scale_of<FMT>(block_max(amax, red));
    if (tid == 0) a.scales[(int64_t)bh * nblk + blk] = scale;
  }
  const Divider<FMT> div(scale);
  if (div.pre != 1.f) {
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[jt][r] *= div.pre;
  }
  if (valid) {
    uint8_t* dst = a.x8 + (((int64_t)b * a.S + row) * a.H + h) * D + 8 * hh;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const f32x16& y = acc[jt];
        const int r0 = 8 * run;
        *(u32x2*)(dst + 32 * jt + 16 * run) =
            u32x2{encode4<FMT>(div(y[r0]), div(y[r0 + 1]), div(y[r0 + 2]), div(y[r0 + 3])),
                  encode4<FMT>(div(y[r0 + 4]), div(y[r0 + 5]), div(y[r0 + 6]), div(y[r0 + 7]))};
      }
  }
}

// per-tensor mode helpers: clear the reduction cell, then turn amax into the scale
__global__ void fp8_fill_kernel(float* p, float v) { *p = v; }
template <int FMT>
__global__ void fp8_finalize_scale_kernel(float* p) { *p = scale_of<FMT>(*p); }

template <int D, int MODE, int FMT>
void launch_quant_pass(const QuantArgs& a, dim3 grid, hipStream_t s) {
  if (a.signs != nullptr)
    hipLaunchKernelGGL((quant_rot_kernel<D, MODE, FMT>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((quant_plain_kernel<D, MODE, FMT>), grid, dim3(256), 0, s, a);
}

template <int D, int FMT>
hipError_t launch_quant_d(const QuantArgs& a, hipStream_t s) {
  const int nblk = (a.S + 127) / 128;
  const dim3 grid(a.B * a.H * nblk);
  if (a.block_rows == 128) {
    launch_quant_pass<D, kQuantBlock, FMT>(a, grid, s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fp8_fill_kernel, dim3(1), dim3(1), 0, s, a.scales, 0.f);
  launch_quant_pass<D, kAmaxOnly, FMT>(a, grid, s);
  hipLaunchKernelGGL(fp8_finalize_scale_kernel<FMT>, dim3(1), dim3(1), 0, s, a.scales);
  launch_quant_pass<D, kQuantGlobal, FMT>(a, grid, s);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_quant(const QuantArgs& a, int D, hipStream_t s) {
  if (D == 64) return launch_quant_d<64, FMT>(a, s);
  if (D == 128) return launch_quant_d<128, FMT>(a, s);
  return launch_quant_d<256, FMT>(a, s);
}

hipError_t launch_fp8_quantize(const QuantArgs& a, int D, hipStream_t s) { return launch_quant<kE4M3>(a, D, s); }
hipError_t launch_fp8_quantize_pow2(const QuantArgs& a, int D, hipStream_t s) {
  return launch_quant<kE4M3Pow2>(a, D, s);
}
hipError_t launch_int8_quantize(const QuantArgs& a, int D, hipStream_t s) { return launch_quant<kInt8>(a, D, s); }

}  // namespace attn
