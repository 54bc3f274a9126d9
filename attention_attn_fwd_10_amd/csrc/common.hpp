// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, conversions, the work-item remap and launch-side argument structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.hpp"

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));



// ---------------------------------------------------------------------------
// MFMA: D(32x32, fp32) += A(32x16) * B(16x32); A/B hold 8 16-bit values/lane.
// Lane l supplies row (l % 32) of A / column (l % 32) of B and the k-slice
// selected by l / 32; the same (lane, element) -> k map applies to A and B.
// The accumulator: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4 and
// column l % 32.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// 8-bit: D(32x32) += A(32x64) * B(64x32), 32 e4m3 values per lane (both operands e4m3).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format selectors 0 = e4m3 for A and B; scale exponents 127 = x1.0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// two floats -> packed 16-bit pair (round to nearest even), low half = a;
// one v_cvt_pk_{bf16,f16}_f32 on gfx950
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// LDS transposing read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives, as its element t (t = 0..3), element i % 4 of the 8-byte
// chunk addressed by lane 4t + i/4 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// max of three (two) floats as one v_maximum3_f32 (v_maximum_f32): the IEEE
// maximum, which needs none of the quieting that fmaxf wraps around its
// operands (a v_max x, x each).  The result is exact, so any order of the
// operands gives the same bits.  Written with the compiler's builtin, not as
// inline assembly: the compiler's hazard checks do not look into inline
// assembly, and a read of a matrix-core result needs wait states after the
// MFMA that writes it (with inline assembly reading score registers right
// after the score MFMAs, stale registers were read).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float max2f(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max of the 32 scores of two 16-value score tiles (16 v_max3)
__device__ __forceinline__ float tile_max32(const f32x16& a, const f32x16& b) {
  float m = max3f(a[0], a[1], a[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = max3f(m, a[r], a[r + 1]);
  m = max3f(m, a[15], b[0]);
#pragma unroll
  for (int r = 1; r < 15; r += 2) m = max3f(m, b[r], b[r + 1]);
  return max2f(m, b[15]);
}

// max / sum of a value with the same lane of the other half-wave (l ^ 32)
__device__ __forceinline__ float halfwave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Asynchronous global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds_wave_base + 16*l; lds_wave_base must be the same
// for every lane of the wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// Buffer resource (V#) for raw byte-addressed buffer loads: base address and
// size in bytes; loads at or past `nbytes` return zeros.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)nbytes, 0x00020000};
}
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// buffer_load_dwordx4 into registers (zeros past the resource's range)
__device__ i32x4 raw_buffer_load_v4(i32x4 rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
// Asynchronous buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l reads rsrc.base + voffset (zeros when out of range) and writes
// lds_wave_base + 16*l; lds_wave_base must be the same for every lane.
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t voffset, void* lds_wave_base) {
  raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, (int)voffset, 0, 0, 0);
}

// 8-bit integer: D(32x32, int32) += A(32x32) * B(32x32), 16 int8 values per
// lane; lane l supplies row (l % 32) of A / column (l % 32) of B and the
// k-slice selected by l / 32 (the same (lane, byte) -> k map for A and B).
// The int32 sums are exact; the accumulator layout is that of the fp32 forms.
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ i32x16 mfma32_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// wait until every global load (including LDS DMA) issued by this wave is done
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Swap bits 2 and 3 of a row index inside a 32-row MFMA tile.  Storing key k
// (or head-dim row d) at LDS row swz(k) and reading row m = lane % 32 makes
// accumulator register r of lane half hh correspond to index
// 16*(r/8) + 8*hh + r%8, i.e. runs of 8 consecutive keys (or d) per lane.
__host__ __device__ constexpr int swz23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Map the hardware
// block id to a logical tile id so that consecutive logical tiles (the q-blocks
// of one head) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int p, int n) {
  constexpr int kXcd = 8;
  const int per = n / kXcd, rem = n % kXcd;
  const int xcd = p % kXcd, slot = p / kXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace attn
