// 8-bit fused attention forward for gfx950 ("Fused attention kernel" page,
// section "8-bit forward pass"): both GEMMs run on e4m3 inputs, V tiles are
// transposed on chip, and every block of Q, K and V carries its own scale.
//
// Layout and schedule follow the 16-bit kernel: 4 waves x 32 query rows per
// workgroup, 64-key K/V tiles copied asynchronously into a two-stage LDS ring,
// scores computed transposed (S^T = K Q^T) with v_mfma_f32_32x32x64_f8f6f4 so a
// lane owns one query row, online softmax in exp2 form, then
// O^T += V^T P^T with the probabilities quantised to e4m3 in registers.
//
// The 8-bit specifics:
//  * V^T comes from the row-major V tile through ds_read_b64_tr_b8 (the pages'
//    in-shared-memory transpose; no global pre-transpose);
//  * scales: a tile's score scale sq * sk * softmax_scale * log2(e) is one
//    scalar folded into the exp2 FMA.  The output accumulator is kept in units
//    of a reference V scale (the largest block scale seen so far); a tile whose
//    V block scale is smaller gets the ratio folded into the exp2 bias of its
//    probabilities, so block scales cost no per-element work, and the
//    accumulator is rescaled only when a larger block scale appears;
//  * power-of-two scales (POW2, inputs of the quantiser's power-of-two form):
//    the Q codes carry the softmax scale times log2(e), so a tile's score
//    scale sq * sk is a power of two that the MFMAs apply themselves through
//    their block-scale exponent operands, and the score MFMAs start from
//    kMu - m (every register of a lane holds its row's value): they return the
//    exp2 argument itself, and the softmax needs no multiply-add per score.
//    The P V MFMAs take each tile's V block scale the same way, so the
//    accumulator holds O times the row sum in absolute units;
//  * probabilities are quantised as p * 2^6 with the running max allowed to
//    lag the true max by at most 2^2, so quantised values stay in (0, 256] —
//    inside the e4m3 range (the converter does not saturate) and mostly in its
//    normal range;
//  * the row sum is accumulated from the e4m3-rounded probabilities, the same
//    values the second GEMM multiplies, so a row dominated by a few keys keeps
//    its weights consistent.
//
// The int8 variant (QK_I8) takes int8 Q and K codes (the case study's int8
// path; block scales and rotation as above) and computes the scores on
// v_mfma_i32_32x32x32_i8, whose int32 sums are exact; V and the probabilities
// stay e4m3.  Its accumulator starts at the bit pattern of 1.5 * 2^23 instead
// of zero: a score s (|s| <= 128 * 127^2 < 2^22) then lands in the mantissa,
// and the accumulator read as a float is exactly 1.5 * 2^23 + s, so the
// conversion costs no instruction — the offset is folded into the exp2 bias.
#include <type_traits>

#include "common.hpp"

namespace attn {

namespace fp8cfg {
constexpr int D = 128;
constexpr int BR = 128;            // query rows per workgroup
constexpr int BC = 64;             // keys per tile
// LDS layout of a 64-row tile (rows of D bytes, CPR 16-byte chunks).  The
// tile is copied by CPR wave instructions of 64 lanes x 16 bytes; instruction
// m writes 1 KB holding the rows R with R % CPR == m (lane l: row m + CPR *
// (l / CPR), chunk l % CPR).  Instructions sit 1 KB plus a gap apart; the gap
// spreads what one read instruction touches over the banks: 16 bytes for K
// (16 rows read by 16 lanes with ds_read_b128 start in 16 distinct 16-byte
// bank groups), 32 bytes for V (the 8 rows x 32 bytes of a 32-lane
// transposing read fall in 8 distinct 32-byte groups).  Row R starts at byte
// row(R) = (R % CPR) * GRP + (R / CPR) * D, additive over index bits.
constexpr int CPR = D / 16;
constexpr int KGRP = 1024 + 16;  // bytes
constexpr int VGRP = 1024 + 32;
constexpr int K_BYTES = CPR * KGRP;
constexpr int V_BYTES = CPR * VGRP;
constexpr int CI_W = CPR / 4;      // copy instructions per wave per tile and operand
constexpr int krow(int r) { return (r % CPR) * KGRP + (r / CPR) * D; }
constexpr int vrow(int r) { return (r % CPR) * VGRP + (r / CPR) * D; }
// LDS row R of a K tile holds key 32((m>>2)&1) + 16(R/32) + 4(m>>3) + (m&3),
// m = R % 32: then score register r of tile tt in lane half hh belongs to key
// 32hh + 16tt + r, so each lane's 32 probabilities are 32 consecutive keys.
// V row R holds key R.
constexpr int k_row_key(int R) {
  return 32 * (((R & 31) >> 2) & 1) + 16 * (R >> 5) + 4 * ((R & 31) >> 3) + (R & 3);
}
// copy round ii of wave w is tile instruction w + 4 ii; lane l copies chunk
// copy_chunk(l) of LDS row copy_row(w, ii, l) to byte (w + 4 ii) * GRP + 16 l
constexpr int copy_row(int w, int ii, int l) { return w + 4 * ii + CPR * (l / CPR); }
constexpr int copy_chunk(int l) { return l % CPR; }
constexpr float kMu = 6.0f;        // probabilities are quantised as p * 2^kMu
constexpr float kTau = 2.0f;       // the running max may lag by 2^kTau

// Compile-time check of the tile layout against the kernel's addressing: the
// copies fill each byte of the 64 rows once, at row(R) + column; a round's
// key is the round-0 key plus the shift the copies add; the K reads (both
// operand layouts) find their keys and start 16 rows of 16 lanes in 16
// distinct 16-byte bank groups; the transposing V reads of 32 lanes touch 32
// distinct 8-byte pieces of the 256 bytes of banks.
constexpr bool layout_ok() {
  bool kseen[K_BYTES / 16] = {}, vseen[V_BYTES / 16] = {};
  int kkey[K_BYTES / 16] = {}, vkey[V_BYTES / 16] = {};
  for (int w = 0; w < 4; ++w)
    for (int ii = 0; ii < CI_W; ++ii)
      for (int l = 0; l < 64; ++l) {
        const int r = copy_row(w, ii, l), ch = copy_chunk(l);
        const int kd = (w + 4 * ii) * KGRP + 16 * l, vd = (w + 4 * ii) * VGRP + 16 * l;
        if (r >= 64 || kd + 16 > K_BYTES || vd + 16 > V_BYTES) return false;
        if (kd != krow(r) + 16 * ch || vd != vrow(r) + 16 * ch || kseen[kd / 16] || vseen[vd / 16]) return false;
        kseen[kd / 16] = vseen[vd / 16] = true;
        kkey[kd / 16] = k_row_key(r) * 8 + ch;
        vkey[vd / 16] = r * 8 + ch;
        if (k_row_key(r) != k_row_key(copy_row(w, 0, l)) + k_row_key(4 * ii)) return false;
      }
  for (int i8 = 0; i8 < 2; ++i8) {
    const int hs = i8 ? 16 : 32, sec = i8 ? 32 : 16;
    for (int l = 0; l < 64; ++l)
      for (int tt = 0; tt < 2; ++tt)
        for (int kk = 0; kk < 2; ++kk)
          for (int x = 0; x <= sec; x += sec) {
            const int b = krow(l % 32) + hs * (l / 32) + krow(32 * tt) + 64 * kk + x;
            const int colb = 64 * kk + hs * (l / 32) + x;
            if (b % 16 || kkey[b / 16] != k_row_key(32 * tt + l % 32) * 8 + colb / 16) return false;
          }
    for (int tt = 0; tt < 2; ++tt)
      for (int hh = 0; hh < 2; ++hh)
        for (int kk = 0; kk < 2; ++kk) {
          unsigned seen = 0;
          for (int l = 0; l < 16; ++l) seen |= 1u << (((krow(32 * tt + l) + hs * hh + 64 * kk) / 16) % 16);
          if (seen != 0xffffu) return false;
        }
  }
  for (int half = 0; half < 2; ++half)
    for (int u = 0; u < 4; ++u)
      for (int dt = 0; dt < D / 32; ++dt) {
        unsigned seen = 0;
        for (int l = 32 * half; l < 32 * half + 32; ++l) {
          const int g = l >> 4, j = l & 15;
          const int row = 32 * (g >> 1) + (j >> 1) + 8 * u, col = 32 * dt + 16 * (g & 1) + 8 * (j & 1);
          const int b = vrow(32 * (g >> 1) + (j >> 1)) + 16 * (g & 1) + 8 * (j & 1) + vrow(8 * u) + 32 * dt;
          if (vkey[b / 16] != row * 8 + col / 16 || b % 16 != col % 16) return false;
          seen |= 1u << ((b / 8) % 32);
        }
        if (seen != 0xffffffffu) return false;
      }
  return true;
}
static_assert(layout_ok(), "8-bit forward tile layout");
}  // namespace fp8cfg

// two floats -> two e4m3 bytes (nearest-even; values above 464 would become NaN)
// written into the low (HI = false) or high 16 bits of `old`
template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_fp8(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// LDS transposing byte read (ds_read_b64_tr_b8).  Within each group of 16
// lanes, lane i receives, as its byte t (t = 0..7), byte i % 8 of the 8-byte
// chunk addressed by lane 2t + i/8 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int v2i __attribute__((vector_size(8)));
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// mfma32_fp8 with block scales: D += 2^(ea - 127) 2^(eb - 127) A B, ea and eb
// biased 8-bit exponents (byte 0 of the operand), here one per operand for
// all lanes.  A power-of-two float32's exponent field is that byte.
__device__ __forceinline__ f32x16 mfma32_fp8s(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// max of three floats: max3f (v_maximum3_f32, written so that the compiler
// sees the reads of the score MFMAs' results and waits for them)
__device__ __forceinline__ float max3(float a, float b, float c) { return max3f(a, b, c); }

template <int N>
using C = std::integral_constant<int, N>;

template <bool CAUSAL, bool QK_I8, bool POW2>
__global__ void __launch_bounds__(256, 3) fwd_fp8_kernel(Fp8Args a) {
  using namespace fp8cfg;
  static_assert(!(QK_I8 && POW2), "the power-of-two scale form is an e4m3 one");
  // score offset of the int8 form (see the file comment); 0 for e4m3
  constexpr float kSOff = QK_I8 ? 12582912.0f : 0.0f;
  // two-slot rings (tile j in slot j % 2) as four separate arrays, addressed
  // with compile-time slot numbers: the compiler then sees that a tile's LDS
  // reads never touch the slot the next tile is being copied into, and does
  // not make them wait for that copy
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[V_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[V_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / a.n_qblk;
  int qblk = t - bh * a.n_qblk;
  if (CAUSAL) qblk = a.n_qblk - 1 - qblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Lq = a.Sq, Lk = a.Sk;
  const int qs = qblk * BR;

  const int64_t row_q = (int64_t)a.H * D;  // bytes between consecutive rows (contiguous [B,S,H,D])
  const int64_t qoff = ((int64_t)b * Lq) * row_q + (int64_t)h * D;
  const int64_t koff = ((int64_t)b * Lk) * row_q + (int64_t)h * D;

  int n_kv = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last = min(qs + BR, Lq) - 1 + (Lk - Lq);
    n_kv = last < 0 ? 0 : min(n_kv, last / BC + 1);
  }
  const int qw = qs + 32 * wave;
  const int qi = qw + l32;
  const bool wave_active = qw < Lq;
  const int diag = Lk - Lq;
  const int wave_last_key = CAUSAL ? min(qw + 31, Lq - 1) + diag : Lk - 1;

  // scales: per (b, h, 128-row block), or one per tensor
  const bool blocked = a.block_rows != 0;
  const int nbq = (Lq + 127) / 128, nbk = (Lk + 127) / 128;
  const float sq = blocked ? a.qs[(int64_t)bh * nbq + qblk] : a.qs[0];
  // (read through the constant address space: the kernel never writes them,
  // so the uniform per-tile reads become scalar loads)
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* const ks_scale = (cfloat*)(blocked ? a.ks + (int64_t)bh * nbk : a.ks);
  cfloat* const vs_scale = (cfloat*)(blocked ? a.vs + (int64_t)bh * nbk : a.vs);
  const float qk_scale = sq * a.scale_log2;

  // Q fragments: lane (query l32, half hh) holds q[64kk + 32hh .. +31] (e4m3,
  // one 64-wide k step per qf[kk]) or q[64kk + 16hh .. +15] and
  // q[64kk + 32 + 16hh .. +15] (int8, two 32-wide k steps per qf[kk])
  constexpr int kHalfStride = QK_I8 ? 16 : 32;  // bytes between the two lane halves
  constexpr int kSecond = QK_I8 ? 32 : 16;      // bytes between a lane's two 16-byte runs
  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    if (qi < Lq) {
      const uint8_t* qp = a.q + qoff + (int64_t)qi * row_q + 64 * kk + kHalfStride * hh;
      const u32x4 x0 = *(const u32x4*)qp, x1 = *(const u32x4*)(qp + kSecond);
      qf[kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    } else {
      qf[kk] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // ---- asynchronous tile copies ----------------------------------------------
  const uint8_t* const kg = a.k + koff;
  const uint8_t* const vg = a.v + koff;
  // Byte offsets of this lane's copy in round 0 (wave instruction `wave`).
  // Round ii copies instruction wave + 4 * ii: only row bit 2 moves, which
  // k_row_key maps to key bit 5 (32 keys) and V's identity map to 4 keys, so
  // each round's offset is the round-0 offset plus a scalar.
  uint32_t k_boff, v_boff;
  {
    const int R = copy_row(wave, 0, lane), c = copy_chunk(lane);
    k_boff = (uint32_t)(k_row_key(R) * (int)row_q + 16 * c);
    v_boff = (uint32_t)(R * (int)row_q + 16 * c);
  }
  static_assert(CI_W == 2, "two copy rounds per wave: the round shift is one row bit");
  // one buffer resource per tile covers rows key0 .. Lk-1: rows past the
  // sequence end read as zeros
  auto dma_tile = [&](int key0, auto buf) {
    uint8_t* kb = (decltype(buf)::value ? lds_k1 : lds_k0) + wave * KGRP;
    uint8_t* vb = (decltype(buf)::value ? lds_v1 : lds_v0) + wave * VGRP;
    const uint64_t n = (uint64_t)(Lk - key0) * (uint64_t)row_q;
    const uint32_t nb = (uint32_t)min(n, (uint64_t)0x7fff0000u);
    const i32x4 kr = make_rsrc(kg + (int64_t)key0 * row_q, nb);
    const i32x4 vr = make_rsrc(vg + (int64_t)key0 * row_q, nb);
#pragma unroll
    for (int ii = 0; ii < CI_W; ++ii) {
      dma16_buf(kr, k_boff + (uint32_t)(k_row_key(4 * ii) * (int)row_q), kb + 4 * ii * KGRP);
      dma16_buf(vr, v_boff + (uint32_t)(4 * ii * (int)row_q), vb + 4 * ii * VGRP);
    }
  };

  // V^T operand: lane (group g, index j) addresses row 32(g/2) + 8u + j/2 and
  // columns 32dt + 16(g%2) + 8(j%2); after the byte transpose lane l holds
  // V[32(l/32) + 8u + t][32dt + l%32] as its elements 8u + t.
  const int vgrp = lane >> 4, vj = lane & 15;
  const int vtr_off = vrow(32 * (vgrp >> 1) + (vj >> 1)) + 16 * (vgrp & 1) + 8 * (vj & 1);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max of the log2-domain scores (lazy)
  float l_run = 0.f;        // this half-wave's share of sum p * 2^kMu (float32 terms)
  float lq_run = 0.f;       // sum over all 64 keys of the e4m3-rounded terms (full row, both halves)
  float sv_ref = 0.f;       // V scale the accumulator is expressed in
  // sv_ref / sv and log2(sv / sv_ref) of the current 128-key V scale block
  // (both tiles of a block share them; sv_ref only moves on a block's first)
  float inv_vratio = 1.f, lv = 0.f;
  const f32x16 zero16 = {};
  // e4m3 1.0 in every byte; kept in registers across the key loop
  i32x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;
  asm volatile("" : "+v"(ones));

  // ---- tiles with any positive scales -----------------------------------------
  auto compute = [&](int j, auto buf) {
    const int key0 = j * BC;
    if (!wave_active) return;
    if (CAUSAL && key0 > wave_last_key) return;
    const float c2 = qk_scale * ks_scale[blocked ? key0 >> 7 : 0];
    const float sv = vs_scale[blocked ? key0 >> 7 : 0];
    // S^T = K Q^T: two 32-key tiles, two 64-wide k steps each (K operands laid
    // out like the Q fragments)
    const uint8_t* ks = (decltype(buf)::value ? lds_k1 : lds_k0) + krow(l32) + kHalfStride * hh;
    i32x8 kop[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 x0 = *(const u32x4*)(ks + krow(32 * tt) + 64 * kk);
        const u32x4 x1 = *(const u32x4*)(ks + krow(32 * tt) + 64 * kk + kSecond);
        kop[tt][kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    f32x16 s[2];
    if constexpr (QK_I8) {
      i32x16 acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tt][r] = 0x4B400000;  // the bits of 1.5 * 2^23
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const i32x8& kv = kop[tt][kk];
            const i32x8& qv = qf[kk];
            acc[tt] = mfma32_i8(i32x4{kv[4 * half], kv[4 * half + 1], kv[4 * half + 2], kv[4 * half + 3]},
                                i32x4{qv[4 * half], qv[4 * half + 1], qv[4 * half + 2], qv[4 * half + 3]}, acc[tt]);
          }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) s[tt] = __builtin_bit_cast(f32x16, acc[tt]);
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) s[tt] = mfma32_fp8(kop[tt][0], qf[0], zero16);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) s[tt] = mfma32_fp8(kop[tt][1], qf[1], s[tt]);
    }
    // register r of tile tt holds key key0 + 32hh + 16tt + r
    const bool need_mask = (key0 + BC > Lk) || (CAUSAL && key0 + BC - 1 > qw + diag);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * hh + 16 * tt + r;
          if (key >= Lk || (CAUSAL && key > qi + diag)) s[tt][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 31; i += 2) mx = max3(mx, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
    mx = max3(mx, s[1][15], s[1][15]);
    const auto mxw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    const float mxs = (max3(mx, __uint_as_float(mxw[0]), __uint_as_float(mxw[1])) - kSOff) * c2;
    // a larger V block scale becomes the accumulator's reference (uniform branch)
    if (sv > sv_ref) {
      const float ratio = sv_ref * __builtin_amdgcn_rcpf(sv);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= ratio;
      sv_ref = sv;
    }
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kTau) != 0) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
      lq_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = m_new;
    }
    // p'' = 2^(c2 s - m + kMu) * sv / sv_ref is what enters the MFMA; the sum
    // keeps p' = p'' * sv_ref / sv (approximate reciprocals: both factors only
    // need to be consistent to float precision)
    if (blocked ? (key0 & 127) == 0 : j == 0) {
      const float vratio = sv * __builtin_amdgcn_rcpf(sv_ref);
      inv_vratio = sv_ref * __builtin_amdgcn_rcpf(sv);
      lv = __log2f(vratio);
    }
    float bias = m_run == -INFINITY ? 0.f : kMu + lv - m_run;
    // the int8 score offset enters once per tile: kSOff * c2 is rounded once,
    // a shift shared by the whole tile of at most one score unit
    if constexpr (QK_I8) bias -= kSOff * c2;
    // the row sum adds the e4m3-rounded probabilities, exactly the values the
    // MFMA multiplies, so numerator and denominator share the rounding
    // (the logsumexp keeps the float32 sum)
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int tt = w >> 2, r0 = 4 * (w & 3);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(fmaf(s[tt][r0 + e], c2, bias));
        psum += p[e];
      }
      // (the untouched half of the first conversion's destination is
      // overwritten by the second, so any register serves as its old value)
      pw[w] = cvt_pk_fp8<true>(p[2], p[3], cvt_pk_fp8<false>(p[0], p[1], __float_as_uint(p[0])));
    }
    l_run += psum * inv_vratio;
    const i32x8 pk = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    // O^T += V^T P^T (64 keys per MFMA)
    const uint8_t* vs = (decltype(buf)::value ? lds_v1 : lds_v0) + vtr_off;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      u32x2 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = lds_read_tr8(vs + vrow(8 * u) + 32 * dt);
      const i32x8 vop = {(int)r[0][0], (int)r[0][1], (int)r[1][0], (int)r[1][1],
                         (int)r[2][0], (int)r[2][1], (int)r[3][0], (int)r[3][1]};
      oacc[dt] = mfma32_fp8(vop, pk, oacc[dt]);
    }
    // the sum of the e4m3-rounded probabilities of all 64 keys, on the matrix
    // core: an all-ones (e4m3 1.0) A operand turns every output row into the
    // column sums of P^T, exact in float32
    const f32x16 qs = mfma32_fp8(ones, pk, zero16);
    lq_run += qs[0] * inv_vratio;
  };

  // ---- tiles with power-of-two scales -------------------------------------------
  // m_e: the running (lazy) max of the row's exp2 arguments c s; minit holds
  // kMu - m_e in all 16 registers, the score MFMAs' starting value.  Until a
  // row's first tile m_e is 0 (l, lq and O are still zero, so the first tile's
  // move rescales nothing that matters).
  const int esq = (int)(__float_as_uint(sq) >> 23);  // Q block scale exponent
  f32x16 minit;
#pragma unroll
  for (int r = 0; r < 16; ++r) minit[r] = kMu;
  float m_e = 0.f;
  auto compute_pow2 = [&](int j, auto buf) {
    const int key0 = j * BC;
    if (!wave_active) return;
    if (CAUSAL && key0 > wave_last_key) return;
    const int blk = blocked ? key0 >> 7 : 0;
    const int esk = (int)(__float_as_uint(ks_scale[blk]) >> 23);
    const int esv = (int)(__float_as_uint(vs_scale[blk]) >> 23);
    const uint8_t* ks = (decltype(buf)::value ? lds_k1 : lds_k0) + krow(l32) + kHalfStride * hh;
    i32x8 kop[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 x0 = *(const u32x4*)(ks + krow(32 * tt) + 64 * kk);
        const u32x4 x1 = *(const u32x4*)(ks + krow(32 * tt) + 64 * kk + kSecond);
        kop[tt][kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    // x = sq sk (Q' K^T) + kMu - m_e: the exp2 argument (Q' = Q times the
    // softmax scale times log2(e))
    f32x16 x[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) x[tt] = mfma32_fp8s(kop[tt][0], qf[0], minit, esk, esq);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) x[tt] = mfma32_fp8s(kop[tt][1], qf[1], x[tt], esk, esq);
    const bool need_mask = (key0 + BC > Lk) || (CAUSAL && key0 + BC - 1 > qw + diag);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * hh + 16 * tt + r;
          if (key >= Lk || (CAUSAL && key > qi + diag)) x[tt][r] = -INFINITY;
        }
    }
    float mx = x[0][0];
#pragma unroll
    for (int i = 1; i < 31; i += 2) mx = max3(mx, x[i >> 4][i & 15], x[(i + 1) >> 4][(i + 1) & 15]);
    mx = max3(mx, x[1][15], x[1][15]);
    const auto mxw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = max3(mx, __uint_as_float(mxw[0]), __uint_as_float(mxw[1]));
    // the row's max moved by more than kTau (or this is its first tile): m_e
    // becomes the tile's max, the accumulators are rescaled, and this tile's
    // arguments and minit move with it (uniform branch, rare after the first
    // tile).  A row with no valid key in its first tile has none at all (keys
    // are masked from the sequence end or past the diagonal) and keeps m_e.
    if (j == 0 || __builtin_amdgcn_ballot_w64(mx > kMu + kTau) != 0) {
      const float m_tile = mx - kMu + m_e;
      const float m_new = j == 0 ? (m_tile == -INFINITY ? m_e : m_tile) : max2f(m_e, m_tile);
      const float delta = m_e - m_new;
      const float alpha = fast_exp2(delta);
      l_run *= alpha;
      lq_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[tt][r] += delta;
      const float mi = kMu - m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) minit[r] = mi;
      m_e = m_new;
    }
    // p = 2^x: float32 terms for the logsumexp, e4m3 codes for the MFMAs
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int tt = w >> 2, r0 = 4 * (w & 3);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(x[tt][r0 + e]);
        psum += p[e];
      }
      pw[w] = cvt_pk_fp8<true>(p[2], p[3], cvt_pk_fp8<false>(p[0], p[1], __float_as_uint(p[0])));
    }
    l_run += psum;
    const i32x8 pk = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    // O^T += sv V^T P^T (the V block scale as the A operand's exponent)
    const uint8_t* vs = (decltype(buf)::value ? lds_v1 : lds_v0) + vtr_off;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      u32x2 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = lds_read_tr8(vs + vrow(8 * u) + 32 * dt);
      const i32x8 vop = {(int)r[0][0], (int)r[0][1], (int)r[1][0], (int)r[1][1],
                         (int)r[2][0], (int)r[2][1], (int)r[3][0], (int)r[3][1]};
      oacc[dt] = mfma32_fp8s(vop, pk, oacc[dt], esv, 127);
    }
    // the sum of the e4m3-rounded probabilities of all 64 keys, as below
    const f32x16 qsum = mfma32_fp8(ones, pk, zero16);
    lq_run += qsum[0];
  };
  auto tile = [&](int j, auto buf) {
    if constexpr (POW2) compute_pow2(j, buf);
    else compute(j, buf);
  };

  if (n_kv > 0) {
    dma_tile(0, C<0>{});
    wait_vmem();
    __syncthreads();
    // two tiles per iteration, so that every slot number is a constant
    for (int j = 0; j < n_kv; j += 2) {
      if (j + 1 < n_kv) dma_tile((j + 1) * BC, C<1>{});
      tile(j, C<0>{});
      wait_vmem();
      __syncthreads();
      if (j + 1 < n_kv) {
        if (j + 2 < n_kv) dma_tile((j + 2) * BC, C<0>{});
        tile(j + 1, C<1>{});
        wait_vmem();
        __syncthreads();
      }
    }
  }

  // epilogue: O = sv_ref * O_acc / lq' (POW2: O_acc / lq'), lse = ln2 * (m - kMu + log2 l')
  const float l_tot = halfwave_sum(l_run);
  const float lq_tot = lq_run;  // already the full row sum
  if (qi < Lq) {
    const float inv = lq_tot > 0.f ? (POW2 ? 1.f : sv_ref) / lq_tot : 0.f;
    uint16_t* op = (uint16_t*)a.o + ((int64_t)b * Lq + qi) * a.H * D + (int64_t)h * D + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& o = oacc[dt];
        *(u32x2*)(op + 32 * dt + 8 * g) = u32x2{pack2<kBF16>(o[4 * g] * inv, o[4 * g + 1] * inv),
                                                pack2<kBF16>(o[4 * g + 2] * inv, o[4 * g + 3] * inv)};
      }
    if (hh == 0 && a.lse != nullptr)
      a.lse[(int64_t)bh * Lq + qi] = l_tot > 0.f ? ((POW2 ? m_e : m_run) - kMu + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <bool QK_I8, bool POW2>
static hipError_t launch_8bit(const Fp8Args& a, int D, bool causal, hipStream_t s) {
  if (D != fp8cfg::D) return hipErrorNotSupported;
  const int n = a.B * a.H * a.n_qblk;
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<true, QK_I8, POW2>), dim3(n), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<false, QK_I8, POW2>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int D, bool causal, hipStream_t s) {
  return launch_8bit<false, false>(a, D, causal, s);
}

hipError_t launch_fwd_fp8_pow2(const Fp8Args& a, int D, bool causal, hipStream_t s) {
  return launch_8bit<false, true>(a, D, causal, s);
}

hipError_t launch_fwd_int8(const Fp8Args& a, int D, bool causal, hipStream_t s) {
  return launch_8bit<true, false>(a, D, causal, s);
}

}  // namespace attn
