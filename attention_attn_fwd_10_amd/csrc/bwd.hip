// Backward pass of the fused attention forward for gfx950 (the FlashAttention-3
// summary page, Key Results: the method has a backward pass; the "Fused
// attention kernel" page, When to use which: it follows the forward's
// pattern).  Given dO, the forward's O and its logsumexp, it computes
//
//   P  = exp(scale Q K^T - LSE)            (recomputed tile by tile, masked)
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),   delta_i = <dO_i, O_i>
//   dQ = scale dS K,   dK = scale dS^T Q
//
// without ever storing P or dS in HBM.  delta_i equals rowsum(P * dP) because
// the rows of P sum to one and O = P V.
//
// Three kernels, none with atomics (every output element is summed by one
// wave in a fixed order, so results are run-to-run identical):
//  * bwd_delta_kernel: delta = rowsum(dO * O) in fp32, [B, H, Sq], and the
//    logsumexp in exp2 units, LSE * log2(e) (+inf for rows with no key, whose
//    probabilities are then exactly 0), beside it;
//  * bwd_dkdv_kernel: a workgroup owns 128 keys of one (b, h) (32 per wave,
//    their K and V rows in registers) and walks the query tiles of 64 rows,
//    Q and dO tiles copied asynchronously into a two-stage LDS ring.  Per
//    32-query sub-tile: S = Q K^T and dP = dO V^T on MFMA (Q and dO rows read
//    from LDS in a bit-2/3-swapped order, so each lane's 16 results are two runs
//    of 8 consecutive queries), P and dS in registers, then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read through the LDS transposing read;
//  * bwd_dq_kernel: the forward's layout — a workgroup owns 128 queries (32 per
//    wave, Q and dO fragments in registers), walks the 64-key K/V tiles, forms
//    S^T = K Q^T and dP^T = V dO^T, dS^T in registers, and dQ^T += K^T dS^T
//    with K^T from the transposing read.
// Masks follow the forward (causal bottom-right, keys past Lk excluded); rows
// with no allowed key (LSE = -inf) and rows past Lq pass no gradient.
#include <type_traits>

#include "bwd.hpp"
#include "common.hpp"

namespace attn {

namespace {

// LDS tile of 64 rows with PAD pad slots per row.  One pad slot (272-byte
// rows at d128) suits row reads (ds_read_b128, 16 lanes on 16 bank groups);
// tiles that are also read through the transposing reads take more.  Row r
// starts at element row(r).
template <int D, int PAD = 1>
struct BwdCfg {
  static constexpr bool GROUPED = false;
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int SLOTS = CPR + PAD;    // pad slots per LDS row
  static constexpr int P = 8 * SLOTS;        // LDS row pitch in elements
  static constexpr int TILE = 64 * P;        // elements of a 64-row tile
  static constexpr int row(int r) { return r * P; }
};
// pad slots of padded tiles read both ways
constexpr int kTrPad = 2;

// Grouped tile at head dim 128 (16 chunks of 16 bytes per row).  The tile is
// copied by 16 wave instructions; instruction m writes 1 KB holding rows m,
// m + 16, m + 32, m + 48 and starts at byte 1088 (m % 4) + 4368 (m / 4), so
// row r starts at bank offset 64 (r % 4) + 16 ((r / 4) % 4) (mod 256 bytes):
//  * the 16 rows of a 16-lane ds_read_b128 (any 16 consecutive row indices
//    modulo 16) start in 16 distinct 16-byte bank groups, and
//  * the 4 consecutive rows x 64 bytes of a 32-lane transposing read fill the
//    256 bytes of the banks once.
// row() is additive over the index bit fields (bits 0-1, 2-3, 4-5), so fixed
// row offsets fold into immediates, and a wave's copy round ii moves its
// global offset by 4 ii rows and its LDS destination by row(4 ii).
template <int D>
struct BwdGrp {
  static_assert(D == 128, "the grouped backward tile is laid out for head dim 128");
  static constexpr bool GROUPED = true;
  static constexpr int CPR = D / 8;
  static constexpr int row(int r) { return 544 * (r & 3) + 2184 * ((r >> 2) & 3) + D * (r >> 4); }
  static constexpr int TILE = row(15) + 512;  // the last instruction's 1 KB
};
// layout of the tiles at head dim D (PAD: pad slots of the padded layout)
template <int D, int PAD>
using BwdTile = std::conditional_t<D == 128, BwdGrp<D>, BwdCfg<D, PAD>>;

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (DT == kBF16) {
    return __uint_as_float((uint32_t)x << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, x);
  }
}

// Asynchronous copy of a 64-row tile (rows of D 16-bit values, `row_elems`
// apart in memory, starting at g) into LDS in layout C; rows at or past
// `valid` arrive as zeros without being read.  Padded layout: slot s of the
// tile (16 bytes) is LDS row s / SLOTS, chunk s % SLOTS, and the pad chunk is
// not copied.  Grouped layout: wave instruction i writes rows i + 16 q, q =
// lane / 16, chunk lane % 16.
template <class C>
__device__ __forceinline__ void copy_tile(const uint16_t* g, int64_t row_elems, int valid, uint16_t* lds,
                                          int wave, int lane) {
  const uint32_t row_bytes = 2u * (uint32_t)row_elems;
  const uint64_t n = valid > 0 ? (uint64_t)valid * row_bytes : 0;
  const i32x4 rs = make_rsrc(g, (uint32_t)min(n, (uint64_t)0x7fff0000u));
  if constexpr (C::GROUPED) {
    const uint32_t off = (uint32_t)(wave + 16 * (lane >> 4)) * row_bytes + 16u * (uint32_t)(lane & 15);
#pragma unroll
    for (int ii = 0; ii < C::CPR / 4; ++ii)
      dma16_buf(rs, off + 4u * (uint32_t)ii * row_bytes, lds + C::row(wave) + C::row(4 * ii));
  } else {
#pragma unroll
    for (int ii = 0; ii < (C::SLOTS + 3) / 4; ++ii) {
      const int w = wave + 4 * ii;
      if (w < C::SLOTS) {
        const int s = 64 * w + lane;
        const int r = s / C::SLOTS, c = s - r * C::SLOTS;
        const uint32_t off = c < C::CPR ? (uint32_t)r * row_bytes + 16u * (uint32_t)c : 0x7ffffff0u;
        dma16_buf(rs, off, (uint8_t*)lds + 1024 * w);
      }
    }
  }
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *(const u32x4*)p; }

// Operand A[m][k] (or B[k][n]) = X[k][m] of a row-major LDS tile X in layout
// C: two transposing reads give this lane X[k0 + 8(l/32) + e][m0 + l%32],
// e = 0..7, when p = X + C::row(k0) + m0 + tr_offset<C>(lane).
template <class C>
__host__ __device__ constexpr int tr_offset(int lane) {
  const int g = lane >> 4, j = lane & 15;
  return C::row(8 * (g >> 1) + (j >> 2)) + 16 * (g & 1) + 4 * (j & 3);
}
template <class C>
__device__ __forceinline__ u32x4 lds_tr(const uint16_t* p) {
  const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + C::row(4));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Compile-time check of the grouped tile against the kernels' addressing: the
// copies (every wave, round and lane) fill each element of the 64 rows once,
// at row(R) + column; the row reads (row 32 st + swz23(l), 8 elements at
// 16 kk + 8 hh) find their rows and start the 16 rows of 16 lanes in 16
// distinct 16-byte bank groups; the transposing reads (tr_offset) find
// theirs and touch 32 distinct 8-byte pieces of the 256 bytes of banks per
// 32 lanes.
template <class C>
constexpr bool bwd_grouped_ok() {
  constexpr int D = C::CPR * 8;
  bool seen[C::TILE / 8] = {};
  int key[C::TILE / 8] = {};
  for (int w = 0; w < 4; ++w)
    for (int ii = 0; ii < C::CPR / 4; ++ii)
      for (int l = 0; l < 64; ++l) {
        const int r = w + 4 * ii + 16 * (l >> 4), ch = l & 15;
        const int d = C::row(w) + C::row(4 * ii) + 8 * l;
        if (d + 8 > C::TILE || d != C::row(r) + 8 * ch || seen[d / 8]) return false;
        seen[d / 8] = true;
        key[d / 8] = r * 16 + ch;
      }
  for (int l = 0; l < 64; ++l)
    for (int st = 0; st < 2; ++st)
      for (int kk = 0; kk < D / 16; ++kk) {
        const int r = 32 * st + swz23(l % 32);
        const int e = C::row(r) + 8 * (l / 32) + 16 * kk;
        if (e % 8 || key[e / 8] != r * 16 + 2 * kk + l / 32) return false;
      }
  for (int st = 0; st < 2; ++st)
    for (int hh = 0; hh < 2; ++hh)
      for (int kk = 0; kk < D / 16; ++kk) {
        unsigned g16 = 0;
        for (int l = 0; l < 16; ++l) g16 |= 1u << (((C::row(32 * st + swz23(l)) + 8 * hh + 16 * kk) * 2 / 16) % 16);
        if (g16 != 0xffffu) return false;
      }
  for (int half = 0; half < 2; ++half)
    for (int st = 0; st < 2; ++st)
      for (int c = 0; c < 2; ++c)
        for (int dt = 0; dt < D / 32; ++dt)
          for (int hi = 0; hi < 2; ++hi) {
            unsigned pieces = 0;
            for (int l = 32 * half; l < 32 * half + 32; ++l) {
              const int g = l >> 4, j = l & 15;
              const int r = 8 * (g >> 1) + (j >> 2) + 32 * st + 16 * c + 4 * hi;
              const int col = 32 * dt + 16 * (g & 1) + 4 * (j & 3);
              const int e = tr_offset<C>(l) + C::row(32 * st + 16 * c) + 32 * dt + (hi ? C::row(4) : 0);
              if (key[e / 8] != r * 16 + col / 8 || e % 8 != col % 8) return false;
              pieces |= 1u << ((e * 2 / 8) % 32);
            }
            if (pieces != 0xffffffffu) return false;
          }
  return true;
}
static_assert(bwd_grouped_ok<BwdGrp<128>>(), "grouped backward tile layout");

template <int DT>
__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack2<DT>(x[0], x[1]), pack2<DT>(x[2], x[3]), pack2<DT>(x[4], x[5]), pack2<DT>(x[6], x[7])};
}

// Store an MFMA accumulator of D^T (rows d, column = this lane's row of the
// output) times `mul`: register 4g + i holds d = 32 dt + 8g + 4hh + i.
template <int D, int DT>
__device__ __forceinline__ void store_rows(uint16_t* row, const f32x16 (&acc)[D / 32], float mul, int hh) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& x = acc[dt];
      *(u32x2*)(row + 32 * dt + 8 * g + 4 * hh) =
          u32x2{pack2<DT>(x[4 * g] * mul, x[4 * g + 1] * mul), pack2<DT>(x[4 * g + 2] * mul, x[4 * g + 3] * mul)};
    }
}

}  // namespace

// delta[b, h, i] = sum_d dO[b, i, h, d] * O[b, i, h, d]: D/8 lanes per row.
template <int D, int DT>
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8, RPW = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPW + tid / LPR;  // index into [B, Sq, H]
  const int64_t rows = (int64_t)a.B * a.Sq * a.H;
  const int c = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = *(const u32x4*)((const uint16_t*)a.dout + row * D + 8 * c);
    const u32x4 y = *(const u32x4*)((const uint16_t*)a.o + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(to_f32<DT>((uint16_t)(x[e] & 0xffffu)), to_f32<DT>((uint16_t)(y[e] & 0xffffu)), acc);
      acc = fmaf(to_f32<DT>((uint16_t)(x[e] >> 16)), to_f32<DT>((uint16_t)(y[e] >> 16)), acc);
    }
  }
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < rows && c == 0) {
    const int h = (int)(row % a.H);
    const int64_t bi = row / a.H;
    const int i = (int)(bi % a.Sq), b = (int)(bi / a.Sq);
    const int64_t at = ((int64_t)b * a.H + h) * a.Sq + i;
    a.delta[at] = acc;
    const float l = a.lse[at];
    a.lse2[at] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// (two workgroups per CU: 256 VGPRs per lane at most)
template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdTile<D, kTrPad>;  // Q and dO tiles are read as rows and transposed
  constexpr int BK = 128, BQ = 64;
  __shared__ __attribute__((aligned(16))) uint16_t sq0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sq1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sd0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sd1[C::TILE];
  // per-row vectors of each stage: LSE * log2(e) (64 floats), then delta (64)
  __shared__ __attribute__((aligned(16))) float sv0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sv1[2 * BQ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nkb = (a.Sk + BK - 1) / BK;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / nkb, kb = t - bh * nkb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Lq = a.Sq, Lk = a.Sk, diag = Lk - Lq;
  const int64_t rs = (int64_t)a.H * D;
  const int kw = kb * BK + 32 * wave;  // first key of this wave
  const int key = kw + l32;            // this lane's key
  const uint16_t* const qg = (const uint16_t*)a.q + ((int64_t)b * Lq * a.H + h) * D;
  const uint16_t* const dog = (const uint16_t*)a.dout + ((int64_t)b * Lq * a.H + h) * D;
  const float c2 = a.scale_log2;

  // K and V rows of this lane's key as B operands (column = key, d-slice 16kk + 8hh)
  u32x4 kf[D / 16], vf[D / 16];
  {
    const int64_t kr = ((int64_t)b * Lk + key) * a.H * D + (int64_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = key < Lk ? *(const u32x4*)((const uint16_t*)a.k + kr + 16 * kk) : u32x4{0, 0, 0, 0};
      vf[kk] = key < Lk ? *(const u32x4*)((const uint16_t*)a.v + kr + 16 * kk) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[dt][r] = dk[dt][r] = 0.f;
  const f32x16 zero16 = {};
  const int tro = tr_offset<C>(lane);

  // per-row vectors of a query tile, copied like the tiles (waves 0 and 1, one
  // dword per lane; rows past Lq read as 0, harmless: their Q and dO rows are 0)
  const float* const l2g = a.lse2 + (int64_t)bh * Lq;
  const float* const dlg = a.delta + (int64_t)bh * Lq;
  auto copy_vec = [&](int qt, float* dst) {
    if (wave < 2) {
      const float* g = (wave == 0 ? l2g : dlg) + (int64_t)qt * BQ;
      const int valid = Lq - qt * BQ;
      const i32x4 rs4 = make_rsrc(g, (uint32_t)(4 * min(valid, BQ)));
      raw_buffer_load_lds(rs4, (__attribute__((address_space(3))) void*)(dst + BQ * wave), 4, 4 * lane, 0, 0, 0);
    }
  };

  // (stages are compile-time constants, so the compiler sees that a stage's
  // LDS reads never alias the copies into the other one and does not wait for them)
  auto compute = [&](int qt, auto stage) {
    if (kw >= Lk) return;  // a wave with no key only copies and synchronises
    constexpr bool S1 = decltype(stage)::value;
    const uint16_t* const Qs = S1 ? sq1 : sq0;
    const uint16_t* const Ds = S1 ? sd1 : sd0;
    const float* const Ls = S1 ? sv1 : sv0;
#pragma unroll
    for (int st = 0; st < BQ / 32; ++st) {
      const int qa = qt * BQ + 32 * st;  // first query of the sub-tile
      if (qa >= Lq) break;
      if (CAUSAL && kw > qa + 31 + diag) continue;  // every pair of the wave is masked
      f32x16 s = zero16, dp = zero16;
      const uint16_t* qr = Qs + C::row(32 * st + swz23(l32)) + 8 * hh;
      const uint16_t* dr = Ds + C::row(32 * st + swz23(l32)) + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32<DT>(lds16(qr + 16 * kk), kf[kk], s);
        dp = mfma32<DT>(lds16(dr + 16 * kk), vf[kk], dp);
      }
      // register r: query qa + 16(r/8) + 8hh + r%8 (runs of 8 per lane half);
      // the row vectors are read one run at a time
      u32x4 pk[2], sk[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float* lrow = Ls + 32 * st + 16 * half + 8 * hh;
        const f32x4 l0 = *(const f32x4*)lrow, l1 = *(const f32x4*)(lrow + 4);
        const f32x4 e0 = *(const f32x4*)(lrow + BQ), e1 = *(const f32x4*)(lrow + BQ + 4);
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          float pr = fast_exp2(fmaf(s[r], c2, -(e < 4 ? l0[e] : l1[e - 4])));
          if (CAUSAL) {
            const int qi = qa + 16 * half + 8 * hh + e;
            pr = key > qi + diag ? 0.f : pr;
          }
          p[e] = pr;
          ds[e] = pr * (dp[r] - (e < 4 ? e0[e] : e1[e - 4]));
        }
        pk[half] = pack8<DT>(p);
        sk[half] = pack8<DT>(ds);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int off = C::row(32 * st + 16 * c) + 32 * dt + tro;
          dv[dt] = mfma32<DT>(lds_tr<C>(Ds + off), pk[c], dv[dt]);
          dk[dt] = mfma32<DT>(lds_tr<C>(Qs + off), sk[c], dk[dt]);
        }
    }
  };

  // query tiles that can see this block's keys (causal: i + diag >= first key)
  const int qt0 = CAUSAL ? max(0, kb * BK - diag) / BQ : 0;
  const int nqt = (Lq + BQ - 1) / BQ;
  auto load = [&](int qt, auto stage) {
    constexpr bool S1 = decltype(stage)::value;
    const int64_t r0 = (int64_t)qt * BQ;
    copy_tile<C>(qg + r0 * rs, rs, Lq - (int)r0, S1 ? sq1 : sq0, wave, lane);
    copy_tile<C>(dog + r0 * rs, rs, Lq - (int)r0, S1 ? sd1 : sd0, wave, lane);
    copy_vec(qt, S1 ? sv1 : sv0);
  };
  constexpr std::integral_constant<bool, false> T0{};
  constexpr std::integral_constant<bool, true> T1{};
  if (qt0 < nqt) {
    load(qt0, T0);
    wait_vmem();
    __syncthreads();
    // two tiles per iteration, so that every stage number is a constant
    for (int qt = qt0; qt < nqt; qt += 2) {
      if (qt + 1 < nqt) load(qt + 1, T1);
      compute(qt, T0);
      wait_vmem();
      __syncthreads();
      if (qt + 1 < nqt) {
        if (qt + 2 < nqt) load(qt + 2, T0);
        compute(qt + 1, T1);
        wait_vmem();
        __syncthreads();
      }
    }
  }
  if (key < Lk) {
    const int64_t off = ((int64_t)b * Lk + key) * a.H * D + (int64_t)h * D;
    store_rows<D, DT>((uint16_t*)a.dk + off, dk, a.scale, hh);
    store_rows<D, DT>((uint16_t*)a.dv + off, dv, 1.f, hh);
  }
}

template <int D, int DT, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdArgs a) {
  // K tiles are read as rows and transposed, V tiles as rows only
  using CK = BwdTile<D, kTrPad>;
  using CV = BwdTile<D, 1>;
  constexpr int BQ = 128, BC = 64;
  __shared__ __attribute__((aligned(16))) uint16_t sk0[CK::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[CK::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[CV::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[CV::TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nqb = (a.Sq + BQ - 1) / BQ;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / nqb;
  int qb = t - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest key ranges first
  const int b = bh / a.H, h = bh - b * a.H;
  const int Lq = a.Sq, Lk = a.Sk, diag = Lk - Lq;
  const int64_t rs = (int64_t)a.H * D;
  const int q0 = qb * BQ, qw = q0 + 32 * wave, qi = qw + l32;
  const bool wave_active = qw < Lq;
  const int wave_last_key = CAUSAL ? min(qw + 31, Lq - 1) + diag : Lk - 1;
  const uint16_t* const kg = (const uint16_t*)a.k + ((int64_t)b * Lk * a.H + h) * D;
  const uint16_t* const vg = (const uint16_t*)a.v + ((int64_t)b * Lk * a.H + h) * D;
  const float c2 = a.scale_log2;

  // Q and dO rows of this lane's query as B operands (column = query)
  u32x4 qf[D / 16], df[D / 16];
  {
    const int64_t qr = ((int64_t)b * Lq + qi) * a.H * D + (int64_t)h * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = qi < Lq ? *(const u32x4*)((const uint16_t*)a.q + qr + 16 * kk) : u32x4{0, 0, 0, 0};
      df[kk] = qi < Lq ? *(const u32x4*)((const uint16_t*)a.dout + qr + 16 * kk) : u32x4{0, 0, 0, 0};
    }
  }
  float lse2 = INFINITY, del = 0.f;
  if (qi < Lq) {
    lse2 = a.lse2[(int64_t)bh * Lq + qi];
    del = a.delta[(int64_t)bh * Lq + qi];
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;
  const f32x16 zero16 = {};
  const int tro = tr_offset<CK>(lane);

  auto compute = [&](int j, auto stage) {
    const int key0 = j * BC;
    if (!wave_active || (CAUSAL && key0 > wave_last_key)) return;
    constexpr bool S1 = decltype(stage)::value;
    const uint16_t* const Ks = S1 ? sk1 : sk0;
    const uint16_t* const Vs = S1 ? sv1 : sv0;
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt) {
      f32x16 s = zero16, dp = zero16;
      const uint16_t* kr = Ks + CK::row(32 * tt + swz23(l32)) + 8 * hh;
      const uint16_t* vr = Vs + CV::row(32 * tt + swz23(l32)) + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32<DT>(lds16(kr + 16 * kk), qf[kk], s);
        dp = mfma32<DT>(lds16(vr + 16 * kk), df[kk], dp);
      }
      // register r: key key0 + 32tt + 16(r/8) + 8hh + r%8
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = key0 + 32 * tt + 16 * (r >> 3) + 8 * hh + (r & 7);
        float pr = fast_exp2(fmaf(s[r], c2, -lse2));
        const bool masked = kj >= Lk || (CAUSAL && kj > qi + diag);
        pr = masked ? 0.f : pr;
        ds[r] = pr * (dp[r] - del);
      }
      // dQ^T += K^T dS^T for this sub-tile's two 16-key steps
      const u32x4 dsk[2] = {pack8<DT>(ds), pack8<DT>(ds + 8)};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          dq[dt] = mfma32<DT>(lds_tr<CK>(Ks + CK::row(32 * tt + 16 * c) + 32 * dt + tro), dsk[c], dq[dt]);
    }
  };

  int n_kv = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last = min(q0 + BQ, Lq) - 1 + diag;
    n_kv = last < 0 ? 0 : min(n_kv, last / BC + 1);
  }
  auto load = [&](int j, auto stage) {
    constexpr bool S1 = decltype(stage)::value;
    const int64_t r0 = (int64_t)j * BC;
    copy_tile<CK>(kg + r0 * rs, rs, Lk - (int)r0, S1 ? sk1 : sk0, wave, lane);
    copy_tile<CV>(vg + r0 * rs, rs, Lk - (int)r0, S1 ? sv1 : sv0, wave, lane);
  };
  constexpr std::integral_constant<bool, false> T0{};
  constexpr std::integral_constant<bool, true> T1{};
  if (n_kv > 0) {
    load(0, T0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < n_kv; j += 2) {
      if (j + 1 < n_kv) load(j + 1, T1);
      compute(j, T0);
      wait_vmem();
      __syncthreads();
      if (j + 1 < n_kv) {
        if (j + 2 < n_kv) load(j + 2, T0);
        compute(j + 1, T1);
        wait_vmem();
        __syncthreads();
      }
    }
  }
  if (qi < Lq)
    store_rows<D, DT>((uint16_t*)a.dq + ((int64_t)b * Lq + qi) * a.H * D + (int64_t)h * D, dq, a.scale, hh);
}

template <int D, int DT, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.H;
  const int rpw = 256 / (D / 8);
  const int nkb = (a.Sk + 127) / 128, nqb = (a.Sq + 127) / 128;
  // (with no query every key gradient is zero: the dK/dV kernel then writes zeros)
  if (rows > 0)
    hipLaunchKernelGGL((bwd_delta_kernel<D, DT>), dim3((unsigned)((rows + rpw - 1) / rpw)), dim3(256), 0, s, a);
  if (nkb > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, CAUSAL>), dim3(a.B * a.H * nkb), dim3(256), 0, s, a);
  if (nqb > 0) hipLaunchKernelGGL((bwd_dq_kernel<D, DT, CAUSAL>), dim3(a.B * a.H * nqb), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t launch_bwd_c(const BwdArgs& a, bool causal, hipStream_t s) {
  return causal ? launch_bwd_t<D, DT, true>(a, s) : launch_bwd_t<D, DT, false>(a, s);
}

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t s) {
  if (D == 64) return dtype == kBF16 ? launch_bwd_c<64, kBF16>(a, causal, s) : launch_bwd_c<64, kFP16>(a, causal, s);
  if (D == 128) return dtype == kBF16 ? launch_bwd_c<128, kBF16>(a, causal, s) : launch_bwd_c<128, kFP16>(a, causal, s);
  return hipErrorNotSupported;
}

}  // namespace attn
