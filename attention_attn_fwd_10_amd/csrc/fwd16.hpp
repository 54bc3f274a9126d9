// Fused attention forward, 16-bit inputs (bf16 / fp16), for gfx950.
//
// What is computed follows the "Fused attention kernel" page (Implementation
// sketch): one query block stays on chip, key/value blocks stream past it, a
// running row max m and row sum l are kept, the old state is rescaled by
// alpha = exp(m_old - m_new), every key block (including a partial last one)
// is scored, and o / l and lse = m + log l are formed once at the end.
//
// How it maps to CDNA4:
//  * one workgroup = 4 waves = 128 query rows (8 waves = 256 rows for the
//    dense causal layout); each wave owns 32 rows and keeps its Q fragments in
//    registers for the whole key loop;
//  * K and V tiles of 64 keys go through a two-stage LDS ring filled by
//    asynchronous global -> LDS copies (buffer_load_dwordx4 ... lds): the
//    copies of a tile are issued a step before it is used and need no
//    registers (one barrier per tile);
//  * tiles that need no mask are software-pipelined inside each wave: the
//    score MFMAs of tile j+1 are interleaved, in a fixed order, with the
//    softmax of tile j, then the P V MFMAs of tile j with its last
//    exponentials, so one wave keeps the matrix core and the vector ALU busy
//    at the same time; tiles with a mask run one at a time;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16, so
//    every lane owns one query column: the row max and row sum are in-lane
//    reductions plus one half-wave exchange (v_permlane32_swap);
//  * the second GEMM is O^T = V^T P^T: P^T comes straight from the score
//    accumulators (no LDS round trip) and V^T is read from the row-major V tile
//    with the LDS transposing read ds_read_b64_tr_b16, so V is never
//    transposed in memory;
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA;
//  * the running max is only moved when a row's new maximum exceeds it by more
//    than 2^8 (in probability units): between moves the probabilities are
//    bounded by 256, the result is the same exact identity, and the output
//    rescale (D/32 x 16 multiplies per lane) is skipped on almost every tile;
//  * tiles are copied with buffer loads whose range ends at the sequence's
//    last key row: rows past Lk arrive as zeros without being read, and are
//    masked; query rows past the sequence end are zero-filled, so whatever
//    memory lies past the sequence never reaches the result.
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "ring.hpp"

namespace attn {

// Waves per workgroup: 8 (256 query rows, one workgroup per CU, each K/V tile
// copied once for all 8 waves) for the dense causal layout at head dim 128 and
// for the wide dense layout (kDenseWide), where they measured faster;
// otherwise 4 (128 rows, two or more workgroups per CU), which suits the
// packed layouts, whose sequences may be short, runs a grid that does not fill
// whole rounds of one-workgroup-per-CU slots with a shorter tail, lets head
// dim 64 run three or four workgroups per CU (below), and is the only choice
// at head dim 256, where a SIMD holds one wave.
constexpr int fwd16_waves(int D, int MODE, bool CAUSAL) {
  return MODE == kDenseWide || (D == 128 && CAUSAL && (MODE == kDense || MODE == kDenseBias)) ? 8 : 4;
}

// The software-pipelined key loop (the next tile's scores during this tile's
// softmax) keeps two score tiles in registers.  At head dim 64 it needs about
// 193 VGPRs, i.e. 2 waves per SIMD, while the tile-at-a-time loop needs about
// 125 and runs 3-4 waves per SIMD (34 KB of LDS per 4-wave workgroup), which
// hides the vector work of one wave behind the matrix work of the others
// better than the in-wave overlap does: measured 2-15 % faster non-causal and
// up to 48 % causal over the sweep, bit-identical.  At head dim 128 the
// tile-at-a-time loop still needs 2 waves per SIMD (and 68 KB of LDS per
// workgroup), and the pipelined one is faster.
constexpr bool fwd16_pipelined(int D, int MODE) { return D != 64 && MODE != kDenseBias; }

template <int D, int NW = 4>
struct Fwd16Cfg {
  static constexpr int BR = 32 * NW;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  // LDS layout of a 64-row tile.  A tile is copied by CPR wave instructions of
  // 64 lanes x 16 bytes, each writing 1 KB of whole rows: instruction m holds
  // the rows R with R % CPR == m (lane l: row m + CPR * (l / CPR), chunk
  // l % CPR).  The instructions sit 1 KB plus a gap apart, and the gap spreads
  // the rows that one LDS read instruction touches together over the banks:
  // 16 bytes for K, whose 16 rows read by 16 consecutive lanes (ds_read_b128)
  // then start in 16 different 16-byte bank groups; 64 bytes for V, whose
  // transposing reads fetch, per 32 lanes, 4 consecutive rows x 2 x 32 bytes
  // (the 4 rows then start 64 bytes apart in the banks).  Row R
  // starts at element row(R) = (R % CPR) * GRP + (R / CPR) * D; row() is
  // additive over index bits, so fixed row offsets fold into immediates.
  static constexpr int KGRP = 512 + 8;            // instruction pitches in elements
  static constexpr int VGRP = 512 + 32;
  static constexpr int K_ELEMS = CPR * KGRP;
  static constexpr int V_ELEMS = CPR * VGRP;
  static constexpr int krow(int r) { return (r % CPR) * KGRP + (r / CPR) * D; }
  static constexpr int vrow(int r) { return (r % CPR) * VGRP + (r / CPR) * D; }
  // each wave copies CPR / NW instructions of each of K and V per tile
  static_assert(CPR % NW == 0, "the copy instructions of a tile are dealt evenly to the waves");
  static constexpr int CI_W = CPR / NW;
  // copy round ii of a wave is tile instruction wave + NW * ii; lane l copies
  // 16-byte chunk copy_chunk(l) of LDS row copy_row(wave, ii, l) to element
  // (wave + NW * ii) * GRP + 8 l of the stage
  static constexpr int copy_row(int wave, int ii, int lane) { return wave + NW * ii + CPR * (lane / CPR); }
  static constexpr int copy_chunk(int lane) { return lane % CPR; }
  // key held by LDS row r of a K tile (each 32-row group in swz23 order); V
  // row r holds key r
  static constexpr int k_key(int r) { return (r & ~31) | swz23(r & 31); }
  // waves per SIMD: at least three at head dim 64 (the tile-at-a-time loop),
  // two at 128 (one workgroup of 8 waves or two of 4 per CU), one at 256
  static constexpr int WAVES_PER_EU = D == 64 ? 3 : D <= 128 ? 2 : 1;
  static constexpr int MIN_BLOCKS = WAVES_PER_EU * 4 / NW;
};

// Compile-time check of a tile layout against the kernel's addressing:
//  * the copies (every wave, round and lane) fill each element of the tile's
//    64 rows exactly once, inside the stage, at row(R) + column;
//  * a round's key is the round-0 key plus the compile-time shift the copies
//    add (k_key(NW ii) for K, NW ii for V);
//  * the K operand reads (row 32 tt + swz23(l), 8 elements at 16 kk + 8 hh)
//    find key 32 tt + swz23(l), and the 16 rows of 16 consecutive lanes start
//    in 16 distinct 16-byte bank groups (of 256 bytes);
//  * the transposing V reads of 32 lanes touch 32 distinct 8-byte pieces of
//    the 256 bytes of banks.
template <class C>
constexpr bool fwd16_layout_ok() {
  constexpr int D = C::CPR * 8;
  bool kseen[C::K_ELEMS / 8] = {}, vseen[C::V_ELEMS / 8] = {};
  int kkey[C::K_ELEMS / 8] = {}, vkey[C::V_ELEMS / 8] = {};
  for (int w = 0; w < C::BR / 32; ++w)
    for (int ii = 0; ii < C::CI_W; ++ii)
      for (int l = 0; l < 64; ++l) {
        const int r = C::copy_row(w, ii, l), ch = C::copy_chunk(l);
        const int kd = (w + (C::BR / 32) * ii) * C::KGRP + 8 * l, vd = (w + (C::BR / 32) * ii) * C::VGRP + 8 * l;
        if (r < 0 || r >= 64 || kd + 8 > C::K_ELEMS || vd + 8 > C::V_ELEMS) return false;
        if (kd != C::krow(r) + 8 * ch || vd != C::vrow(r) + 8 * ch) return false;
        if (kseen[kd / 8] || vseen[vd / 8]) return false;
        kseen[kd / 8] = vseen[vd / 8] = true;
        kkey[kd / 8] = C::k_key(r) * 64 + ch;
        vkey[vd / 8] = r * 64 + ch;
        if (C::k_key(r) != C::k_key(C::copy_row(w, 0, l)) + C::k_key((C::BR / 32) * ii)) return false;
        if (r != C::copy_row(w, 0, l) + (C::BR / 32) * ii) return false;
      }
  for (int l = 0; l < 64; ++l)
    for (int tt = 0; tt < 2; ++tt)
      for (int kk = 0; kk < D / 16; ++kk) {
        const int e = C::krow(32 * tt + l % 32) + 8 * (l / 32) + 16 * kk;
        if (e % 8 || !kseen[e / 8] || kkey[e / 8] != (32 * tt + swz23(l % 32)) * 64 + 2 * kk + l / 32) return false;
      }
  for (int tt = 0; tt < 2; ++tt)
    for (int hh = 0; hh < 2; ++hh)
      for (int kk = 0; kk < D / 16; ++kk) {
        unsigned seen = 0;
        for (int l = 0; l < 16; ++l) seen |= 1u << (((C::krow(32 * tt + l) + 8 * hh + 16 * kk) * 2 / 16) % 16);
        if (seen != 0xffffu) return false;
      }
  for (int half = 0; half < 2; ++half)
    for (int hi = 0; hi < 2; ++hi)
      for (int c = 0; c < 4; ++c)
        for (int dt = 0; dt < D / 32; ++dt) {
          unsigned seen = 0;
          for (int l = 32 * half; l < 32 * half + 32; ++l) {
            const int g = l >> 4, j = l & 15;
            const int row = 8 * (g >> 1) + (j >> 2) + 16 * c + 4 * hi;
            const int col = 32 * dt + 16 * (g & 1) + 4 * (((j & 1) << 1) | ((j >> 1) & 1));
            const int e = C::vrow(row) + col;
            if (!vseen[e / 8] || vkey[e / 8] != row * 64 + col / 8) return false;
            seen |= 1u << ((e * 2 / 8) % 32);
          }
          if (seen != 0xffffffffu) return false;
        }
  return true;
}
static_assert(fwd16_layout_ok<Fwd16Cfg<64, 4>>() && fwd16_layout_ok<Fwd16Cfg<64, 8>>(), "fwd16 tile layout, head dim 64");
static_assert(fwd16_layout_ok<Fwd16Cfg<128, 4>>() && fwd16_layout_ok<Fwd16Cfg<128, 8>>(), "fwd16 tile layout, head dim 128");
static_assert(fwd16_layout_ok<Fwd16Cfg<256, 4>>(), "fwd16 tile layout, head dim 256");
static_assert(Fwd16Cfg<64, 8>::BR == kWideRows && Fwd16Cfg<128, 8>::BR == kWideRows, "rows of a wide workgroup");

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Probabilities may grow to 2^kLazyRescale before the running max is moved.
constexpr float kLazyRescale = 8.0f;

template <int D, int DT, bool CAUSAL, int MODE>
__global__ void __launch_bounds__((64 * fwd16_waves(D, MODE, CAUSAL)), (Fwd16Cfg<D, fwd16_waves(D, MODE, CAUSAL)>::MIN_BLOCKS))
    fwd16_kernel(FwdArgs a) {
  constexpr int NW = fwd16_waves(D, MODE, CAUSAL);
  using C = Fwd16Cfg<D, NW>;
  constexpr int BR = C::BR, BC = C::BC, CPR = C::CPR;
  constexpr bool DENSE = MODE == kDense || MODE == kDenseBias || MODE == kDenseWide;
  constexpr bool BIAS = MODE == kDenseBias;
  constexpr bool WIDE = MODE == kDenseWide;
  static_assert(!WIDE || (D == 128 && !CAUSAL), "the wide dense layout is the non-causal forward at head dim 128");
  static_assert(!BIAS || D <= 128, "the score bias is supported up to head dim 128");
  // The two stages of the K and V rings are separate arrays: when a stage is
  // named by a compile-time constant, the compiler can tell the copies into
  // one stage from the reads of the other and does not make those reads wait
  // for the copies (with a run-time stage index it waits for all of them).
  __shared__ __attribute__((aligned(16))) uint16_t lds_k0[C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_k1[C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v0[C::V_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v1[C::V_ELEMS];
  // stage -> array; `buf` is an int or a std::integral_constant
  auto kbuf = [&](auto buf) -> uint16_t* {
    if constexpr (std::is_same_v<decltype(buf), int>) return buf ? lds_k1 : lds_k0;
    else return decltype(buf)::value ? lds_k1 : lds_k0;
  };
  auto vbuf = [&](auto buf) -> uint16_t* {
    if constexpr (std::is_same_v<decltype(buf), int>) return buf ? lds_v1 : lds_v0;
    else return decltype(buf)::value ? lds_v1 : lds_v0;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // ---- work item: (b, h, query block) -------------------------------------
  // Wide layout: workgroups [0, tail_start) run work items [0, tail_start)
  // whole (XCD-remapped); each later work item runs as n_split workgroups,
  // one key range each (the tail of the grid, spread over every CU).
  int t, split = 0;
  bool tail = false;
  if (WIDE && (int)blockIdx.x >= a.tail_start) {
    const int u = (int)blockIdx.x - a.tail_start;
    t = a.tail_start + u / a.n_split;
    split = u - (u / a.n_split) * a.n_split;
    tail = true;
  } else {
    t = xcd_remap(blockIdx.x, WIDE ? a.tail_start : (int)gridDim.x);
  }
  int b, h, qblk;
  if constexpr (DENSE) {
    const int bh = t / a.n_qblk;
    qblk = t - bh * a.n_qblk;
    if (CAUSAL) qblk = a.n_qblk - 1 - qblk;  // longest key ranges first
    b = bh / a.H;
    h = bh - b * a.H;
  } else {
    // compact tile list: sequence b owns H * ceil(Lq_b / BR) consecutive tiles
    // (head-major), so no workgroup is spent on query blocks past a sequence;
    // with split keys, consecutive workgroups are the splits of one tile
    int rem = t, nq = 0;
    if (a.n_split > 1) {
      split = t % a.n_split;
      rem = t / a.n_split;
    }
    for (b = 0; b < a.B; ++b) {
      nq = (a.cu_q[b + 1] - a.cu_q[b] + BR - 1) / BR;
      if (rem < a.H * nq) break;
      rem -= a.H * nq;
    }
    if (b == a.B) return;  // past the last tile (the grid is an upper bound)
    h = rem / nq;
    qblk = rem - h * nq;
    if (CAUSAL) qblk = nq - 1 - qblk;
  }

  int Lq, Lk;
  int64_t qoff, ooff, koff, voff, lse_base;
  if constexpr (DENSE) {
    Lq = a.Sq;
    Lk = a.Sk;
    qoff = b * a.q_sb + h * a.q_sh;
    ooff = b * a.o_sb + h * a.o_sh;
    koff = b * a.k_sb + h * a.k_sh;
    voff = b * a.v_sb + h * a.v_sh;
    lse_base = ((int64_t)b * a.H + h) * a.Sq;
  } else {
    const int q0 = a.cu_q[b];
    Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b];
    Lk = a.cu_k[b + 1] - k0;
    qoff = (int64_t)q0 * a.q_ss + h * a.q_sh;
    ooff = (int64_t)q0 * a.o_ss + h * a.o_sh;
    if constexpr (MODE == kVarlen) {
      koff = (int64_t)k0 * a.k_ss + h * a.k_sh;
      voff = (int64_t)k0 * a.v_ss + h * a.v_sh;
    } else {
      koff = h * a.k_sh;
      voff = h * a.v_sh;
    }
    lse_base = (int64_t)h * a.total_q + q0;
  }
  const int qs = qblk * BR;
  if (qs >= Lq) return;  // uniform over the workgroup

  int n_kv = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last = min(qs + BR, Lq) - 1 + (Lk - Lq);  // last key any row of the block may see
    n_kv = last < 0 ? 0 : min(n_kv, last / BC + 1);
  }
  // key tiles [j0, j1) of this work item (all of them unless keys are split)
  int j0 = 0, j1 = n_kv;
  if (WIDE && tail) {
    j0 = min(n_kv, split * a.split_tiles);
    j1 = min(n_kv, j0 + a.split_tiles);
  }
  if constexpr (!DENSE) {
    if (a.n_split > 1) {
      j0 = min(n_kv, split * a.split_tiles);
      j1 = min(n_kv, j0 + a.split_tiles);
    }
  }

  const int qw = qs + 32 * wave;  // first query row of this wave
  const int qi = qw + l32;        // this lane's query row
  const bool wave_active = qw < Lq;
  const int diag = Lk - Lq;       // causal: key j allowed for row i iff j <= i + diag
  const int wave_last_key = CAUSAL ? min(qw + 31, Lq - 1) + diag : Lk - 1;

  // ---- Q fragments: lane (query l32, half hh) holds q[16kk + 8hh .. +7] ----
  u32x4 qf[D / 16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + qoff + (int64_t)qi * a.q_ss + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = qi < Lq ? *(const u32x4*)(qp + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // ---- K/V tiles: asynchronous global -> LDS copies --------------------------
  // LDS row R of a K tile holds key (R & ~31) | swz23(R & 31), i.e. the rows of
  // each 32-row group in swz23 order; row R of a V tile holds key R.
  // score bias: one buffer resource over this (b, h) plane (rows of bias_ss
  // elements, the last one readable up to a multiple of 8 elements, so that no
  // 16-byte read straddles the range end; reads past it return zeros), and
  // this lane's row offset
  i32x4 bias_rsrc = {0, 0, 0, 0};
  uint32_t bias_row = 0;
  if constexpr (BIAS) {
    const uint16_t* bp = (const uint16_t*)a.bias + b * a.bias_sb + h * a.bias_sh;
    const uint64_t nbytes = 2ull * ((uint64_t)(Lq - 1) * (uint64_t)a.bias_ss + (uint64_t)((Lk + 7) & ~7));
    bias_rsrc = make_rsrc(bp, (uint32_t)min(nbytes, (uint64_t)0x7fff0000u));
    bias_row = 2u * (uint32_t)((int64_t)min(qi, Lq - 1) * a.bias_ss);
  }
  const uint16_t* const kg = (const uint16_t*)a.k + koff;
  const uint16_t* const vg = (const uint16_t*)a.v + voff;
  // the key and 16-byte chunk this lane copies in its copy round ii (wave
  // instruction wave + NW * ii of the tile)
  auto k_slot = [&](int ii, int& key_local, int& chunk) {
    key_local = C::k_key(C::copy_row(wave, ii, lane));
    chunk = C::copy_chunk(lane);
  };
  auto v_slot = [&](int ii, int& key_local, int& chunk) {
    key_local = C::copy_row(wave, ii, lane);
    chunk = C::copy_chunk(lane);
  };
  // From one round to the next only the instruction index moves, by NW, in
  // index bits that no other term of the row uses; the key therefore moves by
  // a compile-time amount (swz23(NW * ii) for K, NW * ii for V) and the lane's
  // byte offset inside the tile is that of round 0 plus a scalar, so one
  // register per operand holds the offsets of every round.
  auto k_key_shift = [](int ii) { return C::k_key(NW * ii); };
  auto v_key_shift = [](int ii) { return NW * ii; };
  uint32_t k_boff, v_boff;
  {
    int kl, ch;
    k_slot(0, kl, ch);
    k_boff = 2u * (uint32_t)(kl * (int)a.k_ss + ch * 8);
    v_slot(0, kl, ch);
    v_boff = 2u * (uint32_t)(kl * (int)a.v_ss + ch * 8);
  }
  auto row_of = [&](int key) -> int64_t {  // element offset of key's row (paged: through the table)
    if constexpr (MODE == kPaged) {
      const int page = a.block_table[(int64_t)b * a.max_pages + (key >> a.page_shift)];
      return (((int64_t)page << a.page_shift) | (key & ((1 << a.page_shift) - 1)));
    } else {
      return key;
    }
  };
  // A 64-key tile is contiguous in memory for the dense and varlen layouts,
  // and inside one page of a paged cache whose pages hold >= 64 tokens.  Then
  // every copy is a single buffer load whose resource ends at row Lk (rows
  // past the sequence end read as zeros).  Smaller pages: each row through
  // the block table.
  const bool contiguous = MODE != kPaged || a.page_shift >= 6;
  // (the table is read through the constant address space: with a uniform
  // index that is a scalar load, which the tile copies never wait behind)
  typedef const __attribute__((address_space(4))) int32_t cint32;
  auto tile_row0 = [&](int key0) -> int64_t {  // element row of key0 (paged: page base + slot)
    if constexpr (MODE == kPaged) {
      const int page = ((cint32*)a.block_table)[(int64_t)b * a.max_pages + (key0 >> a.page_shift)];
      return ((int64_t)page << a.page_shift) + (key0 & ((1 << a.page_shift) - 1));
    } else {
      return key0;
    }
  };
  // (row0: tile_row0(key0), looked up once per tile by the caller)
  // Copies of a tile whose rows are contiguous: one buffer resource from the
  // tile's first row to row Lk (rows past the sequence end read as zeros);
  // round ii adds the byte offset of its key shift to the lane's round-0
  // offset (a scalar, below 2^31 since the shift is < 64 rows).
  // (a resource covers the tile's own rows, at most 64, so its size fits
  // 32 bits: 64 rows of at most 2^25 bytes; the copies never address past
  // row 63 of a tile, and rows past Lk read as zeros)
  const uint32_t k_rowb = 2u * (uint32_t)a.k_ss, v_rowb = 2u * (uint32_t)a.v_ss;
  // (one copy round ii of this wave: one instruction)
  auto dma_k_round = [&](int key0, auto buf, int64_t row0, int ii) {
    uint16_t* kb = kbuf(buf) + wave * C::KGRP;
    const i32x4 kr = make_rsrc(kg + row0 * a.k_ss, (uint32_t)min(Lk - key0, BC) * k_rowb);
    dma16_buf(kr, k_boff + 2u * (uint32_t)k_key_shift(ii) * (uint32_t)a.k_ss, kb + NW * ii * C::KGRP);
  };
  auto dma_v_round = [&](int key0, auto buf, int64_t row0, int ii) {
    uint16_t* vb = vbuf(buf) + wave * C::VGRP;
    const i32x4 vr = make_rsrc(vg + row0 * a.v_ss, (uint32_t)min(Lk - key0, BC) * v_rowb);
    dma16_buf(vr, v_boff + 2u * (uint32_t)v_key_shift(ii) * (uint32_t)a.v_ss, vb + NW * ii * C::VGRP);
  };
  auto dma_k_c = [&](int key0, auto buf, int64_t row0) {
#pragma unroll
    for (int ii = 0; ii < C::CI_W; ++ii) dma_k_round(key0, buf, row0, ii);
  };
  auto dma_v_c = [&](int key0, auto buf, int64_t row0) {
#pragma unroll
    for (int ii = 0; ii < C::CI_W; ++ii) dma_v_round(key0, buf, row0, ii);
  };
  // Copies for any layout: contiguous tiles as above; otherwise (pages of
  // fewer than 64 tokens) each row through the block table, rows past Lk
  // repeating row Lk-1 (finite data, masked out of the scores and multiplied
  // by p = 0).
  auto dma_k = [&](int key0, auto buf, int64_t row0) {
    if (contiguous) {
      dma_k_c(key0, buf, row0);
    } else {
      uint16_t* kb = kbuf(buf) + wave * C::KGRP;
#pragma unroll
      for (int ii = 0; ii < C::CI_W; ++ii) {
        int kl, ch;
        k_slot(ii, kl, ch);
        dma16(kg + row_of(min(key0 + kl, Lk - 1)) * a.k_ss + ch * 8, kb + NW * ii * C::KGRP);
      }
    }
  };
  auto dma_v = [&](int key0, auto buf, int64_t row0) {
    if (contiguous) {
      dma_v_c(key0, buf, row0);
    } else {
      uint16_t* vb = vbuf(buf) + wave * C::VGRP;
#pragma unroll
      for (int ii = 0; ii < C::CI_W; ++ii) {
        int kl, ch;
        v_slot(ii, kl, ch);
        dma16(vg + row_of(min(key0 + kl, Lk - 1)) * a.v_ss + ch * 8, vb + NW * ii * C::VGRP);
      }
    }
  };
  auto dma_tile = [&](int key0, int buf) {
    const int64_t row0 = contiguous ? tile_row0(key0) : 0;
    dma_k(key0, buf, row0);
    dma_v(key0, buf, row0);
  };

  // V^T operand addressing for ds_read_b64_tr_b16: lane (group g, index j)
  // points at key 8*(g/2) + j/4 (+4 for the second read) and head-dim column
  // 16*(g%2) + 4*swap(j%4), so that after the transpose lane l holds
  // V[key 8*(l/32) + e][d = swz23(l % 32)] for e = 0..7.
  const int vg_grp = lane >> 4, vg_j = lane & 15;
  const int vtr_off = C::vrow(8 * (vg_grp >> 1) + (vg_j >> 2)) + 16 * (vg_grp & 1) +
                      4 * (((vg_j & 1) << 1) | ((vg_j >> 1) & 1));

  // ---- running state ---------------------------------------------------------
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*s (moved lazily)
  float l_run = 0.f;        // this half-wave's share of the running sum
  const float c2 = a.scale_log2;
  const f32x16 zero16 = {};
  if constexpr (D == 256) {
    // At D = 256 the registers exceed the 256 VGPRs; an AGPR operand here makes
    // the compiler select the MFMA forms whose accumulators live in AGPRs, so
    // the 128 output accumulators stay there instead of being copied between
    // the two register files every tile.
    int agpr_hint;
    asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(agpr_hint));
    (void)agpr_hint;
  }

  // score bias of this lane's row for the tile at key0: four 16-byte loads,
  // one per run of 8 consecutive keys it holds (issued before the tile's copy
  // of the next tile so that waiting for them does not wait for that copy)
  struct BiasRaw {
    i32x4 r[BC / 32][2];
  };
  auto bias_fetch = [&](int key0) {
    BiasRaw br;
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        br.r[tt][half] = raw_buffer_load_v4(bias_rsrc, (int)(bias_row + 2u * (uint32_t)(key0 + 32 * tt + 16 * half + 8 * hh)), 0, 0);
    return br;
  };
  // s <- s * c2 + bias * log2(e): the scores in exp2 units with the bias added
  auto bias_apply = [&](f32x16 (&sc)[BC / 32], const BiasRaw& br) {
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t u = (uint32_t)br.r[tt][half][w];
          float lo, hi;
          if constexpr (DT == kBF16) {
            lo = __uint_as_float(u << 16);
            hi = __uint_as_float(u & 0xffff0000u);
          } else {
            lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
            hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
          }
          const int r = 8 * half + 2 * w;
          sc[tt][r] = fmaf(sc[tt][r], c2, lo * kLog2e);
          sc[tt][r + 1] = fmaf(sc[tt][r + 1], c2, hi * kLog2e);
        }
  };
  // with a bias the scores are already in exp2 units after bias_apply
  const float c2k = BIAS ? 1.f : c2;

  // one key tile (head dims up to 128)
  auto compute = [&](int key0, int buf, const BiasRaw& br) {
    if (!wave_active) return;
    if (CAUSAL && key0 > wave_last_key) return;  // tile fully masked for this wave
    // S^T = K Q^T
    const uint16_t* ks = kbuf(buf) + C::krow(l32) + 8 * hh;
    f32x16 s[BC / 32];
    {
      // the K operands of the tile are read before the first MFMA so that the
      // LDS latency is paid once (at D = 256 in two halves, which keeps them
      // within the register budget); the two score tiles form independent
      // chains
      constexpr int NKK = D / 16;
      constexpr int KG = D == 256 ? NKK / 4 : NKK;  // k steps read per group
#pragma unroll
      for (int g = 0; g < NKK / KG; ++g) {
        u32x4 kop[BC / 32][KG];
#pragma unroll
        for (int kk = 0; kk < KG; ++kk)
#pragma unroll
          for (int tt = 0; tt < BC / 32; ++tt) kop[tt][kk] = *(const u32x4*)(ks + C::krow(32 * tt) + 16 * (g * KG + kk));
        __builtin_amdgcn_sched_barrier(0);  // keep the group's reads ahead of its MFMAs
        __builtin_amdgcn_s_setprio(1);       // favour this wave while it feeds the matrix core
#pragma unroll
        for (int kk = 0; kk < KG; ++kk)
#pragma unroll
          for (int tt = 0; tt < BC / 32; ++tt)
            s[tt] = mfma32<DT>(kop[tt][kk], qf[g * KG + kk], g == 0 && kk == 0 ? zero16 : s[tt]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if constexpr (BIAS) bias_apply(s, br);
    // register r of tile tt holds key key0 + 32tt + 16(r/8) + 8hh + r%8
    const bool need_mask = (key0 + BC > Lk) || (CAUSAL && key0 + BC - 1 > qw + diag);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * tt + 16 * (r >> 3) + 8 * hh + (r & 7);
          const bool bad = key >= Lk || (CAUSAL && key > qi + diag);
          if (bad) s[tt][r] = -INFINITY;
        }
    }
    const float mx = tile_max32(s[0], s[1]);
    const float mxs = halfwave_max(mx) * c2k;
    // move the running max only when some row's new max exceeds it by > 2^8;
    // the row sum takes alpha in the same fused update as the pipelined tiles
    // (l = fma(l, alpha, psum)), so every path rounds it identically
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0) {
      const float m_new = max2f(m_run, mxs);
      alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (D == 256) {
            // the accumulator stays in its AGPR: read, scale, write back
            float t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32_e32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(oacc[dt][r]), "=&v"(t)
                         : "v"(alpha));
          } else {
            oacc[dt][r] *= alpha;
          }
        }
      m_run = m_new;
    }
    const float nb = m_run == -INFINITY ? 0.f : -m_run;
    const uint16_t* vs = vbuf(buf) + vtr_off;
    float psum;  // (starts at the first probability: 0 + p is p exactly)
    // O^T += V^T P^T over four 16-key chunks: the exponentials of a chunk, then
    // its D/32 MFMAs, so the matrix work of one chunk overlaps the next chunk's
    // exponentials
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int tt = c >> 1, r0p = 8 * (c & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(s[tt][r0p + e], c2k, nb));
        psum = c == 0 && e == 0 ? p[e] : psum + p[e];
      }
      const u32x4 pk = {pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]),
                        pack2<DT>(p[6], p[7])};
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint16_t* vp = vs + C::vrow(16 * c) + 32 * dt;
        const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + C::vrow(4));
        oacc[dt] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk, oacc[dt]);
      }
    }
    l_run = fmaf(l_run, alpha, psum);
  };

  // ---- one key tile in three pieces (head dim 256) ---------------------------
  f32x16 s[BC / 32];  // scores of the current tile
  float mxs = 0.f;    // their row max (scaled, log2 units)
  // tiles past this wave's causal diagonal are skipped whole
  auto tile_active = [&](int key0) { return wave_active && !(CAUSAL && key0 > wave_last_key); };
  // S^T = K Q^T, masking and the row max; true when the running max must move
  auto scores_max = [&](int key0, int buf) -> bool {
    const uint16_t* ks = kbuf(buf) + C::krow(l32) + 8 * hh;
    {
      // the K operands of the tile are read before the first MFMA so that the
      // LDS latency is paid once (at D = 256 in quarters, which keeps them
      // within the register budget); the two score tiles form independent
      // chains
      constexpr int NKK = D / 16;
      constexpr int KG = D == 256 ? NKK / 4 : NKK;  // k steps read per group
#pragma unroll
      for (int g = 0; g < NKK / KG; ++g) {
        u32x4 kop[BC / 32][KG];
#pragma unroll
        for (int kk = 0; kk < KG; ++kk)
#pragma unroll
          for (int tt = 0; tt < BC / 32; ++tt) kop[tt][kk] = *(const u32x4*)(ks + C::krow(32 * tt) + 16 * (g * KG + kk));
        __builtin_amdgcn_sched_barrier(0);  // keep the group's reads ahead of its MFMAs
        __builtin_amdgcn_s_setprio(1);       // favour this wave while it feeds the matrix core
#pragma unroll
        for (int kk = 0; kk < KG; ++kk)
#pragma unroll
          for (int tt = 0; tt < BC / 32; ++tt)
            s[tt] = mfma32<DT>(kop[tt][kk], qf[g * KG + kk], g == 0 && kk == 0 ? zero16 : s[tt]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    // register r of tile tt holds key key0 + 32tt + 16(r/8) + 8hh + r%8
    const bool need_mask = (key0 + BC > Lk) || (CAUSAL && key0 + BC - 1 > qw + diag);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * tt + 16 * (r >> 3) + 8 * hh + (r & 7);
          const bool bad = key >= Lk || (CAUSAL && key > qi + diag);
          if (bad) s[tt][r] = -INFINITY;
        }
    }
    const float mx = tile_max32(s[0], s[1]);
    mxs = halfwave_max(mx) * c2;
    // move the running max only when some row's new max exceeds it by > 2^8
    return __builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0;
  };
  // move the running max and rescale the accumulators; the row sum takes
  // alpha in softmax_pv's fused update
  float alpha_pend = 1.f;
  auto rescale = [&]() {
    const float m_new = max2f(m_run, mxs);
    const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
    alpha_pend = alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (D == 256) {
          // the accumulator stays in its AGPR: read, scale, write back
          float t;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32_e32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(oacc[dt][r]), "=&v"(t)
                       : "v"(alpha));
        } else {
          oacc[dt][r] *= alpha;
        }
      }
    m_run = m_new;
  };
  // P = exp2(c2 s - m), O^T += V^T P^T over four 16-key chunks: the
  // exponentials of a chunk, then its D/32 MFMAs, so the matrix work of one
  // chunk overlaps the next chunk's exponentials
  auto softmax_pv = [&](int buf) {
    const float nb = m_run == -INFINITY ? 0.f : -m_run;
    const uint16_t* vs = vbuf(buf) + vtr_off;
    float psum;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int tt = c >> 1, r0p = 8 * (c & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(s[tt][r0p + e], c2, nb));
        psum = c == 0 && e == 0 ? p[e] : psum + p[e];
      }
      const u32x4 pk = {pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]),
                        pack2<DT>(p[6], p[7])};
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint16_t* vp = vs + C::vrow(16 * c) + 32 * dt;
        const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + C::vrow(4));
        oacc[dt] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk, oacc[dt]);
      }
    }
    l_run = fmaf(l_run, alpha_pend, psum);
    alpha_pend = 1.f;
  };

  // ---- software-pipelined pieces (head dims up to 128, tiles needing no mask)
  // S^T = K Q^T of one tile
  auto qk_tile = [&](auto buf, f32x16 (&sc)[BC / 32]) {
    const uint16_t* ks = kbuf(buf) + C::krow(l32) + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int tt = 0; tt < BC / 32; ++tt) {
        const u32x4 kop = *(const u32x4*)(ks + C::krow(32 * tt) + 16 * kk);
        sc[tt] = mfma32<DT>(kop, qf[kk], kk == 0 ? zero16 : sc[tt]);
      }
  };
  // row max, lazy max move, P = exp2(c2 s - m) packed to 16 bits and the row
  // sum, with no branch; returns whether the running max moved, in which case
  // the accumulators must still be multiplied by alpha
  auto softmax_pack = [&](const f32x16 (&sc)[BC / 32], u32x4 (&pk)[BC / 16], float& alpha) -> bool {
    const float mx = tile_max32(sc[0], sc[1]);
    const float mxs = halfwave_max(mx) * c2;
    const bool moved = __builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0;
    const float m_new = moved ? max2f(m_run, mxs) : m_run;
    const float m_safe = m_new == -INFINITY ? 0.f : m_new;
    alpha = fast_exp2(m_run - m_safe);
    m_run = m_new;
    float psum;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int tt = c >> 1, r0p = 8 * (c & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sc[tt][r0p + e], c2, -m_safe));
        psum = c == 0 && e == 0 ? p[e] : psum + p[e];
      }
      pk[c] = u32x4{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]), pack2<DT>(p[6], p[7])};
    }
    l_run = fmaf(l_run, alpha, psum);
    return moved;
  };
  auto scale_acc = [&](float alpha) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
  };
  // O^T += V^T P^T of one tile
  auto pv_tile = [&](auto buf, const u32x4 (&pk)[BC / 16]) {
    const uint16_t* vs = vbuf(buf) + vtr_off;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint16_t* vp = vs + C::vrow(16 * c) + 32 * dt;
        const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + C::vrow(4));
        oacc[dt] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[c], oacc[dt]);
      }
  };
  // ---- key loop: two-stage LDS ring; tile j uses stage (j - j0) % 2 --------
  if (j1 > j0) {
    if constexpr (D != 256) {
      // The ring's schedule (ring.hpp) is executed from its tables: op o of a
      // table run for tile j acts on tile j + o.d, in stage (j + o.d - j0) %
      // 2; `par` is the stage of tile j, a compile-time constant in the
      // pipelined loop and an int in the one-at-a-time loop, and `math(kind,
      // stage, copy)` does the reads.  Copies marked in_math are left to the
      // math, which issues round r of the table's k-th such copy as
      // copy(k * CI_W + r) (every round once).  The tables are proven free of
      // stage hazards at compile time (ring.hpp), so no copy, wait or barrier
      // exists outside them.
      int jm = j0;  // end of the pipelined tiles
      auto stage_of = [](auto par, auto dd) {
        constexpr int DD = decltype(dd)::value;
        if constexpr (std::is_same_v<decltype(par), int>) return (par + DD) & 1;
        else return std::integral_constant<int, (decltype(par)::value + DD) & 1>{};
      };
      // (contig: the pipelined tiles, whose copies are single buffer loads)
      auto run = [&](auto table, int j, auto par, auto contig, auto&& math) {
        using T = decltype(table);
        // the in_math copies' buffer resources and guards, formed once
        constexpr int NIM = T::in_math_count > 0 ? T::in_math_count : 1;
        i32x4 im_rsrc[NIM];
        bool im_ok[NIM];
        static_for<T::size>([&](auto I) {
          constexpr ring::Op o = T::at(decltype(I)::value);
          if constexpr (o.in_math) {
            constexpr int k = T::in_math_index(decltype(I)::value);
            const int t = j + o.d;
            im_ok[k] = ring::guard_ok(o.guard, t - j0, jm - j0, j1 - j0);
            const int64_t row0 = tile_row0(t * BC);
            if constexpr (o.kind == ring::kCopyK)
              im_rsrc[k] = make_rsrc(kg + row0 * a.k_ss, (uint32_t)min(Lk - t * BC, BC) * k_rowb);
            else
              im_rsrc[k] = make_rsrc(vg + row0 * a.v_ss, (uint32_t)min(Lk - t * BC, BC) * v_rowb);
          }
        });
        // round `part % CI_W` of the table's (part / CI_W)-th in_math copy
        auto copy = [&](int part) {
          static_for<T::size>([&](auto I) {
            constexpr ring::Op o = T::at(decltype(I)::value);
            if constexpr (o.in_math) {
              static_assert(decltype(contig)::value && (o.kind == ring::kCopyK || o.kind == ring::kCopyV),
                            "copies left to the math are the pipelined single-buffer K or V copies");
              constexpr int k = T::in_math_index(decltype(I)::value);
              if (part / C::CI_W != k || !im_ok[k]) return;
              const auto st = stage_of(par, std::integral_constant<int, o.d>{});
              const int ii = part % C::CI_W;
              if constexpr (o.kind == ring::kCopyK)
                dma16_buf(im_rsrc[k], k_boff + 2u * (uint32_t)k_key_shift(ii) * (uint32_t)a.k_ss,
                          kbuf(st) + wave * C::KGRP + NW * ii * C::KGRP);
              else
                dma16_buf(im_rsrc[k], v_boff + 2u * (uint32_t)v_key_shift(ii) * (uint32_t)a.v_ss,
                          vbuf(st) + wave * C::VGRP + NW * ii * C::VGRP);
            }
          });
        };
        static_for<T::size>([&](auto I) {
          constexpr ring::Op o = T::at(decltype(I)::value);
          if constexpr (o.in_math) return;  // issued by the math through `copy`
          const int t = j + o.d;
          if (!ring::guard_ok(o.guard, t - j0, jm - j0, j1 - j0)) return;
          const auto st = stage_of(par, std::integral_constant<int, o.d>{});
          if constexpr (o.kind == ring::kCopyK) {
            if constexpr (decltype(contig)::value) dma_k_c(t * BC, st, tile_row0(t * BC));
            else dma_k(t * BC, st, contiguous ? tile_row0(t * BC) : 0);
          } else if constexpr (o.kind == ring::kCopyV) {
            if constexpr (decltype(contig)::value) dma_v_c(t * BC, st, tile_row0(t * BC));
            else dma_v(t * BC, st, contiguous ? tile_row0(t * BC) : 0);
          } else if constexpr (o.kind == ring::kCopyKV) {
            static_assert(!decltype(contig)::value, "the pipelined tables copy K and V separately");
            dma_tile(t * BC, st);
          } else if constexpr (o.kind == ring::kWait) {
            wait_vmem();
          } else if constexpr (o.kind == ring::kSync) {
            __syncthreads();
          } else {
            math(std::integral_constant<int, o.kind>{}, st, copy);
          }
        });
      };
      int jg = j0;  // first tile of the generic loop below
      // (not with a score bias, and for paged caches only with pages of >= 64
      // tokens, whose tiles are copied like contiguous ones: the registers of
      // the pipeline and of the per-row page-table copies do not fit together)
      if (fwd16_pipelined(D, MODE) && contiguous) {
        // Tiles [j0, jm) need no mask for any row of the block.  They run
        // software-pipelined: while the softmax of tile j is on the vector
        // units, the same wave issues the score MFMAs of tile j+1; then P V of
        // tile j.  K and V copies are a step apart (K(j+2) and V(j+1) land
        // during step j), so the ring keeps two stages of each.
        jm = CAUSAL ? (qs + diag + 1) / BC : Lk / BC;
        jm = min(j1, max(j0, jm));
        if (jm > j0) {
          constexpr std::integral_constant<int, 0> S0{};
          constexpr std::integral_constant<int, 1> S1{};
          f32x16 sa[BC / 32], sb[BC / 32];
          // (a tile's first row: its first key, or for a paged cache its
          // page's base plus the slot, one table read per copied tile)
          // prologue: K(j0), V(j0), K(j0 + 1); the scores of tile j0.  Waves
          // whose rows all lie past the sequence end only copy and
          // synchronise (with one query row, as in decoding, three of four).
          // The first step copies K(j0 + 2) into stage 0, so a barrier
          // separates the scores from it: every wave must have read K(j0)
          // first (waves with no rows skip the read and would otherwise
          // overwrite the stage while it is still being read).
          run(ring::Table<ring::kPrologue>{}, j0, S0, std::true_type{}, [&](auto, auto st, auto&&) {
            if (wave_active) qk_tile(st, sa);
          });
          // One step with the next tile's scores overlapped (needs j + 1 < jm).
          // The order of the work is fixed by scheduling fences: region A
          // issues the NA score MFMAs of tile j+1, and after each one a share
          // of the softmax of tile j (row max, lazy max move, then the first
          // 24 of the 32 exponentials per lane); region B issues the NB P V
          // MFMAs of tile j, in 16-key chunks, and the last 8 exponentials
          // after its first MFMAs (they feed the last chunk).
          // In the wide layout the step's copies (K(j+2), V(j+1): D/64 rounds
          // each per wave) are spread over region A, one after each of the
          // score MFMAs 4, 6, 8 and 10 (at d128, measured 1 % faster than issuing them
          // first; in region B they land too late for the step's closing
          // wait, and the step ran 6 % slower).  Elsewhere they precede the
          // step: the causal 8-wave kernel spills about 190 registers with
          // them spread, and the 4-wave kernels issue twice the rounds.
          constexpr bool kSpread = WIDE;
          using StepTable = std::conditional_t<kSpread, ring::Table<ring::kStepSpread>, ring::Table<ring::kStep>>;
          constexpr int kParts = StepTable::in_math_count * C::CI_W;  // copy rounds the math issues
          static_assert(kParts == 0 || 4 + 2 * (kParts - 1) < (D / 16) * (BC / 32), "the spread copies fit region A");
          auto step_math = [&](auto cur, auto nxt, f32x16 (&sc)[BC / 32], f32x16 (&sn)[BC / 32], auto&& copy) {
            constexpr int NA = (D / 16) * (BC / 32), NB = (D / 32) * (BC / 16);
            constexpr int KPRE = 3, VPRE = 2;
            const uint16_t* ks = kbuf(nxt) + C::krow(l32) + 8 * hh;
            const uint16_t* vs = vbuf(cur) + vtr_off;
            float p[BC / 2];
            u32x4 pk[BC / 16];
            float psum = 0.f, mx = 0.f, m_safe = 0.f, alpha = 1.f;  // (psum starts at p[0])
            bool moved = false;
            // exponentials [lo, hi) in chunk-major order (value 8c + e is
            // register 8(c%2) + e of score tile c/2); a chunk is packed as soon
            // as its 8 values exist
            auto exps = [&](int lo, int hi) {
#pragma unroll
              for (int x = lo; x < hi; ++x) {
                const int c = x >> 3, e = x & 7;
                p[x] = fast_exp2(fmaf(sc[c >> 1][8 * (c & 1) + e], c2, -m_safe));
                psum = x == 0 ? p[x] : psum + p[x];
                if (e == 7)
                  pk[c] = u32x4{pack2<DT>(p[x - 7], p[x - 6]), pack2<DT>(p[x - 5], p[x - 4]),
                                pack2<DT>(p[x - 3], p[x - 2]), pack2<DT>(p[x - 1], p[x])};
              }
            };
            // (8 waves: the second wave of each SIMD, waves 4-7, is raised
            // over region A; the hardware otherwise favours the older wave,
            // which then idles at the barrier while the younger one finishes,
            // measured 0.7 % slower in the wide layout and 3 % slower causal)
            __builtin_amdgcn_sched_barrier(0);
            if (NW == 8 && wave >= 4) __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);
            u32x4 kop[NA];
#pragma unroll
            for (int i = 0; i < KPRE; ++i) kop[i] = *(const u32x4*)(ks + C::krow(32 * (i & 1)) + 16 * (i >> 1));
#pragma unroll
            for (int i = 0; i < NA; ++i) {
              const int kk = i >> 1, tt = i & 1;
              sn[tt] = mfma32<DT>(kop[i], qf[kk], kk == 0 ? zero16 : sn[tt]);
              if (i + KPRE < NA)
                kop[i + KPRE] = *(const u32x4*)(ks + C::krow(32 * ((i + KPRE) & 1)) + 16 * ((i + KPRE) >> 1));
              if (i == 0) {
                mx = max3f(sc[0][0], sc[0][1], sc[0][2]);
#pragma unroll
                for (int r = 3; r < 15; r += 2) mx = max3f(mx, sc[0][r], sc[0][r + 1]);
              } else if (i == 1) {
                mx = max3f(mx, sc[0][15], sc[1][0]);
#pragma unroll
                for (int r = 1; r < 15; r += 2) mx = max3f(mx, sc[1][r], sc[1][r + 1]);
                mx = max2f(mx, sc[1][15]);
              } else if (i == 2) {
                // (no mask in these tiles: every score and the new max are
                // finite, and alpha = 2^(m_old - m_new) is 0 on a row's first tile)
                const float mxs = halfwave_max(mx) * c2;
                moved = __builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0;
                m_safe = moved ? max2f(m_run, mxs) : m_run;
                alpha = fast_exp2(m_run - m_safe);
                m_run = m_safe;
              } else {
                exps((i - 3) * 24 / (NA - 3), (i - 2) * 24 / (NA - 3));
              }
              if constexpr (kParts > 0) {
                if (i >= 4 && (i & 1) == 0 && (i - 4) / 2 < kParts) copy((i - 4) / 2);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (NW == 8) __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            // keep P here: otherwise it is sunk past the rescale branch below
#pragma unroll
            for (int c = 0; c < 3; ++c) asm volatile("" : "+v"(pk[c]));
            if (moved) scale_acc(alpha);
            __builtin_amdgcn_sched_barrier(0);
            u32x2 vop[NB][2];
#pragma unroll
            for (int i = 0; i < VPRE; ++i) {
              const uint16_t* vp = vs + C::vrow(16 * (i / (D / 32))) + 32 * (i % (D / 32));
              vop[i][0] = lds_read_tr16(vp);
              vop[i][1] = lds_read_tr16(vp + C::vrow(4));
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
              const int c = i / (D / 32), dt = i % (D / 32);
              oacc[dt] = mfma32<DT>(u32x4{vop[i][0][0], vop[i][0][1], vop[i][1][0], vop[i][1][1]}, pk[c], oacc[dt]);
              if (i + VPRE < NB) {
                const uint16_t* vp = vs + C::vrow(16 * ((i + VPRE) / (D / 32))) + 32 * ((i + VPRE) % (D / 32));
                vop[i + VPRE][0] = lds_read_tr16(vp);
                vop[i + VPRE][1] = lds_read_tr16(vp + C::vrow(4));
              }
              if (i < NB / 2) exps(24 + i * 8 / (NB / 2), 24 + (i + 1) * 8 / (NB / 2));
              if (i == NB / 2 - 1) l_run = fmaf(l_run, alpha, psum);
              __builtin_amdgcn_sched_barrier(0);
            }
          };
          auto step = [&](int j, auto cur, auto nxt, f32x16 (&sc)[BC / 32], f32x16 (&sn)[BC / 32]) {
            run(StepTable{}, j, cur, std::true_type{}, [&](auto, auto, auto&& copy) {
              if (wave_active) {
                step_math(cur, nxt, sc, sn, copy);
              } else {
#pragma unroll
                for (int part = 0; part < kParts; ++part) copy(part);  // a wave with no rows still copies its share
              }
            });
          };
          // the last pipelined tile: softmax and P V only
          auto last = [&](int j, auto cur, f32x16 (&sc)[BC / 32]) {
            run(ring::Table<ring::kLast>{}, j, cur, std::true_type{}, [&](auto, auto, auto&&) {
              if (wave_active) {
                u32x4 pk[BC / 16];
                float alpha;
                if (softmax_pack(sc, pk, alpha)) scale_acc(alpha);
                pv_tile(cur, pk);
              }
            });
          };
          int j = j0;
          for (; j + 2 < jm; j += 2) {
            step(j, S0, S1, sa, sb);
            step(j + 1, S1, S0, sb, sa);
          }
          if (j + 1 < jm) {
            step(j, S0, S1, sa, sb);
            last(j + 1, S1, sb);
          } else {
            last(j, S0, sa);
          }
          jg = jm;  // tile jm (if any) is in stage (jm - j0) % 2
        }
      }
      // tiles one at a time (tile j + 1 lands while tile j is computed)
      if (jg == j0) run(ring::Table<ring::kTileStart>{}, j0, 0, std::false_type{}, [](auto, auto, auto&&) {});
      for (int j = jg; j < j1; ++j) {
        const int buf = (j - j0) & 1;
        BiasRaw br{};
        if constexpr (BIAS) br = bias_fetch(j * BC);
        run(ring::Table<ring::kTile>{}, j, buf, std::false_type{}, [&](auto, auto st, auto&&) { compute(j * BC, st, br); });
      }
    } else {
      dma_tile(j0 * BC, 0);
      wait_vmem();
      __syncthreads();
      // The inner loop runs the tiles that need no rescale and leaves at the
      // first that does; the rescale (rare after the first tiles) happens
      // outside it, so the accumulators, which live in AGPRs at this head
      // dim, are only ever touched by MFMAs inside the inner loop.
      int j = j0;
      while (j < j1) {
        bool pending = false;
        for (; j < j1; ++j) {
          const int buf = (j - j0) & 1;
          if (j + 1 < j1) dma_tile((j + 1) * BC, buf ^ 1);
          if (tile_active(j * BC)) {
            if (scores_max(j * BC, buf)) {
              pending = true;
              break;
            }
            softmax_pv(buf);
          }
          wait_vmem();
          __syncthreads();
        }
        if (pending) {
          rescale();
          softmax_pv((j - j0) & 1);
          wait_vmem();
          __syncthreads();
          ++j;
        }
      }
    }
  }

  // ---- epilogue: o / l, lse = ln2 * (m + log2 l) -----------------------------
  const float l_tot = halfwave_sum(l_run);
  // partial result of a key range, in fp32, at pp (this row's D values) and
  // pl (its logsumexp); register r of tile dt is head-dim column 32dt +
  // 16(r/8) + 8hh + r%8
  auto store_partial = [&](float* pp, float* pl) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    pp += 8 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x16& o = oacc[dt];
        const int r0p = 8 * half;
        float* dst = pp + 32 * dt + 16 * half;
        *(f32x4*)dst = f32x4{o[r0p] * inv, o[r0p + 1] * inv, o[r0p + 2] * inv, o[r0p + 3] * inv};
        *(f32x4*)(dst + 4) = f32x4{o[r0p + 4] * inv, o[r0p + 5] * inv, o[r0p + 6] * inv, o[r0p + 7] * inv};
      }
    if (hh == 0) *pl = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  };
  if constexpr (WIDE) {
    if (tail) {
      if (qi < Lq) {
        const int64_t n_rows = ((int64_t)a.B * a.H * a.n_qblk - a.tail_start) * BR;
        const int64_t row = (int64_t)split * n_rows + (int64_t)(t - a.tail_start) * BR + (qi - qs);
        store_partial(a.part_o + row * D, a.part_lse + row);
      }
      return;
    }
  }
  if constexpr (!DENSE) {
    if (a.n_split > 1) {
      if (qi < Lq) {
        const int64_t row = (int64_t)split * a.total_q + (lse_base - (int64_t)h * a.total_q) + qi;
        store_partial(a.part_o + (row * a.H + h) * D, a.part_lse + (int64_t)split * a.H * a.total_q + lse_base + qi);
      }
      return;
    }
  }
  if (qi < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)a.o + ooff + (int64_t)qi * a.o_ss + 8 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0p = 8 * half;
        const f32x16& o = oacc[dt];
        *(u32x4*)(op + 32 * dt + 16 * half) =
            u32x4{pack2<DT>(o[r0p + 0] * inv, o[r0p + 1] * inv), pack2<DT>(o[r0p + 2] * inv, o[r0p + 3] * inv),
                  pack2<DT>(o[r0p + 4] * inv, o[r0p + 5] * inv), pack2<DT>(o[r0p + 6] * inv, o[r0p + 7] * inv)};
      }
    if (hh == 0 && a.lse != nullptr)
      a.lse[lse_base + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int DT, bool CAUSAL, int MODE>
hipError_t launch_fwd16(FwdArgs a, hipStream_t s) {
  constexpr int NW = fwd16_waves(D, MODE, CAUSAL), BR = Fwd16Cfg<D, NW>::BR;
  // dense: every (b, h, q-block); varlen: an upper bound on the compact tile list
  int n;
  if constexpr (MODE == kDense || MODE == kDenseBias) {
    a.n_qblk = (a.Sq + BR - 1) / BR;
    n = a.B * a.H * a.n_qblk;
  } else if constexpr (MODE == kDenseWide) {
    // (n_qblk, tail_start and the split are set by the caller, which sizes
    // the partial results)
    n = a.tail_start + (a.B * a.H * a.n_qblk - a.tail_start) * a.n_split;
  } else {
    n = a.H * ((a.total_q + BR - 1) / BR + a.B) * max(a.n_split, 1);
  }
  hipLaunchKernelGGL((fwd16_kernel<D, DT, CAUSAL, MODE>), dim3(n), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

#define ATTN_INSTANTIATE_FWD16_BIAS(D)                                                        \
  template hipError_t launch_fwd16<D, kBF16, false, kDenseBias>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16<D, kBF16, true, kDenseBias>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, false, kDenseBias>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16<D, kFP16, true, kDenseBias>(FwdArgs, hipStream_t);

#define ATTN_INSTANTIATE_FWD16_WIDE(D)                                                       \
  template hipError_t launch_fwd16<D, kBF16, false, kDenseWide>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16<D, kFP16, false, kDenseWide>(FwdArgs, hipStream_t);

#define ATTN_INSTANTIATE_FWD16(D)                                          \
  template hipError_t launch_fwd16<D, kBF16, false, kDense>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, true, kDense>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16<D, kFP16, false, kDense>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, true, kDense>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16<D, kBF16, false, kVarlen>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16<D, kBF16, true, kVarlen>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, false, kVarlen>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16<D, kFP16, true, kVarlen>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, false, kPaged>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, true, kPaged>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16<D, kFP16, false, kPaged>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, true, kPaged>(FwdArgs, hipStream_t);

}  // namespace attn
