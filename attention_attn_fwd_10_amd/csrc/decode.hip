// Decoding forward ("Fused attention kernel" page, section "Implementation
// sketch": a row's running max and running sum over key blocks; the
// FlashAttention-3 page's future-work note on LLM inference): one query row
// per sequence against a long, optionally paged key cache, at head dim 64,
// 128 or 256 (its own kernel below: two lanes per key).
//
// With one query row the two products are matrix-vector products, so the
// matrix cores have nothing to share and the work is bound by the bytes of K
// and V.  What matters is how many of them are in flight: the tiled kernel
// stages every K/V tile through a two-stage LDS ring, one tile ahead, which
// caps the bytes in flight at about half the LDS of a CU.  Here every wave
// owns a (sequence, key range, head) and streams its K/V tiles straight into
// registers, a tile's V and the next tile's K in flight while it computes.
//
// Work items run with the head index fastest: the waves that run together
// read the neighbouring 256-byte head slices of the same cache rows, so every
// row is fetched from memory as a whole (head-slowest order left each row to
// be read in 256-byte pieces at different times: 14-17 % slower).
//
// Per 64-key tile and wave:
//  * K: lane j loads the 2D-byte row of key j (D/8 16-byte buffer loads);
//    its score is D/2 dot2 products (bf16 or fp16 pairs, fp32 accumulation,
//    four independent chains) against the query's D/2 pairs, held in scalar
//    registers;
//  * the next tile's K loads are issued as soon as the scores are formed, so
//    they are in flight during the softmax and the P V product;
//  * online softmax across the lanes: the tile's max over the wave, the
//    running max m (in base-2 units of scale * q.k), p = 2^(x - m), the row
//    sum in fp32 (a per-lane share, summed over the wave at the end);
//  * V: each of the 64 key rows is one coalesced 2D-byte load, lane l taking
//    head-dim columns 2l and 2l+1 (at D = 64 lanes 32..63 repeat the addresses
//    of lanes 0..31, which adds no memory traffic, and their results are
//    dropped); a byte permute pairs two keys' values of
//    one column, and a dot2 against the two keys' probabilities (rounded to
//    the input type, as for the matrix-core product of the tiled kernel,
//    broadcast from the lanes that computed them) accumulates the output.
// Every buffer resource ends at the last key of the tile that belongs to the
// range (and is empty past the range), so rows past the sequence (or past a
// page's used slots) read as zeros and never reach the output.
//
// With several key ranges each (range, row, head) writes the split-key
// path's partial result: its normalised fp32 output and natural-log
// logsumexp (0 and -inf for an empty range), which splitkv_merge_kernel
// combines.  With one range it writes the output in the input type and the
// logsumexp directly.
#include "common.hpp"

namespace attn {

// buffer_load_dword / _dwordx2 into registers (zeros past the resource's range)
__device__ int raw_buffer_load_b32(i32x4 rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.i32");
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
__device__ i32x2 raw_buffer_load_v2(i32x4 rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.v2i32");

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) x = max2f(x, __shfl_xor(x, s));
  return halfwave_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) x += __shfl_xor(x, s);
  return halfwave_sum(x);
}

// A wave's work item: (sequence b, key range `split`, head h), head index
// fastest, and what both decode kernels derive from it.
struct DecodeItem {
  int b, h, split, row;  // row: the sequence's query row in the packed q / o
  int kseq, kbeg, kend;  // first key row of a packed cache; key range [kbeg, kend)
};
// False when the item is past the grid or its sequence has no query row.
// Ranges are split_tiles 64-key tiles long; one range takes every key.
__device__ __forceinline__ bool decode_item(const FwdArgs& a, DecodeItem& it) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  if (item >= (int64_t)a.B * a.H * a.n_split) return false;
  it.h = (int)(item % a.H);
  const int64_t bs = item / a.H;
  it.split = (int)(bs % a.n_split);
  it.b = (int)(bs / a.n_split);
  it.row = a.cu_q[it.b];
  if (a.cu_q[it.b + 1] - it.row <= 0) return false;
  it.kseq = a.cu_k[it.b];
  const int Lk = a.cu_k[it.b + 1] - it.kseq;
  it.kbeg = it.split * a.split_tiles * 64;
  it.kend = a.n_split == 1 ? Lk : min(Lk, it.kbeg + a.split_tiles * 64);
  return true;
}
// Element offset of key k0's (b, h) slice of a [rows, H, D] cache (paged:
// through the block table; a tile starting at k0 never straddles a page).
__device__ __forceinline__ int64_t decode_tile_off(const FwdArgs& a, const DecodeItem& it, int D, int k0) {
  int64_t base_row;
  if (a.block_table != nullptr) {
    const int page = a.block_table[(int64_t)it.b * a.max_pages + (k0 >> a.page_shift)];
    base_row = ((int64_t)page << a.page_shift) + (k0 & ((1 << a.page_shift) - 1));
  } else {
    base_row = (int64_t)it.kseq + k0;
  }
  return (base_row * a.H + it.h) * D;
}
// Pages of 2^PS tokens (PS = 4 or 5): the first cache row of each of the NPG
// pages of the tile at k0 with nvalid keys in the range; the table entries
// are read as scalars and clamped to the range's last page, so no entry past
// the keys the range owns is read.
template <int PS, int NPG>
__device__ __forceinline__ void decode_tile_pages(const FwdArgs& a, const DecodeItem& it, int k0, int nvalid,
                                                  int64_t (&pg)[NPG]) {
  typedef const __attribute__((address_space(4))) int32_t cint32;
  cint32* tab = (cint32*)a.block_table + (int64_t)it.b * a.max_pages + (k0 >> PS);
#pragma unroll
  for (int g = 0; g < NPG; ++g) pg[g] = (int64_t)tab[min(g, (nvalid - 1) >> PS)] << PS;
}

// FwdArgs of the packed or paged varlen forward: every sequence with at most
// one query row, head dim D; n_split >= 1 key ranges of split_tiles tiles
// (part_o / part_lse when n_split > 1).  PS = 0: a packed cache or pages of at
// least 64 tokens (a 64-key tile lies in one page: buffer loads whose resource
// ends at the range's last key).  PS = 4 or 5: pages of 2^PS tokens; a tile
// spans 64 >> PS pages, whose table entries it reads once (as scalars), and
// every K and V row is addressed through its page.  Keys of the last tile past
// the range then read the range's last row again (their scores are masked),
// and the prefetch past the range reads the current tile again (from L2), so
// no address leaves the range's pages.
template <int DT, int D, int PS>
__global__ void __launch_bounds__(256) decode_kernel(FwdArgs a) {
  static_assert(D == 64 || D == 128, "head dims of the decode kernel");
  static_assert(PS == 0 || PS == 4 || PS == 5, "small pages of 16 or 32 tokens");
  constexpr int BC = 64;
  constexpr int NPG = PS > 0 ? BC >> PS : 1;  // pages per tile
  constexpr int NCOL = D / 2;  // lanes that own a head-dim column pair
  const int lane = threadIdx.x & 63;
  DecodeItem it;
  if (!decode_item(a, it)) return;  // (no barriers below)
  const int h = it.h, split = it.split, row = it.row, kbeg = it.kbeg, kend = it.kend;

  // the query's D/2 pairs, in scalar registers (read through the constant
  // address space: a uniform address the kernel never writes)
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  cu32* qp = (cu32*)((const uint16_t*)a.q + ((int64_t)row * a.H + h) * D);
  uint32_t qw[D / 2];
#pragma unroll
  for (int i = 0; i < D / 2; ++i) qw[i] = qp[i];

  const uint32_t row_bytes = (uint32_t)a.H * D * 2;  // <= 2^25 (H * D <= 2^24, checked by the caller)
  auto tile_off = [&](int k0) { return decode_tile_off(a, it, D, k0); };
  auto tile_bytes = [&](int k0) -> uint32_t { return (uint32_t)(min(BC, kend - k0) - 1) * row_bytes + D * 2; };
  float m = -INFINITY;       // running max (uniform over the wave)
  float l_lane = 0.f;        // this lane's share of the row sum
  float o0 = 0.f, o1 = 0.f;  // head-dim columns 2 col and 2 col + 1
  const int col = lane % NCOL;
  // small pages: the first cache row of each page of the tile at k0, and the
  // element offset of a row slice
  auto tile_pages = [&](int k0, int64_t (&pg)[NPG]) { decode_tile_pages<PS>(a, it, k0, min(BC, kend - k0), pg); };
  auto row_slice = [&](int64_t cache_row) { return (cache_row * a.H + h) * D; };
  uint32_t kw[D / 2];  // K row of key `lane` of the current tile
  // K rows of the tile at k0 (< kend) into kw
  auto load_k_small = [&](int k0) {
    int64_t pg[NPG];
    tile_pages(k0, pg);
    const int jj = min(lane, kend - k0 - 1);  // (keys past the range: the last row again)
    int64_t base = pg[0];
#pragma unroll
    for (int g = 1; g < NPG; ++g) base = (jj >> PS) == g ? pg[g] : base;
    const u32x4* kp = (const u32x4*)((const uint16_t*)a.k + row_slice(base + (jj & ((1 << PS) - 1))));
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 x = kp[c];
#pragma unroll
      for (int w = 0; w < 4; ++w) kw[4 * c + w] = x[w];
    }
  };
  if constexpr (PS > 0) {
    if (kbeg < kend) load_k_small(kbeg);
  } else if (kbeg < kend) {
    const i32x4 krs = make_rsrc((const uint16_t*)a.k + tile_off(kbeg), tile_bytes(kbeg));
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const i32x4 x = raw_buffer_load_v4(krs, (int)(lane * row_bytes + 16 * c), 0, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) kw[4 * c + w] = (uint32_t)x[w];
    }
  }
  for (int k0 = kbeg; k0 < kend; k0 += BC) {
    const int nvalid = min(BC, kend - k0);
    uint32_t vw[BC];  // V column pair `lane` of every key of the tile
    if constexpr (PS > 0) {
      int64_t pg[NPG];
      tile_pages(k0, pg);
#pragma unroll
      for (int j = 0; j < BC; ++j) {
        const int jj = min(j, nvalid - 1);  // (uniform)
        const uint32_t* vp = (const uint32_t*)((const uint16_t*)a.v + row_slice(pg[jj >> PS] + (jj & ((1 << PS) - 1))));
        vw[j] = vp[col];
      }
    } else {
      const i32x4 vrs = make_rsrc((const uint16_t*)a.v + tile_off(k0), tile_bytes(k0));
#pragma unroll
      for (int j = 0; j < BC; ++j) vw[j] = (uint32_t)raw_buffer_load_b32(vrs, (int)(j * row_bytes + 4 * col), 0, 0);
    }
    // score of key `lane`
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 2; ++i) acc[i & 3] = dot2<DT>(kw[i], qw[i], acc[i & 3]);
    const float x = lane < nvalid ? ((acc[0] + acc[1]) + (acc[2] + acc[3])) * a.scale_log2 : -INFINITY;
    // the next tile's K, into the registers the scores have just released
    // (kept after the scores, and before the softmax, by the fences)
    __builtin_amdgcn_sched_barrier(0);
    const int k1 = k0 + BC;
    if constexpr (PS > 0) {
      load_k_small(k1 < kend ? k1 : k0);  // (past the range: this tile again, from L2)
    } else {
      int64_t off1 = 0;
      uint32_t nb1 = 0;  // past the range: an empty resource, the loads return zeros
      if (k1 < kend) {
        off1 = tile_off(k1);
        nb1 = tile_bytes(k1);
      }
      const i32x4 krs = make_rsrc((const uint16_t*)a.k + off1, nb1);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const i32x4 y = raw_buffer_load_v4(krs, (int)(lane * row_bytes + 16 * c), 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) kw[4 * c + w] = (uint32_t)y[w];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const float m_new = max2f(m, wave_max(x));
    const float m_safe = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_safe);
    const float p = fast_exp2(x - m_safe);
    l_lane = fmaf(l_lane, alpha, p);
    m = m_new;
    o0 *= alpha;
    o1 *= alpha;
    // probabilities of keys 2i, 2i+1 as one 16-bit pair, from lane 2i
    const uint32_t pp = pack2<DT>(p, __shfl_xor(p, 1));
#pragma unroll
    for (int i = 0; i < BC / 2; ++i) {
      const uint32_t pi = (uint32_t)__builtin_amdgcn_readlane((int)pp, 2 * i);
      const uint32_t lo = __builtin_amdgcn_perm(vw[2 * i + 1], vw[2 * i], 0x05040100u);  // column 2 col
      const uint32_t hi = __builtin_amdgcn_perm(vw[2 * i + 1], vw[2 * i], 0x07060302u);  // column 2 col + 1
      o0 = dot2<DT>(lo, pi, o0);
      o1 = dot2<DT>(hi, pi, o1);
    }
  }
  const float l = wave_sum(l_lane);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  if (a.n_split == 1) {
    uint16_t* o = (uint16_t*)a.o + (int64_t)row * a.o_ss + (int64_t)h * a.o_sh;
    if (lane < NCOL) *(uint32_t*)(o + 2 * lane) = pack2<DT>(o0 * inv, o1 * inv);
    if (lane == 0 && a.lse != nullptr) a.lse[(int64_t)h * a.total_q + row] = lse;
  } else {
    const int64_t prow = (int64_t)split * a.total_q + row;
    if (lane < NCOL) *(f32x2*)(a.part_o + (prow * a.H + h) * D + 2 * lane) = f32x2{o0 * inv, o1 * inv};
    if (lane == 0) a.part_lse[(int64_t)split * a.H * a.total_q + (int64_t)h * a.total_q + row] = lse;
  }
}

// Head dim 256: a key's 512-byte row is split between lanes j and j + 32
// (head-dim half `half` = lane / 32 each), so a tile holds 32 keys and a
// score is the sum of the two halves' dot products (one half-wave swap; both
// lanes then hold the same score).  The query's half sits in vector registers
// (its 128 pairs would not fit the scalar ones).  V: each 512-byte key row is
// one coalesced load of 8 bytes per lane, lane l holding columns 4l .. 4l+3.
// Otherwise as decode_kernel: head index fastest, the next tile's K in flight
// during the softmax and P V, the same outputs, and the same two addressing
// forms (PS = 0: buffer loads over a tile inside one page; PS = 4 or 5: pages
// of 16 or 32 tokens, every row through its page, keys past the range on the
// range's last row).
template <int DT, int PS>
__global__ void __launch_bounds__(256) decode_kernel_d256(FwdArgs a) {
  static_assert(PS == 0 || PS == 4 || PS == 5, "small pages of 16 or 32 tokens");
  constexpr int D = 256, BC = 32, HP = D / 4;  // HP: query / K pairs per lane half
  constexpr int NPG = PS > 0 ? BC >> PS : 1;   // pages per tile
  const int lane = threadIdx.x & 63, key_l = lane & 31, half = lane >> 5;
  DecodeItem it;
  if (!decode_item(a, it)) return;  // (no barriers below)
  const int h = it.h, split = it.split, row = it.row, kbeg = it.kbeg, kend = it.kend;

  uint32_t qv[HP];  // query pairs 64 half .. 64 half + 63
  {
    const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + ((int64_t)row * a.H + h) * D + (D / 2) * half);
#pragma unroll
    for (int c = 0; c < HP / 4; ++c) {
      const u32x4 x = qp[c];
#pragma unroll
      for (int w = 0; w < 4; ++w) qv[4 * c + w] = x[w];
    }
  }
  const uint32_t row_bytes = (uint32_t)a.H * D * 2;  // <= 2^25 (H * D <= 2^24, checked by the caller)
  auto tile_off = [&](int k0) { return decode_tile_off(a, it, D, k0); };
  auto tile_bytes = [&](int k0) -> uint32_t { return (uint32_t)(min(BC, kend - k0) - 1) * row_bytes + D * 2; };
  const uint32_t k_lane = (uint32_t)key_l * row_bytes + (D / 2) * 2 * half;  // this lane's K half-row
  float m = -INFINITY;
  float l_lane = 0.f;  // (lanes of the lower half only: each key counted once)
  float o[4] = {0.f, 0.f, 0.f, 0.f};  // head-dim columns 4 lane .. 4 lane + 3
  uint32_t kw[HP];
  auto tile_pages = [&](int k0, int64_t (&pg)[NPG]) { decode_tile_pages<PS>(a, it, k0, min(BC, kend - k0), pg); };
  auto row_slice = [&](int64_t cache_row) { return (cache_row * a.H + h) * D; };
  // small pages: this lane's K half-row of the tile at k0 (< kend)
  auto load_k_small = [&](int k0) {
    int64_t pg[NPG];
    tile_pages(k0, pg);
    const int jj = min(key_l, kend - k0 - 1);  // (keys past the range: the last row again)
    int64_t base = pg[0];
#pragma unroll
    for (int g = 1; g < NPG; ++g) base = (jj >> PS) == g ? pg[g] : base;
    const u32x4* kp = (const u32x4*)((const uint16_t*)a.k + row_slice(base + (jj & ((1 << PS) - 1))) + (D / 2) * half);
#pragma unroll
    for (int c = 0; c < HP / 4; ++c) {
      const u32x4 x = kp[c];
#pragma unroll
      for (int w = 0; w < 4; ++w) kw[4 * c + w] = x[w];
    }
  };
  if constexpr (PS > 0) {
    if (kbeg < kend) load_k_small(kbeg);
  } else if (kbeg < kend) {
    const i32x4 krs = make_rsrc((const uint16_t*)a.k + tile_off(kbeg), tile_bytes(kbeg));
#pragma unroll
    for (int c = 0; c < HP / 4; ++c) {
      const i32x4 x = raw_buffer_load_v4(krs, (int)(k_lane + 16 * c), 0, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) kw[4 * c + w] = (uint32_t)x[w];
    }
  }
  for (int k0 = kbeg; k0 < kend; k0 += BC) {
    const int nvalid = min(BC, kend - k0);
    i32x2 vw[BC];
    if constexpr (PS > 0) {
      int64_t pg[NPG];
      tile_pages(k0, pg);
#pragma unroll
      for (int j = 0; j < BC; ++j) {
        const int jj = min(j, nvalid - 1);  // (uniform)
        const i32x2* vp = (const i32x2*)((const uint16_t*)a.v + row_slice(pg[jj >> PS] + (jj & ((1 << PS) - 1))));
        vw[j] = vp[lane];
      }
    } else {
      const i32x4 vrs = make_rsrc((const uint16_t*)a.v + tile_off(k0), tile_bytes(k0));
#pragma unroll
      for (int j = 0; j < BC; ++j) vw[j] = raw_buffer_load_v2(vrs, (int)(j * row_bytes + 8 * lane), 0, 0);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < HP; ++i) acc[i & 3] = dot2<DT>(kw[i], qv[i], acc[i & 3]);
    const float part = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const float x = key_l < nvalid ? halfwave_sum(part) * a.scale_log2 : -INFINITY;
    __builtin_amdgcn_sched_barrier(0);
    const int k1 = k0 + BC;
    if constexpr (PS > 0) {
      load_k_small(k1 < kend ? k1 : k0);  // (past the range: this tile again, from L2)
    } else {
      int64_t off1 = 0;
      uint32_t nb1 = 0;  // past the range: an empty resource, the loads return zeros
      if (k1 < kend) {
        off1 = tile_off(k1);
        nb1 = tile_bytes(k1);
      }
      const i32x4 krs = make_rsrc((const uint16_t*)a.k + off1, nb1);
#pragma unroll
      for (int c = 0; c < HP / 4; ++c) {
        const i32x4 y = raw_buffer_load_v4(krs, (int)(k_lane + 16 * c), 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) kw[4 * c + w] = (uint32_t)y[w];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const float m_new = max2f(m, wave_max(x));
    const float m_safe = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_safe);
    const float p = fast_exp2(x - m_safe);
    l_lane = fmaf(l_lane, alpha, half == 0 ? p : 0.f);
    m = m_new;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] *= alpha;
    const uint32_t pp = pack2<DT>(p, __shfl_xor(p, 1));  // keys 2i, 2i+1 at lane 2i
#pragma unroll
    for (int i = 0; i < BC / 2; ++i) {
      const uint32_t pi = (uint32_t)__builtin_amdgcn_readlane((int)pp, 2 * i);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t a0 = (uint32_t)vw[2 * i][w], a1 = (uint32_t)vw[2 * i + 1][w];
        o[2 * w] = dot2<DT>(__builtin_amdgcn_perm(a1, a0, 0x05040100u), pi, o[2 * w]);
        o[2 * w + 1] = dot2<DT>(__builtin_amdgcn_perm(a1, a0, 0x07060302u), pi, o[2 * w + 1]);
      }
    }
  }
  const float l = wave_sum(l_lane);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  if (a.n_split == 1) {
    uint16_t* op = (uint16_t*)a.o + (int64_t)row * a.o_ss + (int64_t)h * a.o_sh;
    *(u32x2*)(op + 4 * lane) = u32x2{pack2<DT>(o[0] * inv, o[1] * inv), pack2<DT>(o[2] * inv, o[3] * inv)};
    if (lane == 0 && a.lse != nullptr) a.lse[(int64_t)h * a.total_q + row] = lse;
  } else {
    const int64_t prow = (int64_t)split * a.total_q + row;
    *(f32x4*)(a.part_o + (prow * a.H + h) * D + 4 * lane) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    if (lane == 0) a.part_lse[(int64_t)split * a.H * a.total_q + (int64_t)h * a.total_q + row] = lse;
  }
}

hipError_t launch_decode(const FwdArgs& a, int D, int dtype, hipStream_t s) {
  const int64_t items = (int64_t)a.B * a.H * a.n_split;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  // small pages (a paged cache with pages of 16 or 32 tokens)
  const int ps = a.block_table != nullptr && a.page_shift < 6 ? a.page_shift : 0;
  if (ps != 0 && ps != 4 && ps != 5) return hipErrorNotSupported;
  auto go = [&](auto k) { hipLaunchKernelGGL(k, grid, block, 0, s, a); };
  if (D == 64) {
    if (dtype == kBF16) ps == 0 ? go(decode_kernel<kBF16, 64, 0>) : ps == 4 ? go(decode_kernel<kBF16, 64, 4>) : go(decode_kernel<kBF16, 64, 5>);
    else ps == 0 ? go(decode_kernel<kFP16, 64, 0>) : ps == 4 ? go(decode_kernel<kFP16, 64, 4>) : go(decode_kernel<kFP16, 64, 5>);
  } else if (D == 128) {
    if (dtype == kBF16) ps == 0 ? go(decode_kernel<kBF16, 128, 0>) : ps == 4 ? go(decode_kernel<kBF16, 128, 4>) : go(decode_kernel<kBF16, 128, 5>);
    else ps == 0 ? go(decode_kernel<kFP16, 128, 0>) : ps == 4 ? go(decode_kernel<kFP16, 128, 4>) : go(decode_kernel<kFP16, 128, 5>);
  } else if (D == 256) {
    if (dtype == kBF16) ps == 0 ? go(decode_kernel_d256<kBF16, 0>) : ps == 4 ? go(decode_kernel_d256<kBF16, 4>) : go(decode_kernel_d256<kBF16, 5>);
    else ps == 0 ? go(decode_kernel_d256<kFP16, 0>) : ps == 4 ? go(decode_kernel_d256<kFP16, 4>) : go(decode_kernel_d256<kFP16, 5>);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace attn
