// Fused attention forward, 16-bit inputs (bf16 / fp16), for gfx950.
//
// What is computed follows the "Fused attention kernel" page (Implementation
// sketch): one query block stays on chip, key/value blocks stream past it, a
// running row max m and row sum l are kept, the old state is rescaled by
// alpha = exp(m_old - m_new), every key block (including a partial last one)
// is scored, and o / l and lse = m + log l are formed once at the end.
//
// How it maps to CDNA4:
//  * one workgroup = 4 waves = 128 query rows; each wave owns 32 rows and keeps
//    its Q fragments in registers for the whole key loop;
//  * K and V tiles of 64 keys go through a two-stage LDS ring: the global loads
//    of tile j+1 are issued before the matrix work on tile j, and land in the
//    other LDS stage after it (one barrier per tile);
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16, so
//    every lane owns one query column: the row max and row sum are in-lane
//    reductions plus one exchange between the two half-waves;
//  * V is written to LDS transposed (head_dim-major) so that the second GEMM,
//    O^T = V^T P^T, reads its operand with one 16-byte LDS load and takes P^T
//    straight from the score accumulators (no LDS round trip for P);
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA;
//  * rows past the sequence end and keys past Lk are zero-filled in LDS and
//    masked, so whatever memory lies there never reaches the result.
#pragma once

#include "common.hpp"

namespace attn {

template <int D>
struct Fwd16Cfg {
  static constexpr int BR = 128;                  // query rows per workgroup
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int KSTR = D + 8;              // LDS row pitch of K tiles (elements)
  static constexpr int VSTR = BC + 8;             // LDS row pitch of transposed V tiles
  static constexpr int K_ELEMS = BC * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int NK = BC * D / 8 / 256;     // 16-byte K chunks per thread
  static constexpr int NVB = (BC / 4) * (D / 8);  // 4-key x 8-dim V blocks per tile
  static constexpr int NV = (NVB + 255) / 256;    // V blocks per thread
  static constexpr int WAVES_PER_EU = D <= 128 ? 2 : 1;
  static constexpr int LDS_BYTES = 2 * (2 * K_ELEMS + 2 * V_ELEMS);
};

template <int D, int DT, bool CAUSAL, int MODE>
__global__ void __launch_bounds__(256, Fwd16Cfg<D>::WAVES_PER_EU) fwd16_kernel(FwdArgs a) {
  using C = Fwd16Cfg<D>;
  constexpr int BR = C::BR, BC = C::BC, KSTR = C::KSTR, VSTR = C::VSTR;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::K_ELEMS + 2 * C::V_ELEMS];
  uint16_t* const ks_base = smem;
  uint16_t* const vt_base = smem + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // ---- work item: (b, h, query block) -------------------------------------
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / a.n_qblk;
  int qblk = t - bh * a.n_qblk;
  if (CAUSAL) qblk = a.n_qblk - 1 - qblk;  // longest key ranges first
  const int b = bh / a.H, h = bh - b * a.H;

  int Lq, Lk;
  int64_t qoff, ooff, koff, voff, lse_base;
  if constexpr (MODE == kDense) {
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

  // ---- K/V tile staging ----------------------------------------------------
  auto row_off = [&](int key, int64_t base, int64_t ss) -> int64_t {
    if constexpr (MODE == kPaged) {
      const int page = a.block_table[(int64_t)b * a.max_pages + (key >> a.page_shift)];
      const int64_t phys = ((int64_t)page << a.page_shift) | (key & ((1 << a.page_shift) - 1));
      return base + phys * ss;
    } else {
      return base + (int64_t)key * ss;
    }
  };

  u32x4 kreg[C::NK];
  u32x4 vreg[C::NV][4];
  const uint16_t* const kg = (const uint16_t*)a.k;
  const uint16_t* const vg = (const uint16_t*)a.v;

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 8), col = c % (D / 8);
      const int key = key0 + row;
      kreg[i] = key < Lk ? *(const u32x4*)(kg + row_off(key, koff, a.k_ss) + col * 8)
                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int blk = tid + 256 * i;
      if (C::NVB % 256 == 0 || blk < C::NVB) {
        const int kgp = blk % (BC / 4), dc = blk / (BC / 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int key = key0 + 4 * kgp + u;
          vreg[i][u] = key < Lk ? *(const u32x4*)(vg + row_off(key, voff, a.v_ss) + dc * 8)
                                : u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = ks_base + buf * C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 8), col = c % (D / 8);
      const int lrow = (row & ~31) | swz23(row & 31);
      *(u32x4*)(ks + lrow * KSTR + col * 8) = kreg[i];
    }
    uint16_t* vt = vt_base + buf * C::V_ELEMS;
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int blk = tid + 256 * i;
      if (C::NVB % 256 == 0 || blk < C::NVB) {
        const int kgp = blk % (BC / 4), dc = blk / (BC / 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * dc + e;
          const int lrow = (d & ~31) | swz23(d & 31);
          const int w = e >> 1, sh = (e & 1) * 16;
          const uint32_t x0 = (vreg[i][0][w] >> sh) & 0xffffu;
          const uint32_t x1 = (vreg[i][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (vreg[i][2][w] >> sh) & 0xffffu;
          const uint32_t x3 = (vreg[i][3][w] >> sh) & 0xffffu;
          *(u32x2*)(vt + lrow * VSTR + 4 * kgp) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
        }
      }
    }
  };

  // ---- running state ---------------------------------------------------------
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*s
  float l_run = 0.f;        // this half-wave's share of the running sum
  const float c2 = a.scale_log2;

  auto compute = [&](int key0, int buf) {
    if (!wave_active) return;
    if (CAUSAL && key0 > wave_last_key) return;  // tile fully masked for this wave
    const uint16_t* ks = ks_base + buf * C::K_ELEMS + l32 * KSTR + 8 * hh;
    f32x16 s[BC / 32];
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[tt][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        s[tt] = mfma32<DT>(*(const u32x4*)(ks + tt * 32 * KSTR + 16 * kk), qf[kk], s[tt]);
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
    float mx = s[0][0];
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    const float nb = -m_use;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[tt][r], c2, nb));
        s[tt][r] = p;
        psum += p;
      }
    l_run = alpha * l_run + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    u32x4 pk[BC / 16];
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int tt = c >> 1, r0 = 8 * (c & 1);
      pk[c] = u32x4{pack2<DT>(s[tt][r0 + 0], s[tt][r0 + 1]), pack2<DT>(s[tt][r0 + 2], s[tt][r0 + 3]),
                    pack2<DT>(s[tt][r0 + 4], s[tt][r0 + 5]), pack2<DT>(s[tt][r0 + 6], s[tt][r0 + 7])};
    }
    const uint16_t* vt = vt_base + buf * C::V_ELEMS + l32 * VSTR + 8 * hh;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        oacc[dt] = mfma32<DT>(*(const u32x4*)(vt + dt * 32 * VSTR + 16 * c), pk[c], oacc[dt]);
  };

  // ---- key loop: two-stage LDS ring ------------------------------------------
  if (n_kv > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int j = 0; j < n_kv; ++j) {
      const int buf = j & 1;
      if (j + 1 < n_kv) load_tile((j + 1) * BC);
      compute(j * BC, buf);
      if (j + 1 < n_kv) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: o / l, lse = ln2 * (m + log2 l) -----------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)a.o + ooff + (int64_t)qi * a.o_ss + 8 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0 = 8 * half;
        const f32x16& o = oacc[dt];
        *(u32x4*)(op + 32 * dt + 16 * half) =
            u32x4{pack2<DT>(o[r0 + 0] * inv, o[r0 + 1] * inv), pack2<DT>(o[r0 + 2] * inv, o[r0 + 3] * inv),
                  pack2<DT>(o[r0 + 4] * inv, o[r0 + 5] * inv), pack2<DT>(o[r0 + 6] * inv, o[r0 + 7] * inv)};
      }
    if (hh == 0 && a.lse != nullptr)
      a.lse[lse_base + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int DT, bool CAUSAL, int MODE>
hipError_t launch_fwd16(const FwdArgs& a, hipStream_t s) {
  const int n = a.B * a.H * a.n_qblk;
  hipLaunchKernelGGL((fwd16_kernel<D, DT, CAUSAL, MODE>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define ATTN_INSTANTIATE_FWD16(D)                                          \
  template hipError_t launch_fwd16<D, kBF16, false, kDense>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, true, kDense>(const FwdArgs&, hipStream_t);   \
  template hipError_t launch_fwd16<D, kFP16, false, kDense>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, true, kDense>(const FwdArgs&, hipStream_t);   \
  template hipError_t launch_fwd16<D, kBF16, false, kVarlen>(const FwdArgs&, hipStream_t); \
  template hipError_t launch_fwd16<D, kBF16, true, kVarlen>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, false, kVarlen>(const FwdArgs&, hipStream_t); \
  template hipError_t launch_fwd16<D, kFP16, true, kVarlen>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, false, kPaged>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kBF16, true, kPaged>(const FwdArgs&, hipStream_t);   \
  template hipError_t launch_fwd16<D, kFP16, false, kPaged>(const FwdArgs&, hipStream_t);  \
  template hipError_t launch_fwd16<D, kFP16, true, kPaged>(const FwdArgs&, hipStream_t);

}  // namespace attn
