// Fused attention forward, 16-bit inputs, ping-pong schedule (head_dim 64/128).
//
// The "Fused attention kernel" page (Variants: warp-specialised forward pass,
// pingpong schedule) describes two consumer groups whose matrix multiplies and
// softmax are made to alternate by barriers, so that one group's matrix work
// runs while the other computes its softmax.  This is that schedule on CDNA4:
//
//  * a workgroup has 8 waves = 256 query rows (32 per wave); waves w and w+4
//    run on the same SIMD, and form group A (waves 0-3) and group B (4-7);
//  * the work of one wave on key tile t is split into an MFMA phase
//    (O += P(t-1) V(t-1), then S(t) = K(t) Q^T) and a vector phase (the online
//    softmax of S(t), producing P(t) in registers);
//  * the workgroup advances in steps separated by s_barrier; at step s group A
//    runs phase s and group B runs phase s-1, so on every SIMD one wave feeds
//    the matrix core while the other runs exponentials;
//  * K and V tiles sit in separate two-stage LDS rings: the copies of K(t+1)
//    and V(t) are issued at step 2t and waited for at the end of step 2t+1;
//  * everything else (transposed scores, V^T through ds_read_b64_tr_b16,
//    exp2 with folded scale, lazy max, buffer-LDS copies with zero-fill past
//    Lk) is as in fwd16.hpp.
#pragma once

#include "fwd16.hpp"

namespace attn {

template <int D>
struct PPCfg {
  static constexpr int NW = 8;                     // waves per workgroup
  static constexpr int BR = 32 * NW;               // query rows per workgroup
  static constexpr int BC = 64;                    // keys per tile
  static constexpr int CPR = D / 8;
  // LDS row pitches in 16-byte slots: one pad slot for K (16 rows read by 16
  // lanes with ds_read_b128 start in distinct bank groups); for V a pitch that
  // puts the 4 rows of a transposing read in distinct 32-byte bank groups
  static constexpr int KSLOTS = CPR + 1;
  static constexpr int VSLOTS = D == 64 ? 10 : (D == 128 ? 19 : 34);
  static constexpr int KP = 8 * KSLOTS;
  static constexpr int VP = 8 * VSLOTS;
  static constexpr int K_ELEMS = BC * KP;
  static constexpr int V_ELEMS = BC * VP;
  static constexpr int KI_W = (KSLOTS + NW - 1) / NW;
  static constexpr int VI_W = (VSLOTS + NW - 1) / NW;
};

template <int D, int DT, bool CAUSAL, int MODE>
__global__ void __launch_bounds__(512, 2) fwd16pp_kernel(FwdArgs a) {
  using C = PPCfg<D>;
  constexpr int NW = C::NW, BR = C::BR, BC = C::BC, KP = C::KP, VP = C::VP, CPR = C::CPR;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::K_ELEMS + 2 * C::V_ELEMS];
  uint16_t* const ks_base = smem;
  uint16_t* const vs_base = smem + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B (one step behind)
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // ---- work item: (b, h, query block of 256 rows) ---------------------------
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / a.n_qblk;
  int qblk = t - bh * a.n_qblk;
  if (CAUSAL) qblk = a.n_qblk - 1 - qblk;
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
    const int last = min(qs + BR, Lq) - 1 + (Lk - Lq);
    n_kv = last < 0 ? 0 : min(n_kv, last / BC + 1);
  }
  const int qw = qs + 32 * wave;
  const int qi = qw + l32;
  const bool wave_active = qw < Lq;
  const int diag = Lk - Lq;
  const int wave_last_key = CAUSAL ? min(qw + 31, Lq - 1) + diag : Lk - 1;
  auto wave_needs = [&](int j) { return wave_active && (!CAUSAL || j * BC <= wave_last_key); };

  u32x4 qf[D / 16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + qoff + (int64_t)qi * a.q_ss + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = qi < Lq ? *(const u32x4*)(qp + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // ---- tile copies (slots dealt round-robin to the 8 waves) -----------------
  const uint16_t* const kg = (const uint16_t*)a.k + koff;
  const uint16_t* const vg = (const uint16_t*)a.v + voff;
  auto k_slot = [&](int ii, int& key_local, int& chunk) {
    const int s = 64 * (wave + NW * ii) + lane;
    const int r = s / C::KSLOTS;
    chunk = s - r * C::KSLOTS;
    key_local = (r & ~31) | swz23(r & 31);
  };
  auto v_slot = [&](int ii, int& key_local, int& chunk) {
    const int s = 64 * (wave + NW * ii) + lane;
    key_local = s / C::VSLOTS;
    chunk = s - key_local * C::VSLOTS;
  };
  constexpr uint32_t kOutOfRange = 0x7ffffff0u;
  uint32_t k_boff[C::KI_W], v_boff[C::VI_W];
#pragma unroll
  for (int ii = 0; ii < C::KI_W; ++ii) {
    int kl, ch;
    k_slot(ii, kl, ch);
    k_boff[ii] = ch < CPR ? 2u * (uint32_t)(kl * (int)a.k_ss + ch * 8) : kOutOfRange;
  }
#pragma unroll
  for (int ii = 0; ii < C::VI_W; ++ii) {
    int kl, ch;
    v_slot(ii, kl, ch);
    v_boff[ii] = ch < CPR ? 2u * (uint32_t)(kl * (int)a.v_ss + ch * 8) : kOutOfRange;
  }
  auto row_of = [&](int key) -> int64_t {
    if constexpr (MODE == kPaged) {
      const int page = a.block_table[(int64_t)b * a.max_pages + (key >> a.page_shift)];
      return (((int64_t)page << a.page_shift) | (key & ((1 << a.page_shift) - 1)));
    } else {
      return key;
    }
  };
  auto dma_k = [&](int key0, int kbuf) {
    uint16_t* kb = ks_base + kbuf * C::K_ELEMS;
    if constexpr (MODE != kPaged) {
      const uint64_t kn = 2ull * (uint64_t)(Lk - key0) * (uint64_t)a.k_ss;
      const i32x4 kr = make_rsrc(kg + (int64_t)key0 * a.k_ss, (uint32_t)min(kn, (uint64_t)0x7fff0000u));
#pragma unroll
      for (int ii = 0; ii < C::KI_W; ++ii)
        if (wave + NW * ii < C::KSLOTS) dma16_buf(kr, k_boff[ii], kb + (wave + NW * ii) * 512);
    } else {
#pragma unroll
      for (int ii = 0; ii < C::KI_W; ++ii) {
        const int i = wave + NW * ii;
        if (i < C::KSLOTS) {
          int kl, ch;
          k_slot(ii, kl, ch);
          if (ch < CPR) dma16(kg + row_of(min(key0 + kl, Lk - 1)) * a.k_ss + ch * 8, kb + i * 512);
        }
      }
    }
  };
  auto dma_v = [&](int key0, int vbuf) {
    uint16_t* vb = vs_base + vbuf * C::V_ELEMS;
    if constexpr (MODE != kPaged) {
      const uint64_t vn = 2ull * (uint64_t)(Lk - key0) * (uint64_t)a.v_ss;
      const i32x4 vr = make_rsrc(vg + (int64_t)key0 * a.v_ss, (uint32_t)min(vn, (uint64_t)0x7fff0000u));
#pragma unroll
      for (int ii = 0; ii < C::VI_W; ++ii)
        if (wave + NW * ii < C::VSLOTS) dma16_buf(vr, v_boff[ii], vb + (wave + NW * ii) * 512);
    } else {
#pragma unroll
      for (int ii = 0; ii < C::VI_W; ++ii) {
        const int i = wave + NW * ii;
        if (i < C::VSLOTS) {
          int kl, ch;
          v_slot(ii, kl, ch);
          if (ch < CPR) dma16(vg + row_of(min(key0 + kl, Lk - 1)) * a.v_ss + ch * 8, vb + i * 512);
        }
      }
    }
  };

  const int vg_grp = lane >> 4, vg_j = lane & 15;
  const int vtr_off = (8 * (vg_grp >> 1) + (vg_j >> 2)) * VP + 16 * (vg_grp & 1) +
                      4 * (((vg_j & 1) << 1) | ((vg_j >> 1) & 1));

  // ---- per-wave state ----------------------------------------------------------
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;
  const f32x16 zero16 = {};
  f32x16 s[BC / 32];   // scores of the tile between its MFMA phase and its softmax phase
  u32x4 pk[BC / 16];   // packed probabilities between the softmax phase and the next MFMA phase

  // MFMA phase of tile j: S(j) = K(j) Q^T, then O += P(j-1) V(j-1)
  auto mfma_phase = [&](int j) {
    const bool do_pv = j >= 1 && wave_needs(j - 1);
    const bool do_s = j < n_kv && wave_needs(j);
    __builtin_amdgcn_s_setprio(1);
    if (do_s) {
      // K operands in two batches of D/32 k-steps (both 32-key halves each), so
      // at most 8 operands (32 VGPRs) are in flight
      constexpr int NKK = D / 16, HALF = NKK / 2;
      const uint16_t* ks = ks_base + (j & 1) * C::K_ELEMS + l32 * KP + 8 * hh;
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        u32x4 kop[BC / 32][HALF];
#pragma unroll
        for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
          for (int k2 = 0; k2 < HALF; ++k2)
            kop[tt][k2] = *(const u32x4*)(ks + tt * 32 * KP + 16 * (part * HALF + k2));
#pragma unroll
        for (int k2 = 0; k2 < HALF; ++k2) {
          const int kk = part * HALF + k2;
#pragma unroll
          for (int tt = 0; tt < BC / 32; ++tt)
            s[tt] = mfma32<DT>(kop[tt][k2], qf[kk], kk == 0 ? zero16 : s[tt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the V operands are read only after the K operands are dead
    if (do_pv) {
      const uint16_t* vs = vs_base + ((j - 1) & 1) * C::V_ELEMS + vtr_off;
#pragma unroll
      for (int c = 0; c < BC / 16; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const uint16_t* vp = vs + 16 * c * VP + 32 * dt;
          const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * VP);
          oacc[dt] = mfma32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[c], oacc[dt]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // vector phase of tile j: mask, running max (lazy), exponentials, row sum, pack P(j)
  auto softmax_phase = [&](int j) {
    if (!(j < n_kv && wave_needs(j))) return;
    const int key0 = j * BC;
    const bool need_mask = (key0 + BC > Lk) || (CAUSAL && key0 + BC - 1 > qw + diag);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * tt + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key >= Lk || (CAUSAL && key > qi + diag)) s[tt][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int tt = 0; tt < BC / 32; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tt][r]);
    const float mxs = halfwave_max(mx) * c2;
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = m_new;
    }
    const float nb = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
      const int tt = c >> 1, r0p = 8 * (c & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(s[tt][r0p + e], c2, nb));
        psum += p[e];
      }
      pk[c] = u32x4{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]), pack2<DT>(p[6], p[7])};
    }
    l_run += psum;
  };

  // ---- the stepped loop ----------------------------------------------------------
  // Steps st = 0 .. 2n+1, each closed by a barrier.  Group A runs phase st
  // (even: MFMA phase of tile st/2, odd: softmax of tile st/2), group B runs
  // phase st-1.  At even steps 2t every wave issues its share of the copies of
  // K(t+1) and V(t); at odd steps it waits for them before the barrier.  The
  // two groups get their own loops so that each sees a fixed phase order.
  auto copies = [&](int tj) {
    if (tj + 1 < n_kv) dma_k((tj + 1) * BC, (tj + 1) & 1);
    if (tj < n_kv) dma_v(tj * BC, tj & 1);
  };
  if (n_kv > 0) dma_k(0, 0);
  wait_vmem();
  __syncthreads();
  if (grp == 0) {
    for (int tj = 0; tj <= n_kv; ++tj) {
      copies(tj);            // step 2tj
      mfma_phase(tj);
      __syncthreads();
      softmax_phase(tj);     // step 2tj+1
      wait_vmem();
      __syncthreads();
    }
  } else {
    copies(0);               // step 0: nothing to compute yet
    __syncthreads();
    for (int tj = 0; tj <= n_kv; ++tj) {
      mfma_phase(tj);        // step 2tj+1
      wait_vmem();
      __syncthreads();
      if (tj < n_kv) {
        copies(tj + 1);      // step 2tj+2
        softmax_phase(tj);
        __syncthreads();
      }
    }
  }

  // ---- epilogue --------------------------------------------------------------------
  const float l_tot = halfwave_sum(l_run);
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
hipError_t launch_fwd16pp(FwdArgs a, hipStream_t s) {
  a.n_qblk = (a.Sq + PPCfg<D>::BR - 1) / PPCfg<D>::BR;
  const int n = a.B * a.H * a.n_qblk;
  hipLaunchKernelGGL((fwd16pp_kernel<D, DT, CAUSAL, MODE>), dim3(n), dim3(512), 0, s, a);
  return hipGetLastError();
}

#define ATTN_INSTANTIATE_FWD16PP(D)                                                            \
  template hipError_t launch_fwd16pp<D, kBF16, false, kDense>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kBF16, true, kDense>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16pp<D, kFP16, false, kDense>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kFP16, true, kDense>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16pp<D, kBF16, false, kVarlen>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16pp<D, kBF16, true, kVarlen>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kFP16, false, kVarlen>(FwdArgs, hipStream_t); \
  template hipError_t launch_fwd16pp<D, kFP16, true, kVarlen>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kBF16, false, kPaged>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kBF16, true, kPaged>(FwdArgs, hipStream_t);   \
  template hipError_t launch_fwd16pp<D, kFP16, false, kPaged>(FwdArgs, hipStream_t);  \
  template hipError_t launch_fwd16pp<D, kFP16, true, kPaged>(FwdArgs, hipStream_t);

}  // namespace attn
