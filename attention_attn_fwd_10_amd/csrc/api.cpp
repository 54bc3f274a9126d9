// C ABI of the attention forward library: host-side argument validation and
// dispatch to the kernel instantiations.  Nothing here touches the device
// before every argument has been checked, so an error return means that no
// work was queued and nothing was written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "args.hpp"
#include "bwd.hpp"

namespace attn {
template <int D, int DT, bool CAUSAL, int MODE>
hipError_t launch_fwd16(FwdArgs a, hipStream_t s);
hipError_t launch_fp8_quantize(const QuantArgs& a, int D, hipStream_t s);
hipError_t launch_fp8_quantize_pow2(const QuantArgs& a, int D, hipStream_t s);
hipError_t launch_splitkv_merge(const MergeArgs& a, int D, int dtype, hipStream_t s);
hipError_t launch_tail_merge(const TailMergeArgs& a, int D, int dtype, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8Args& a, int D, bool causal, hipStream_t s);
hipError_t launch_fwd_fp8_pow2(const Fp8Args& a, int D, bool causal, hipStream_t s);
hipError_t launch_decode(const FwdArgs& a, int D, int dtype, hipStream_t s);
hipError_t launch_int8_quantize(const QuantArgs& a, int D, hipStream_t s);
hipError_t launch_fwd_int8(const Fp8Args& a, int D, bool causal, hipStream_t s);
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(float** out);
}  // namespace attn

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

attn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b * c > INT32_MAX for non-negative factors below 2^62, without overflow
// (a grid size: workgroups per launch)
bool grid_too_large(int64_t a, int64_t b, int64_t c) { return (__int128)a * b * c > INT32_MAX; }

attn_status_t check_strides(const char* name, const int64_t* s) {
  if (s == nullptr) return fail(ATTN_ERR_INVALID, "%s_strides is NULL", name);
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(ATTN_ERR_INVALID, "%s_strides[%d] = %lld is negative", name, i, (long long)s[i]);
    if (s[i] % 8 != 0)
      return fail(ATTN_ERR_INVALID, "%s_strides[%d] = %lld is not a multiple of 8 elements", name, i,
                  (long long)s[i]);
  }
  return ATTN_OK;
}

attn_status_t check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_ERR_INVALID, "softmax_scale must be finite and > 0 (got %g)", (double)scale);
  return ATTN_OK;
}

attn_status_t check_head_dim(int D) {
  if (D <= 0) return fail(ATTN_ERR_INVALID, "head_dim %d must be positive", D);
  if (D != 64 && D != 128 && D != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d is not one of 64, 128, 256", D);
  return ATTN_OK;
}

template <int D, int DT, bool CAUSAL, int MODE>
hipError_t launch_one(const attn::FwdArgs& a, hipStream_t s) {
  return attn::launch_fwd16<D, DT, CAUSAL, MODE>(a, s);
}

template <int D, int DT>
hipError_t dispatch_causal_mode(const attn::FwdArgs& a, bool causal, int mode, hipStream_t s) {
  using namespace attn;
  if constexpr (D <= 128) {
    if (mode == kDenseBias)
      return causal ? launch_one<D, DT, true, kDenseBias>(a, s) : launch_one<D, DT, false, kDenseBias>(a, s);
  }
  if constexpr (D == 128) {
    if (mode == kDenseWide && !causal) return launch_one<D, DT, false, kDenseWide>(a, s);
  }
  if (mode == kDense)
    return causal ? launch_one<D, DT, true, kDense>(a, s) : launch_one<D, DT, false, kDense>(a, s);
  if (mode == kVarlen)
    return causal ? launch_one<D, DT, true, kVarlen>(a, s) : launch_one<D, DT, false, kVarlen>(a, s);
  return causal ? launch_one<D, DT, true, kPaged>(a, s) : launch_one<D, DT, false, kPaged>(a, s);
}

hipError_t dispatch_fwd16(const attn::FwdArgs& a, int D, int dtype, bool causal, int mode, hipStream_t s) {
  if (dtype == ATTN_BF16) {
    if (D == 64) return dispatch_causal_mode<64, attn::kBF16>(a, causal, mode, s);
    if (D == 128) return dispatch_causal_mode<128, attn::kBF16>(a, causal, mode, s);
    return dispatch_causal_mode<256, attn::kBF16>(a, causal, mode, s);
  }
  if (D == 64) return dispatch_causal_mode<64, attn::kFP16>(a, causal, mode, s);
  if (D == 128) return dispatch_causal_mode<128, attn::kFP16>(a, causal, mode, s);
  return dispatch_causal_mode<256, attn::kFP16>(a, causal, mode, s);
}

constexpr int kBR = 128;  // query rows per workgroup of every forward kernel
// K/V tiles are read through 32-bit buffer offsets: 64 rows of a tile must fit in 2^31 bytes
constexpr int64_t kMaxSeqStride = int64_t(1) << 24;
constexpr int kMaxSplits = 256;  // key splits per sequence in attn_fwd_splitkv
// Fewest work items (waves) of the streaming decode kernel: with fewer, its
// one tile in flight per wave leaves HBM idle and the tiled kernel is faster
// (measured: 144 and 336 waves ran at 0.5x and 0.85x of it, 512 at 1.1x).
constexpr int64_t kDecodeMinWaves = 512;

// Compute units of the current device (0 if the query fails), looked up once
// per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Schedule of the dense forward.  The non-causal forward at head dim 128 with
// at least kWideMinKeys keys runs in 256-row workgroups (attn::kDenseWide,
// one per CU, each K/V tile copied once for 8 waves) when its grid fills
// whole rounds of the CUs; when the last round is at most half full and a
// workspace is at hand, the work items of that round run as key ranges
// spread over the whole chip (at most kMaxTailSplits per item), and a merge
// combines their partial results.  Anything else runs the 128-row workgroups
// of attn::kDense.  (Measured: the wide layout is 4-5 % faster at head dim 128
// from 4096 keys on; below 4096 keys it is at best even (2048 keys) and down
// to 6 % slower at 512, where the fixed cost of a work item weighs more and
// one workgroup per CU cannot hide it behind another's key loop.  Head dim 64
// runs 3-4 of the 128-row workgroups per CU instead, which beat it.)
constexpr int kMaxTailSplits = 8;
constexpr int kWideMinKeys = 4096;
struct DensePlan {
  int mode = attn::kDense;
  int n_qblk = 0, tail_start = 0, n_split = 1, split_tiles = 0;
  size_t ws_bytes = 0;  // partial outputs and logsumexps of the split tail
};
DensePlan plan_dense(int B, int H, int Sq, int Sk, int D, bool causal, int cus, bool have_workspace) {
  DensePlan p;
  if (causal || D != 128 || cus <= 0 || Sk < kWideMinKeys) return p;
  const int64_t nq = ((int64_t)Sq + attn::kWideRows - 1) / attn::kWideRows;
  const int64_t n = (int64_t)B * H * nq;
  if (n < cus || n > INT32_MAX - (int64_t)cus * kMaxTailSplits) return p;
  const int64_t r = n % cus;
  DensePlan w;
  w.mode = attn::kDenseWide;
  w.n_qblk = (int)nq;
  w.tail_start = (int)n;
  if (r == 0) return w;
  const int tiles = (int)(((int64_t)Sk + 63) / 64);
  if (!have_workspace || 2 * r > cus || tiles < 4) return p;
  int splits = (int)std::min<int64_t>(kMaxTailSplits, cus / r);
  w.split_tiles = (tiles + splits - 1) / splits;
  splits = (tiles + w.split_tiles - 1) / w.split_tiles;  // no empty key range
  if (splits < 2) return p;
  w.tail_start = (int)(n - r);
  w.n_split = splits;
  w.ws_bytes = (size_t)splits * (size_t)r * attn::kWideRows * (size_t)(D + 1) * sizeof(float);
  return w;
}

// Launch of a validated dense forward (attn_fwd, attn_fwd_ws) under its plan.
attn_status_t dense_launch(attn::FwdArgs a, int D, int dtype, bool causal, void* workspace, size_t workspace_bytes,
                           hipStream_t s) {
  const DensePlan p = plan_dense(a.B, a.H, a.Sq, a.Sk, D, causal, device_cus(), workspace != nullptr);
  if (p.ws_bytes > workspace_bytes)
    return fail(ATTN_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu bytes this problem needs",
                workspace_bytes, p.ws_bytes);
  if (p.mode == attn::kDense) return hip_status(dispatch_fwd16(a, D, dtype, causal, attn::kDense, s), "attn_fwd launch");
  a.n_qblk = p.n_qblk;
  a.tail_start = p.tail_start;
  a.n_split = p.n_split;
  a.split_tiles = p.split_tiles;
  const int n_tail = (int)((int64_t)a.B * a.H * p.n_qblk - p.tail_start);
  if (p.n_split > 1) {
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (size_t)p.n_split * (size_t)n_tail * attn::kWideRows * (size_t)D;
  }
  hipError_t e = dispatch_fwd16(a, D, dtype, causal, attn::kDenseWide, s);
  if (e == hipSuccess && p.n_split > 1) {
    attn::TailMergeArgs m{};
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.o = a.o;
    m.lse = a.lse;
    m.o_sb = a.o_sb; m.o_ss = a.o_ss; m.o_sh = a.o_sh;
    m.H = a.H;
    m.Sq = a.Sq;
    m.n_qblk = p.n_qblk;
    m.tail_start = p.tail_start;
    m.n_tail = n_tail;
    m.n_split = p.n_split;
    e = attn::launch_tail_merge(m, D, dtype == ATTN_BF16 ? attn::kBF16 : attn::kFP16, s);
  }
  return hip_status(e, "attn_fwd launch");
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_STATUS_UNKNOWN";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Validation and argument set-up of the dense forward (attn_fwd, attn_fwd_bias).
attn_status_t dense_args(int dtype, const void* q, const int64_t q_strides[3], const void* k,
                         const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                         const int64_t o_strides[3], float* lse, int B, int H, int Sq, int Sk, int D,
                         float softmax_scale, int causal, attn::FwdArgs* a, bool* empty) {
  attn_status_t st;
  *empty = false;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return fail(ATTN_ERR_INVALID, "dtype %d is not bf16/fp16", dtype);
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(ATTN_ERR_INVALID, "negative size (B=%d H=%d Sq=%d Sk=%d)", B, H, Sq, Sk);
  if ((st = check_head_dim(D)) != ATTN_OK) return st;
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  if ((st = check_strides("q", q_strides)) != ATTN_OK) return st;
  if ((st = check_strides("k", k_strides)) != ATTN_OK) return st;
  if ((st = check_strides("v", v_strides)) != ATTN_OK) return st;
  if ((st = check_strides("o", o_strides)) != ATTN_OK) return st;
  if (B == 0 || H == 0 || Sq == 0) {
    *empty = true;
    return ok();
  }
  if (q == nullptr || o == nullptr) return fail(ATTN_ERR_INVALID, "q or o is NULL");
  if (Sk > 0 && (k == nullptr || v == nullptr)) return fail(ATTN_ERR_INVALID, "k or v is NULL");
  if (Sk > 1 && (k_strides[1] < D || v_strides[1] < D))
    return fail(ATTN_ERR_INVALID, "k/v sequence strides must be at least head_dim (rows may not overlap)");
  if (k_strides[1] > kMaxSeqStride || v_strides[1] > kMaxSeqStride)
    return fail(ATTN_ERR_UNSUPPORTED, "k/v sequence strides above 2^24 elements are not supported");
  if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v) || !aligned16(lse))
    return fail(ATTN_ERR_INVALID, "q, k, v, o and lse must be 16-byte aligned");
  const int64_t n_qblk = ((int64_t)Sq + kBR - 1) / kBR;
  if (grid_too_large(B, H, n_qblk)) return fail(ATTN_ERR_INVALID, "problem too large for one launch");

  *a = attn::FwdArgs{};
  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  a->q_sb = q_strides[0]; a->q_ss = q_strides[1]; a->q_sh = q_strides[2];
  a->k_sb = k_strides[0]; a->k_ss = k_strides[1]; a->k_sh = k_strides[2];
  a->v_sb = v_strides[0]; a->v_ss = v_strides[1]; a->v_sh = v_strides[2];
  a->o_sb = o_strides[0]; a->o_ss = o_strides[1]; a->o_sh = o_strides[2];
  a->B = B; a->H = H; a->Sq = Sq; a->Sk = Sk;
  a->scale_log2 = softmax_scale * attn::kLog2e;
  a->n_qblk = (int)n_qblk;
  a->n_split = 1;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(int dtype, const void* q, const int64_t q_strides[3], const void* k,
                       const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                       const int64_t o_strides[3], float* lse, int B, int H, int Sq, int Sk, int D,
                       float softmax_scale, int causal, void* stream) {
  return attn_fwd_ws(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, Sq, Sk, D,
                     softmax_scale, causal, nullptr, 0, stream);
}

size_t attn_fwd_workspace_bytes(int dtype, int B, int H, int Sq, int Sk, int D, int causal) {
  if ((dtype != ATTN_BF16 && dtype != ATTN_FP16) || B <= 0 || H <= 0 || Sq <= 0 || Sk < 0) return 0;
  if ((D != 64 && D != 128 && D != 256) || (causal != 0 && causal != 1)) return 0;
  if (grid_too_large(B, H, ((int64_t)Sq + kBR - 1) / kBR)) return 0;
  return plan_dense(B, H, Sq, Sk, D, causal != 0, device_cus(), true).ws_bytes;
}

attn_status_t attn_fwd_ws(int dtype, const void* q, const int64_t q_strides[3], const void* k,
                          const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* o,
                          const int64_t o_strides[3], float* lse, int B, int H, int Sq, int Sk, int D,
                          float softmax_scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  attn::FwdArgs a;
  bool empty;
  const attn_status_t st = dense_args(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, Sq,
                                      Sk, D, softmax_scale, causal, &a, &empty);
  if (st != ATTN_OK || empty) return st;
  if (workspace == nullptr) workspace_bytes = 0;
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");
  return dense_launch(a, D, dtype, causal != 0, workspace, workspace_bytes, (hipStream_t)stream);
}

attn_status_t attn_fwd_bias(int dtype, const void* q, const int64_t q_strides[3], const void* k,
                            const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                            const void* bias, const int64_t bias_strides[3], void* o, const int64_t o_strides[3],
                            float* lse, int B, int H, int Sq, int Sk, int D, float softmax_scale, int causal,
                            void* stream) {
  attn::FwdArgs a;
  bool empty;
  const attn_status_t st = dense_args(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, B, H, Sq,
                                      Sk, D, softmax_scale, causal, &a, &empty);
  if (st != ATTN_OK) return st;
  if (D > 128) return fail(ATTN_ERR_UNSUPPORTED, "the score bias supports head_dim 64 and 128 (got %d)", D);
  if (bias_strides == nullptr) return fail(ATTN_ERR_INVALID, "bias_strides is NULL");
  for (int i = 0; i < 3; ++i)
    if (bias_strides[i] < 0 || bias_strides[i] % 8 != 0)
      return fail(ATTN_ERR_INVALID, "bias strides must be non-negative multiples of 8 elements");
  if (empty) return ok();
  if (Sk > 0 && (bias == nullptr || !aligned16(bias))) return fail(ATTN_ERR_INVALID, "bias must be a 16-byte aligned pointer");
  if (2 * ((int64_t)(Sq - 1) * bias_strides[2] + (((int64_t)Sk + 7) & ~int64_t(7))) >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one (batch, head) plane of the bias must span less than 2^31 bytes");
  a.bias = bias;
  a.bias_sb = bias_strides[0]; a.bias_sh = bias_strides[1]; a.bias_ss = bias_strides[2];
  return hip_status(dispatch_fwd16(a, D, dtype, causal != 0, attn::kDenseBias, (hipStream_t)stream),
                    "attn_fwd_bias launch");
}

}  // extern "C"



namespace {

// One query row per sequence (any head dim, a packed cache or pages of any
// size), and at least kDecodeMinWaves (sequence, key range, head) items:
// the streaming decode kernel takes it (a causal mask keeps every key of a
// one-row sequence, so it needs no mask).
bool use_decode(const attn::FwdArgs& a, int D, int mode, int n_split) {
  return a.Sq == 1 && (D == 64 || D == 128 || D == 256) && (mode == attn::kVarlen || mode == attn::kPaged) &&
         (int64_t)a.B * a.H * n_split >= kDecodeMinWaves;
}

// The whole-sequence (one key range) forward of a packed or paged batch.
hipError_t dispatch_varlen(attn::FwdArgs a, int D, int dtype, bool causal, int mode, hipStream_t s) {
  if (use_decode(a, D, mode, 1)) {
    a.n_split = 1;
    a.split_tiles = (int)(((int64_t)a.Sk + 63) / 64);
    return attn::launch_decode(a, D, dtype, s);
  }
  return dispatch_fwd16(a, D, dtype, causal, mode, s);
}

// Validation and argument set-up shared by attn_fwd_varlen and
// attn_fwd_splitkv.  *empty is set when there is nothing to compute.
attn_status_t varlen_args(int dtype, const void* q, const int32_t* cu_seqlens_q, const void* k, const void* v,
                          const int32_t* cu_seqlens_k, const int32_t* block_table, int max_pages_per_seq,
                          int page_size, void* o, float* lse, int B, int H, int D, int total_q, int max_seqlen_q,
                          int max_seqlen_k, float softmax_scale, int causal, attn::FwdArgs* a, int* mode,
                          bool* empty) {
  attn_status_t st;
  *empty = false;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return fail(ATTN_ERR_INVALID, "dtype %d is not bf16/fp16", dtype);
  if (B < 0 || H < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(ATTN_ERR_INVALID, "negative size");
  if ((st = check_head_dim(D)) != ATTN_OK) return st;
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  int page_shift = 0;
  if (block_table != nullptr) {
    if (page_size < 16 || (page_size & (page_size - 1)) != 0)
      return fail(ATTN_ERR_INVALID, "page_size %d must be a power of two >= 16", page_size);
    if (max_pages_per_seq < 1) return fail(ATTN_ERR_INVALID, "max_pages_per_seq must be >= 1");
    if ((int64_t)max_pages_per_seq * page_size < max_seqlen_k)
      return fail(ATTN_ERR_INVALID, "max_pages_per_seq * page_size < max_seqlen_k");
    while ((1 << page_shift) < page_size) ++page_shift;
  }
  if (B == 0 || H == 0 || total_q == 0 || max_seqlen_q == 0) {
    *empty = true;
    return ok();
  }
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return fail(ATTN_ERR_INVALID, "cu_seqlens is NULL");
  if (q == nullptr || o == nullptr) return fail(ATTN_ERR_INVALID, "q or o is NULL");
  if (max_seqlen_k > 0 && (k == nullptr || v == nullptr)) return fail(ATTN_ERR_INVALID, "k or v is NULL");
  if ((int64_t)H * D > kMaxSeqStride) return fail(ATTN_ERR_UNSUPPORTED, "H * head_dim above 2^24 elements");
  if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v) || !aligned16(lse))
    return fail(ATTN_ERR_INVALID, "q, k, v, o and lse must be 16-byte aligned");
  const int64_t n_qblk = ((int64_t)max_seqlen_q + kBR - 1) / kBR;
  if (grid_too_large(B, H, n_qblk) || grid_too_large(H, ((int64_t)total_q + kBR - 1) / kBR + B, 1))
    return fail(ATTN_ERR_INVALID, "problem too large for one launch");

  *a = attn::FwdArgs{};
  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  const int64_t tok = (int64_t)H * D;  // packed [tokens, H, D]
  a->q_ss = tok; a->q_sh = D;
  a->k_ss = tok; a->k_sh = D;
  a->v_ss = tok; a->v_sh = D;
  a->o_ss = tok; a->o_sh = D;
  a->B = B; a->H = H; a->Sq = max_seqlen_q; a->Sk = max_seqlen_k;
  a->scale_log2 = softmax_scale * attn::kLog2e;
  a->cu_q = cu_seqlens_q; a->cu_k = cu_seqlens_k;
  a->block_table = block_table; a->max_pages = max_pages_per_seq; a->page_shift = page_shift;
  a->n_qblk = (int)n_qblk;
  a->total_q = total_q;
  a->n_split = 1;
  *mode = block_table != nullptr ? attn::kPaged : attn::kVarlen;
  return ATTN_OK;
}

std::atomic<bool> g_index_checks{false};

// With index checks on: copy the index arrays to the host (on the call's
// stream, after the work that produced them) and validate them there.
attn_status_t check_device_indices(const attn::FwdArgs& a, int B, int total_q, int max_seqlen_q, int max_seqlen_k,
                                   int page_size, hipStream_t stream) {
  if (!g_index_checks.load(std::memory_order_relaxed)) return ATTN_OK;
  std::vector<int32_t> cq(B + 1), ck(B + 1), tab;
  hipError_t e = hipMemcpyAsync(cq.data(), a.cu_q, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(ck.data(), a.cu_k, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && a.block_table != nullptr) {
    tab.resize((size_t)B * a.max_pages);
    e = hipMemcpyAsync(tab.data(), a.block_table, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost, stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "index check copy");
  return attn_check_indices_host(cq.data(), ck.data(), a.block_table != nullptr ? tab.data() : nullptr,
                                 a.max_pages, page_size, B, total_q, max_seqlen_q, max_seqlen_k);
}

}  // namespace

extern "C" {

void attn_set_index_checks(int enable) { g_index_checks.store(enable != 0, std::memory_order_relaxed); }

attn_status_t attn_check_indices_host(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      const int32_t* block_table, int max_pages_per_seq, int page_size, int B,
                                      int total_q, int max_seqlen_q, int max_seqlen_k) {
  if (B < 0) return fail(ATTN_ERR_INVALID, "negative batch");
  if (B == 0) return ok();
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return fail(ATTN_ERR_INVALID, "cu_seqlens is NULL");
  if (cu_seqlens_q[0] != 0) return fail(ATTN_ERR_INVALID, "cu_seqlens_q[0] = %d, not 0", cu_seqlens_q[0]);
  if (cu_seqlens_k[0] < 0) return fail(ATTN_ERR_INVALID, "cu_seqlens_k[0] = %d is negative", cu_seqlens_k[0]);
  for (int b = 0; b < B; ++b) {
    const int64_t lq = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    const int64_t lk = (int64_t)cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    if (lq < 0 || lk < 0) return fail(ATTN_ERR_INVALID, "cu_seqlens decrease at sequence %d", b);
    if (lq > max_seqlen_q)
      return fail(ATTN_ERR_INVALID, "sequence %d has %lld queries, above max_seqlen_q %d", b, (long long)lq, max_seqlen_q);
    if (lk > max_seqlen_k)
      return fail(ATTN_ERR_INVALID, "sequence %d has %lld keys, above max_seqlen_k %d", b, (long long)lk, max_seqlen_k);
    if (block_table != nullptr) {
      if (page_size <= 0) return fail(ATTN_ERR_INVALID, "page_size %d", page_size);
      const int64_t pages = (lk + page_size - 1) / page_size;
      if (pages > max_pages_per_seq)
        return fail(ATTN_ERR_INVALID, "sequence %d needs %lld pages, above max_pages_per_seq %d", b, (long long)pages,
                    max_pages_per_seq);
      for (int64_t p = 0; p < pages; ++p)
        if (block_table[(int64_t)b * max_pages_per_seq + p] < 0)
          return fail(ATTN_ERR_INVALID, "block_table[%d][%lld] = %d is negative", b, (long long)p,
                      block_table[(int64_t)b * max_pages_per_seq + p]);
    }
  }
  if (cu_seqlens_q[B] != total_q)
    return fail(ATTN_ERR_INVALID, "cu_seqlens_q[B] = %d, but total_q is %d", cu_seqlens_q[B], total_q);
  return ok();
}

attn_status_t attn_fwd_varlen(int dtype, const void* q, const int32_t* cu_seqlens_q, const void* k, const void* v,
                              const int32_t* cu_seqlens_k, const int32_t* block_table, int max_pages_per_seq,
                              int page_size, void* o, float* lse, int B, int H, int D, int total_q,
                              int max_seqlen_q, int max_seqlen_k, float softmax_scale, int causal, void* stream) {
  attn::FwdArgs a;
  int mode;
  bool empty;
  const attn_status_t st = varlen_args(dtype, q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, max_pages_per_seq,
                                       page_size, o, lse, B, H, D, total_q, max_seqlen_q, max_seqlen_k,
                                       softmax_scale, causal, &a, &mode, &empty);
  if (st != ATTN_OK || empty) return st;
  if (const attn_status_t ci = check_device_indices(a, B, total_q, max_seqlen_q, max_seqlen_k, page_size,
                                                    (hipStream_t)stream);
      ci != ATTN_OK)
    return ci;
  return hip_status(dispatch_varlen(a, D, dtype, causal != 0, mode, (hipStream_t)stream), "attn_fwd_varlen launch");
}

}  // extern "C"

namespace {

// The split-key launch and its merge, with the partial results in `part`
// (num_splits * total_q * H * (D + 1) floats, validated by the caller).
attn_status_t splitkv_launch(attn::FwdArgs a, int mode, int dtype, int D, int causal, int num_splits, float* part,
                             const char* name, hipStream_t stream) {
  const int total_q = a.total_q, H = a.H, B = a.B;
  if (grid_too_large(H, ((int64_t)total_q + kBR - 1) / kBR + B, num_splits))
    return fail(ATTN_ERR_INVALID, "problem too large for one launch");
  const int tiles = (int)(((int64_t)a.Sk + 63) / 64);
  a.n_split = num_splits;
  a.split_tiles = (tiles + num_splits - 1) / num_splits;
  a.part_o = part;
  a.part_lse = a.part_o + (size_t)num_splits * total_q * H * D;
  hipError_t e = use_decode(a, D, mode, num_splits) ? attn::launch_decode(a, D, dtype, stream)
                                                     : dispatch_fwd16(a, D, dtype, causal != 0, mode, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s launch: %s", name, hipGetErrorString(e));
  attn::MergeArgs m{};
  m.part_o = a.part_o; m.part_lse = a.part_lse; m.o = a.o; m.lse = a.lse;
  m.n_split = num_splits; m.total_q = total_q; m.H = H;
  e = attn::launch_splitkv_merge(m, D, dtype, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s merge launch: %s", name, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

size_t attn_fwd_splitkv_workspace_bytes(int total_q, int H, int D, int num_splits) {
  if (num_splits <= 1 || total_q <= 0 || H <= 0 || D <= 0) return 0;
  return (size_t)num_splits * (size_t)total_q * (size_t)H * (size_t)(D + 1) * sizeof(float);
}

attn_status_t attn_fwd_splitkv(int dtype, const void* q, const int32_t* cu_seqlens_q, const void* k, const void* v,
                               const int32_t* cu_seqlens_k, const int32_t* block_table, int max_pages_per_seq,
                               int page_size, void* o, float* lse, int B, int H, int D, int total_q,
                               int max_seqlen_q, int max_seqlen_k, float softmax_scale, int causal, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(ATTN_ERR_INVALID, "num_splits %d must be in 1..%d", num_splits, kMaxSplits);
  attn::FwdArgs a;
  int mode;
  bool empty;
  const attn_status_t st = varlen_args(dtype, q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, max_pages_per_seq,
                                       page_size, o, lse, B, H, D, total_q, max_seqlen_q, max_seqlen_k,
                                       softmax_scale, causal, &a, &mode, &empty);
  if (st != ATTN_OK || empty) return st;
  if (const attn_status_t ci = check_device_indices(a, B, total_q, max_seqlen_q, max_seqlen_k, page_size,
                                                    (hipStream_t)stream);
      ci != ATTN_OK)
    return ci;
  if (num_splits == 1)
    return hip_status(dispatch_varlen(a, D, dtype, causal != 0, mode, (hipStream_t)stream), "attn_fwd_splitkv launch");
  const size_t need = attn_fwd_splitkv_workspace_bytes(total_q, H, D, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_INVALID, "workspace of %zu bytes needed (got %zu)", need, workspace == nullptr ? 0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");
  return splitkv_launch(a, mode, dtype, D, causal, num_splits, (float*)workspace, "attn_fwd_splitkv", (hipStream_t)stream);
}

attn_status_t attn_fwd_splitkv_noalloc(int dtype, const void* q, const int32_t* cu_seqlens_q, const void* k,
                                       const void* v, const int32_t* cu_seqlens_k, const int32_t* block_table,
                                       int max_pages_per_seq, int page_size, void* o, float* lse, int B, int H, int D,
                                       int total_q, int max_seqlen_q, int max_seqlen_k, float softmax_scale,
                                       int causal, int num_splits, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(ATTN_ERR_INVALID, "num_splits %d must be in 1..%d", num_splits, kMaxSplits);
  attn::FwdArgs a;
  int mode;
  bool empty;
  const attn_status_t st = varlen_args(dtype, q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, max_pages_per_seq,
                                       page_size, o, lse, B, H, D, total_q, max_seqlen_q, max_seqlen_k,
                                       softmax_scale, causal, &a, &mode, &empty);
  if (st != ATTN_OK || empty) return st;
  if (const attn_status_t ci = check_device_indices(a, B, total_q, max_seqlen_q, max_seqlen_k, page_size,
                                                    (hipStream_t)stream);
      ci != ATTN_OK)
    return ci;
  if (num_splits == 1)
    return hip_status(dispatch_varlen(a, D, dtype, causal != 0, mode, (hipStream_t)stream),
                      "attn_fwd_splitkv_noalloc launch");
  const size_t need = attn_fwd_splitkv_workspace_bytes(total_q, H, D, num_splits);
  if (need > attn::noalloc_scratch_bytes())
    return fail(ATTN_ERR_INVALID,
                "num_splits * total_q * H * (D + 1) * 4 = %zu bytes of partial results exceed the %zu-byte scratch "
                "of attn_fwd_splitkv_noalloc (use attn_fwd_splitkv with a workspace, or fewer splits)",
                need, attn::noalloc_scratch_bytes());
  float* scratch_ptr = nullptr;
  const hipError_t e = attn::noalloc_scratch(&scratch_ptr);
  if (e != hipSuccess) return hip_status(e, "attn_fwd_splitkv_noalloc scratch lookup");
  return splitkv_launch(a, mode, dtype, D, causal, num_splits, scratch_ptr, "attn_fwd_splitkv_noalloc",
                        (hipStream_t)stream);
}

typedef hipError_t (*quant_launcher_t)(const attn::QuantArgs&, int, hipStream_t);

static attn_status_t quantize_8bit(const char* name, quant_launcher_t launch, const void* x,
                                   const int64_t x_strides[3], uint8_t* x8, float* scales, int B, int H, int S,
                                   int D, int block_rows, const int8_t* signs, float premul, void* stream) {
  attn_status_t st;
  if (B < 0 || H < 0 || S < 0) return fail(ATTN_ERR_INVALID, "negative size");
  if ((st = check_head_dim(D)) != ATTN_OK) return st;
  if (!std::isfinite(premul) || !(premul > 0.f))
    return fail(ATTN_ERR_INVALID, "premul must be finite and > 0 (got %g)", (double)premul);
  if (block_rows != 0 && block_rows != 128) return fail(ATTN_ERR_INVALID, "block_rows must be 128 or 0 (got %d)", block_rows);
  if ((st = check_strides("x", x_strides)) != ATTN_OK) return st;
  if (B == 0 || H == 0 || S == 0) return ok();
  if (x == nullptr || x8 == nullptr || scales == nullptr) return fail(ATTN_ERR_INVALID, "x, x8 or scales is NULL");
  if (!aligned16(x) || !aligned16(x8)) return fail(ATTN_ERR_INVALID, "x and x8 must be 16-byte aligned");
  if (grid_too_large(B, H, ((int64_t)S + 127) / 128)) return fail(ATTN_ERR_INVALID, "problem too large");
  attn::QuantArgs a{};
  a.x = (const uint16_t*)x;
  a.x_sb = x_strides[0]; a.x_ss = x_strides[1]; a.x_sh = x_strides[2];
  a.x8 = x8; a.scales = scales; a.signs = signs;
  a.B = B; a.H = H; a.S = S; a.block_rows = block_rows;
  a.premul = premul;
  return hip_status(launch(a, D, (hipStream_t)stream), name);
}

attn_status_t attn_fp8_quantize(const void* x, const int64_t x_strides[3], uint8_t* x8, float* scales, int B, int H,
                                int S, int D, int block_rows, const int8_t* signs, void* stream) {
  return quantize_8bit("attn_fp8_quantize launch", attn::launch_fp8_quantize, x, x_strides, x8, scales, B, H, S, D,
                       block_rows, signs, 1.f, stream);
}

attn_status_t attn_fp8_quantize_pow2(const void* x, const int64_t x_strides[3], uint8_t* x8, float* scales, int B,
                                     int H, int S, int D, int block_rows, const int8_t* signs, float premul,
                                     void* stream) {
  return quantize_8bit("attn_fp8_quantize_pow2 launch", attn::launch_fp8_quantize_pow2, x, x_strides, x8, scales, B,
                       H, S, D, block_rows, signs, premul, stream);
}

attn_status_t attn_int8_quantize(const void* x, const int64_t x_strides[3], int8_t* x8, float* scales, int B, int H,
                                 int S, int D, int block_rows, const int8_t* signs, void* stream) {
  return quantize_8bit("attn_int8_quantize launch", attn::launch_int8_quantize, x, x_strides, (uint8_t*)x8, scales,
                       B, H, S, D, block_rows, signs, 1.f, stream);
}

typedef hipError_t (*fwd8_launcher_t)(const attn::Fp8Args&, int, bool, hipStream_t);

static attn_status_t fwd_8bit(const char* name, fwd8_launcher_t launch, const uint8_t* q8, const float* q_scale,
                              const uint8_t* k8, const float* k_scale, const uint8_t* v8, const float* v_scale,
                              int block_rows, void* o, float* lse, int B, int H, int Sq, int Sk, int D,
                              float softmax_scale, int causal, void* stream) {
  attn_status_t st;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(ATTN_ERR_INVALID, "negative size");
  if (D <= 0) return fail(ATTN_ERR_INVALID, "head_dim %d must be positive", D);
  if (D != 128) return fail(ATTN_ERR_UNSUPPORTED, "the 8-bit path supports head_dim 128 only (got %d)", D);
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  if (block_rows != 0 && block_rows != 128) return fail(ATTN_ERR_INVALID, "block_rows must be 128 or 0 (got %d)", block_rows);
  if (B == 0 || H == 0 || Sq == 0) return ok();
  if (q8 == nullptr || q_scale == nullptr || o == nullptr) return fail(ATTN_ERR_INVALID, "q8, q_scale or o is NULL");
  if (Sk > 0 && (k8 == nullptr || v8 == nullptr || k_scale == nullptr || v_scale == nullptr))
    return fail(ATTN_ERR_INVALID, "k8, v8 or their scales are NULL");
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse))
    return fail(ATTN_ERR_INVALID, "q8, k8, v8, o and lse must be 16-byte aligned");
  const int64_t n_qblk = ((int64_t)Sq + kBR - 1) / kBR;
  if (grid_too_large(B, H, n_qblk)) return fail(ATTN_ERR_INVALID, "problem too large for one launch");
  attn::Fp8Args a{};
  a.q = q8; a.k = k8; a.v = v8; a.qs = q_scale; a.ks = k_scale; a.vs = v_scale;
  a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk;
  a.block_rows = block_rows;
  a.scale_log2 = softmax_scale * attn::kLog2e;
  a.n_qblk = (int)n_qblk;
  return hip_status(launch(a, D, causal != 0, (hipStream_t)stream), name);
}

attn_status_t attn_fwd_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                           const uint8_t* v8, const float* v_scale, int block_rows, void* o, float* lse, int B,
                           int H, int Sq, int Sk, int D, float softmax_scale, int causal, void* stream) {
  return fwd_8bit("attn_fwd_fp8 launch", attn::launch_fwd_fp8, q8, q_scale, k8, k_scale, v8, v_scale, block_rows, o,
                  lse, B, H, Sq, Sk, D, softmax_scale, causal, stream);
}

attn_status_t attn_fwd_fp8_pow2(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                                const uint8_t* v8, const float* v_scale, int block_rows, void* o, float* lse, int B,
                                int H, int Sq, int Sk, int D, int causal, void* stream) {
  // (the Q codes carry the softmax scale: 1 passes the shared checks)
  return fwd_8bit("attn_fwd_fp8_pow2 launch", attn::launch_fwd_fp8_pow2, q8, q_scale, k8, k_scale, v8, v_scale,
                  block_rows, o, lse, B, H, Sq, Sk, D, 1.f, causal, stream);
}

attn_status_t attn_fwd_int8(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                            const uint8_t* v8, const float* v_scale, int block_rows, void* o, float* lse, int B,
                            int H, int Sq, int Sk, int D, float softmax_scale, int causal, void* stream) {
  return fwd_8bit("attn_fwd_int8 launch", attn::launch_fwd_int8, (const uint8_t*)q8, q_scale, (const uint8_t*)k8,
                  k_scale, v8, v_scale, block_rows, o, lse, B, H, Sq, Sk, D, softmax_scale, causal, stream);
}

attn_status_t attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* workspace, int B, int H, int Sq, int Sk,
                       int D, float softmax_scale, int causal, void* stream) {
  attn_status_t st;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return fail(ATTN_ERR_INVALID, "dtype %d is not bf16 or fp16", dtype);
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(ATTN_ERR_INVALID, "negative size");
  if ((st = check_head_dim(D)) != ATTN_OK) return st;
  if (D == 256) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass supports head_dim 64 and 128 (got 256)");
  if ((st = check_scale(softmax_scale)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  if (B == 0 || H == 0 || (Sq == 0 && Sk == 0)) return ok();
  if (Sq > 0 && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr ||
                 workspace == nullptr))
    return fail(ATTN_ERR_INVALID, "q, o, lse, dout, dq or workspace is NULL");
  if (Sk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return fail(ATTN_ERR_INVALID, "k, v, dk or dv is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(lse) || !aligned16(workspace))
    return fail(ATTN_ERR_INVALID, "every tensor must be 16-byte aligned");
  if ((int64_t)H * D > kMaxSeqStride) return fail(ATTN_ERR_INVALID, "H * D too large");
  if (grid_too_large(B, H, ((int64_t)std::max(Sq, Sk) + kBR - 1) / kBR))
    return fail(ATTN_ERR_INVALID, "problem too large for one launch");
  attn::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = workspace;
  a.lse2 = workspace + (size_t)B * H * Sq;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * attn::kLog2e;
  return hip_status(attn::launch_bwd(a, D, dtype == ATTN_BF16 ? attn::kBF16 : attn::kFP16, causal != 0,
                                     (hipStream_t)stream), "attn_bwd launch");
}

}  // extern "C"
