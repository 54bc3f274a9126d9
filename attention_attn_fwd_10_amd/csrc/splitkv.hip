// Combine of split-key partial results, for the packed split-key forward and
// for the split tail of the wide dense forward ("Fused attention kernel" page,
// Implementation sketch: the per-row running max and sum are exactly the state
// needed to merge two key ranges).  Each key split s of a row produced a
// normalised output O_s and logsumexp L_s; the row's result is
//   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s,
// computed as m = max_s L_s, w_s = exp(L_s - m), O = sum w_s O_s / sum w_s,
// L = m + ln sum w_s.  Splits that saw no key (L_s = -inf) weigh nothing; a row
// with no key at all gets O = 0 and L = -inf.
#include <mutex>

#include "../../include/attn.h"
#include "common.hpp"

namespace attn {

// ---------------------------------------------------------------------------
// Scratch of the allocation-free split-key entry point: the partial outputs
// and logsumexps live in this file-scope device array instead of a workspace
// the caller allocates.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever passed on.
constexpr size_t kNoAllocScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of this device's `scratch` (the current device's), looked
// up on the first call on each device and kept.
hipError_t noalloc_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

// The merge of one row: partial s has logsumexp pl[s * l_stride] and its D
// outputs at po + s * o_stride (this lane's E of them); writes the lane's E
// merged outputs to op (bf16 / fp16) and, from lane 0, the merged logsumexp
// to *lse when lse is not null.
template <int D, int DT>
__device__ __forceinline__ void merge_row(const float* po, int64_t o_stride, const float* pl, int64_t l_stride,
                                          int n_split, int lane, uint16_t* op, float* lse) {
  constexpr int E = D / 64;
  float m = -INFINITY;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, pl[s * l_stride]);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    po += E * lane;
    for (int s = 0; s < n_split; ++s) {
      const float ls = pl[s * l_stride];
      if (ls == -INFINITY) continue;  // uniform over the wave
      const float w = fast_exp2((ls - m) * kLog2e);
      wsum += w;
      const float* src = po + s * o_stride;
      if constexpr (E == 4) {
        const f32x4 x = *(const f32x4*)src;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += w * x[e];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * src[e];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  op += E * lane;
  if constexpr (E == 1) {
    const uint32_t p = pack2<DT>(acc[0] * inv, 0.f);
    *op = (uint16_t)(p & 0xffffu);
  } else if constexpr (E == 2) {
    *(uint32_t*)op = pack2<DT>(acc[0] * inv, acc[1] * inv);
  } else {
    *(u32x2*)op = u32x2{pack2<DT>(acc[0] * inv, acc[1] * inv), pack2<DT>(acc[2] * inv, acc[3] * inv)};
  }
  if (lane == 0 && lse != nullptr) *lse = wsum > 0.f ? m + __log2f(wsum) * kLn2 : -INFINITY;
}

// one wave per (row, head) of the packed layout; lane l owns head-dim columns
// E*l .. E*l+E-1
template <int D, int DT>
__global__ void __launch_bounds__(256) splitkv_merge_kernel(MergeArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= (int64_t)a.total_q * a.H) return;
  const int row = (int)(item / a.H), h = (int)(item - (int64_t)row * a.H);
  merge_row<D, DT>(a.part_o + ((int64_t)row * a.H + h) * D, (int64_t)a.total_q * a.H * D,
                   a.part_lse + (int64_t)h * a.total_q + row, (int64_t)a.H * a.total_q, a.n_split, lane,
                   (uint16_t*)a.o + ((int64_t)row * a.H + h) * D,
                   a.lse != nullptr ? a.lse + (int64_t)h * a.total_q + row : nullptr);
}

// one wave per row of the split tail of a wide dense launch: tail row
// u * kWideRows + i is query row qblk * kWideRows + i of (b, h), where work
// item tail_start + u = (b * H + h) * n_qblk + qblk
template <int D, int DT>
__global__ void __launch_bounds__(256) tail_merge_kernel(TailMergeArgs a) {
  const int64_t n_rows = (int64_t)a.n_tail * kWideRows;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int u = (int)(row / kWideRows), i = (int)(row - (int64_t)u * kWideRows);
  const int t = a.tail_start + u;
  const int bh = t / a.n_qblk, qblk = t - bh * a.n_qblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int qrow = qblk * kWideRows + i;
  if (qrow >= a.Sq) return;  // rows past the sequence end have no partials
  merge_row<D, DT>(a.part_o + row * D, n_rows * D, a.part_lse + row, n_rows, a.n_split, lane,
                   (uint16_t*)a.o + b * a.o_sb + qrow * a.o_ss + h * a.o_sh,
                   a.lse != nullptr ? a.lse + (int64_t)bh * a.Sq + qrow : nullptr);
}

hipError_t launch_splitkv_merge(const MergeArgs& a, int D, int dtype, hipStream_t s) {
  const int64_t items = (int64_t)a.total_q * a.H;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  if (dtype == kBF16) {
    if (D == 64) hipLaunchKernelGGL((splitkv_merge_kernel<64, kBF16>), grid, block, 0, s, a);
    else if (D == 128) hipLaunchKernelGGL((splitkv_merge_kernel<128, kBF16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((splitkv_merge_kernel<256, kBF16>), grid, block, 0, s, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((splitkv_merge_kernel<64, kFP16>), grid, block, 0, s, a);
    else if (D == 128) hipLaunchKernelGGL((splitkv_merge_kernel<128, kFP16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((splitkv_merge_kernel<256, kFP16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_tail_merge(const TailMergeArgs& a, int D, int dtype, hipStream_t s) {
  const int64_t rows = (int64_t)a.n_tail * kWideRows;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (D != 128) return hipErrorInvalidValue;  // the wide layout's head dim
  if (dtype == kBF16) hipLaunchKernelGGL((tail_merge_kernel<128, kBF16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((tail_merge_kernel<128, kFP16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
