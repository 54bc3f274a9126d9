// Launch-side argument blocks of the attention kernels (plain data, passed by
// value) and the 16-bit dtype tags: what the host code needs of the kernels,
// with no device code, so that the host ABI layer also builds with a plain
// C++ compiler (the sanitizer build of the host validation).
#pragma once

#include <stdint.h>

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// dtype tags
constexpr int kBF16 = 0;
constexpr int kFP16 = 1;

// kDenseWide: the dense layout in workgroups of 256 query rows (8 waves, one
// workgroup per CU, each K/V tile copied once for all of them; non-causal,
// head dim 128); the work items of a last, partial round of the grid may run
// as key ranges (FwdArgs tail_start) whose partial results a merge combines.
enum KvMode { kDense = 0, kVarlen = 1, kPaged = 2, kDenseBias = 3, kDenseWide = 4 };
constexpr int kWideRows = 256;  // query rows per kDenseWide workgroup

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, H, Sq, Sk;          // dense sizes; varlen: B = #sequences, Sq/Sk = max lengths
  float scale_log2;          // softmax_scale * log2(e)
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_table;
  int max_pages;
  int page_shift;            // log2(page_size)
  int n_qblk;                // query blocks per (b, h)
  int total_q;               // varlen: rows of the packed q (LSE row length)
  // split keys (varlen / paged only): n_split > 1 gives every (tile, split) a
  // workgroup over key tiles [split * split_tiles, (split + 1) * split_tiles);
  // each writes its normalised partial output and logsumexp in fp32
  // additive score bias (dense only): [B, H, Sq, Sk] by these element strides
  // (keys contiguous; a stride of 0 broadcasts)
  const void* bias;
  int64_t bias_sb, bias_sh, bias_ss;
  int n_split;
  int split_tiles;
  float* part_o;             // [n_split, total_q, H, D]
  float* part_lse;           // [n_split, H, total_q]
  // kDenseWide: work items (logical tiles) [0, tail_start) run whole, in
  // workgroups [0, tail_start); every later item runs as n_split key ranges of
  // split_tiles tiles, item tail_start + u in workgroups tail_start +
  // u * n_split + split, and writes its partial output and logsumexp to
  // part_o [n_split, n_tail * kWideRows, D] / part_lse [n_split, n_tail *
  // kWideRows] (n_tail = B * H * n_qblk - tail_start); tail_start = B * H *
  // n_qblk when nothing is split
  int tail_start;
};

struct MergeArgs {
  const float* part_o;    // [n_split, total_q, H, D]
  const float* part_lse;  // [n_split, H, total_q]
  void* o;                // [total_q, H, D] bf16 / fp16
  float* lse;             // [H, total_q] or null
  int n_split, total_q, H;
};

// merge of the split tail of a kDenseWide launch: tail row r = u * kWideRows
// + i is row i of work item tail_start + u, written to the dense O / LSE
struct TailMergeArgs {
  const float* part_o;    // [n_split, n_tail * kWideRows, D]
  const float* part_lse;  // [n_split, n_tail * kWideRows]
  void* o;                // [B, Sq, H, D] by the strides below, bf16 / fp16
  float* lse;             // [B, H, Sq] or null
  int64_t o_sb, o_ss, o_sh;
  int H, Sq, n_qblk, tail_start, n_tail, n_split;
};

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* qs;
  const float* ks;
  const float* vs;
  void* o;
  float* lse;
  int B, H, Sq, Sk;
  int block_rows;            // 128 or 0 (per-tensor)
  float scale_log2;
  int n_qblk;
};

struct QuantArgs {
  const uint16_t* x;
  int64_t x_sb, x_ss, x_sh;
  uint8_t* x8;
  float* scales;
  const int8_t* signs;
  int B, H, S;
  int block_rows;
  float premul;              // power-of-two e4m3 form: factor applied to every value before the amax
};

}  // namespace attn
