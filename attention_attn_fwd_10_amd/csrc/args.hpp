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

enum KvMode { kDense = 0, kVarlen = 1, kPaged = 2, kDenseBias = 3 };

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
};

struct MergeArgs {
  const float* part_o;    // [n_split, total_q, H, D]
  const float* part_lse;  // [n_split, H, total_q]
  void* o;                // [total_q, H, D] bf16 / fp16
  float* lse;             // [H, total_q] or null
  int n_split, total_q, H;
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
};

}  // namespace attn
