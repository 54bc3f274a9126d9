// Argument block of the backward kernels (plain data, passed by value).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct BwdArgs {
  const void* q;      // [B, Sq, H, D]
  const void* k;      // [B, Sk, H, D]
  const void* v;      // [B, Sk, H, D]
  const void* o;      // [B, Sq, H, D], the forward's output
  const float* lse;   // [B, H, Sq], the forward's logsumexp (natural log)
  const void* dout;   // [B, Sq, H, D]
  void* dq;           // [B, Sq, H, D]
  void* dk;           // [B, Sk, H, D]
  void* dv;           // [B, Sk, H, D]
  float* delta;       // [B, H, Sq] scratch: rowsum(dO * O)
  float* lse2;        // [B, H, Sq] scratch: lse * log2(e), +inf for rows with no key
  int B, H, Sq, Sk;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
};

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t s);

}  // namespace attn
