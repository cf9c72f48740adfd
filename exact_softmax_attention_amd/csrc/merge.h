// Host-side launch interface of the partial-result merge (merge.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Two partial results of the same query rows: O [B, N, H, d] bf16 and LSE
// [B, H, N] float32 each; out / lse_out may be o_a / lse_a (in place).
struct MergeArgs {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* out;
  float* lse_out;
  int B, N, H, d;
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace attn
