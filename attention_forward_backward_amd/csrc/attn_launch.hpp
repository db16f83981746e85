// attn_launch.hpp -- host-side launch descriptors passed from the C ABI
// (attn_api.hip) to the per-kernel launchers.  Arguments are validated by
// the caller; launchers only pick the compiled variant and enqueue it.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

struct FwdArgs {
  bool bf16;
  const void *q, *k, *v;
  void* o;
  float* lse;
  int BH, S, D;
  bool causal;
  float scale;
  hipStream_t stream;
};

struct BwdArgs {
  bool bf16;
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;  // [B*H*S] f32 workspace
  int BH, S, D;
  bool causal;
  float scale;
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);

}  // namespace attn
