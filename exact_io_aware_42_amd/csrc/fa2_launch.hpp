// Host-side launch interface between the C ABI (fa2_api.cpp) and the kernel translation
// units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa2 {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  bool causal;
  float scale_log2;  // softmax_scale * log2(e)
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: D = rowsum(dO * O), fp32 [B, H, N]
  float* lse2;   // workspace: LSE * log2(e), fp32 [B, H, N]
  int B, H, N, d;
  bool causal;
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);  // pre, then dK/dV, then dQ
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa2
