// fa_launch.h — host-side launchers behind the C ABI (arguments already validated by fa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d, causal;
  float scale;
};

struct Fp8FwdArgs {
  const void* q8;
  const void* k8;
  const void* v8;
  float q_descale, k_descale, v_descale;
  void* o;
  float* lse;
  int B, H, N, d, causal;
  float scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // fp32 [B,H,N] workspace: D_i = dO_i · O_i
  int B, H, N, d, causal;
  float scale;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);

// Backward workspace: the fp32 [B,H,N] array D, rounded up to 256 bytes.
inline size_t round_up_256(size_t x) { return (x + 255u) & ~(size_t)255u; }
inline size_t bwd_delta_bytes(int B, int H, int N) {
  return round_up_256((size_t)B * H * N * sizeof(float));
}

}  // namespace fa
