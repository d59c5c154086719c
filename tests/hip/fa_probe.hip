// fa_probe.hip — test harness for the number conversions the attention kernels apply to their
// results (not part of libfa.so).  It runs the kernels' own device helpers from fa_common.h over
// caller-supplied values so the tests can compare them, value by value, with the CPU's rounding:
//   pack_bf16x2  fp32 → bf16, round to nearest even (every O, dQ, dK, dV element and the bf16 P);
//   pack_e4m3x4  fp32 → OCP e4m3fn, round to nearest even, not saturating (the FP8 forward's P).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../io_aware_exact_18_amd/csrc/fa_common.h"

namespace {

__global__ void pack_bf16_kernel(const float* __restrict__ in, uint32_t* __restrict__ out,
                                 size_t pairs) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < pairs) out[i] = fa::pack_bf16x2(in[2 * i], in[2 * i + 1]);
}

__global__ void pack_e4m3_kernel(const float* __restrict__ in, uint32_t* __restrict__ out,
                                 size_t quads) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < quads) out[i] = fa::pack_e4m3x4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
}

}  // namespace

extern "C" {

// out[i] = bf16(in[2i]) | bf16(in[2i+1]) << 16 for i < pairs.  Device pointers; returns a hipError_t.
int probe_pack_bf16(const float* in, uint32_t* out, size_t pairs, hipStream_t stream) {
  if (pairs == 0) return 0;
  const unsigned blocks = (unsigned)((pairs + 255) / 256);
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks), dim3(256), 0, stream, in, out, pairs);
  return (int)hipGetLastError();
}

// out[i] = the four e4m3 bytes of in[4i .. 4i+3], in[4i] in the lowest byte.
int probe_pack_e4m3(const float* in, uint32_t* out, size_t quads, hipStream_t stream) {
  if (quads == 0) return 0;
  const unsigned blocks = (unsigned)((quads + 255) / 256);
  hipLaunchKernelGGL(pack_e4m3_kernel, dim3(blocks), dim3(256), 0, stream, in, out, quads);
  return (int)hipGetLastError();
}

}  // extern "C"
