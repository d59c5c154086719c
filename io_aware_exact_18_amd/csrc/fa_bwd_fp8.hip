// fa_bwd_fp8.hip — the part of the FP8 backward that is not shared with the bf16 backward.
//
// The FP8 backward differentiates the FP8 forward's attention ("Anatomy of a FlashAttention Kernel",
// sections "How does FlashAttention save memory in the backward pass?" and "What changed between
// FlashAttention 1, 2, and 3?"): Q, K, V arrive as e4m3fn codes with one fp32 scale per tensor.
// Every e4m3 value is exactly a bf16 value, so the codes are widened once into bf16 images and the
// bf16 backward kernels run on them, with the three scales folded into the softmax scale, into D and
// into the dK and dQ output scales (the products stay exact in the codes; only the scalar factors
// move).  This file holds the widening kernel.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kCvtThreads = 256;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16 bit patterns of two e4m3 values held as the two fp32 results of one conversion: an e4m3 value
// has at most 4 significant bits and an exponent inside bf16's range, so keeping the upper half of the
// fp32 pattern is exact.
__device__ inline uint32_t pack_hi16(f32x2 v) {
  return (__float_as_uint(v[1]) & 0xFFFF0000u) | (__float_as_uint(v[0]) >> 16);
}

// Each thread widens 16 codes (one 16-byte load, two 16-byte stores) per grid-stride step.
__global__ __launch_bounds__(kCvtThreads) void e4m3_to_bf16_kernel(const u32x4* __restrict__ src,
                                                                    u32x4* __restrict__ dst,
                                                                    size_t chunks) {
  for (size_t c = (size_t)blockIdx.x * kCvtThreads + threadIdx.x; c < chunks;
       c += (size_t)gridDim.x * kCvtThreads) {
    const u32x4 x = src[c];
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = pack_hi16(__builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], false));
      const uint32_t b = pack_hi16(__builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], true));
      if (w < 2) {
        lo[2 * w] = a;
        lo[2 * w + 1] = b;
      } else {
        hi[2 * w - 4] = a;
        hi[2 * w - 3] = b;
      }
    }
    dst[2 * c] = lo;
    dst[2 * c + 1] = hi;
  }
}

}  // namespace

hipError_t launch_e4m3_to_bf16(const void* src, void* dst, size_t n, hipStream_t stream) {
  const size_t chunks = n / 16;
  if (chunks == 0) return hipSuccess;
  const size_t want = (chunks + kCvtThreads - 1) / kCvtThreads;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);  // grid-stride beyond 8192 blocks
  hipLaunchKernelGGL(e4m3_to_bf16_kernel, dim3(grid), dim3(kCvtThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, chunks);
  return hipGetLastError();
}

}  // namespace fa
