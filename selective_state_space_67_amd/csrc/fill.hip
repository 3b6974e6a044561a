// Results of empty problems (a sequence of length 0, or no batch rows).
//
// Nothing is scanned then, but some outputs still have a value: the state after
// an empty sequence is the initial state (h_last = h0, the conv state passes
// through), its decay product is the identity (P = 1, H = 0), and the gradients
// that are sums over batch rows and steps (dA, dD, d dt_bias, the conv
// parameters) are empty sums, 0. The adjoint passes through an empty sequence
// unchanged (dh0 = dh_last). One elementwise kernel writes each such output.
#include <algorithm>

#include "kernels.h"

namespace ssm {
namespace {

// dst[i] = src[i] when src is given, else v0 at even and v1 at odd i (so a
// complex value v0 + i v1 stored as (re, im) pairs fills an array of them).
__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                   float v0, float v1, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : ((i & 1) ? v1 : v0);
}

}  // namespace

hipError_t launch_fill(float* dst, const float* src, float v0, float v1, int64_t n, hipStream_t stream) {
  if (!dst || n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  SSM_LOG("launch fill_kernel: %lld floats; grid %lld x 256 threads", static_cast<long long>(n),
          static_cast<long long>(blocks));
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dst, src, v0, v1, n);
  return hipGetLastError();
}

}  // namespace ssm
