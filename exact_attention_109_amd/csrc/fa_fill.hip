// Zero-fill of float32 device buffers on a stream. A kernel rather than
// hipMemsetAsync, so that work captured into a graph replays it like every
// other kernel of the library.

#include "fa_internal.h"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void zero_f32x4_kernel(float4* __restrict__ p, size_t n4) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_zero_f32x4(float* p, size_t n4, hipStream_t stream) {
  if (n4 == 0) return hipSuccess;
  const size_t blocks = (n4 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(zero_f32x4_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace fa
