// Streaming copy used to calibrate achievable HBM bandwidth and the hardware
// byte counters (a kernel whose traffic is exactly 2 * bytes).
#include "internal.h"

namespace mlora {
namespace {

__global__ __launch_bounds__(256) void hbm_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                       size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_hbm_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  MLORA_LAUNCH("hbm_copy", hbm_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16);
  return launched();
}

}  // namespace mlora
