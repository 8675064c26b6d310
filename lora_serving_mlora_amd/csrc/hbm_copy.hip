// Streaming kernels of known traffic, used to calibrate achievable HBM
// bandwidth and the hardware byte counters: a copy (reads and writes
// exactly `bytes` each) and a read (reads exactly `bytes`, writes one word
// per workgroup).
#include "internal.h"

namespace mlora {
namespace {

constexpr int kStreamThreads = 256, kStreamDepth = 8;  // 16-byte pieces in flight per thread
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void hbm_copy_kernel(u32x4* __restrict__ dst,
                                                                  const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kStreamDepth - 1) * stride < n16; i += kStreamDepth * stride) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) v[d] = __builtin_nontemporal_load(src + i + d * stride);
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) __builtin_nontemporal_store(v[d], dst + i + d * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// out[0] ^= the xor of every 32-bit word read (a checksum the host can
// compare, so the loads cannot be dropped)
__global__ __launch_bounds__(kStreamThreads) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                  uint32_t* __restrict__ out) {
  __shared__ uint32_t red[kStreamThreads / 64];
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kStreamDepth - 1) * stride < n16; i += kStreamDepth * stride) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) v[d] = __builtin_nontemporal_load(src + i + d * stride);
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) x ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) y ^= red[w];
    atomicXor(out, y);
  }
}

unsigned stream_blocks(size_t n16) {
  size_t blocks = (n16 + kStreamThreads - 1) / kStreamThreads;
  return (unsigned)(blocks > 8192 ? 8192 : blocks);
}

}  // namespace

hipError_t launch_hbm_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  MLORA_LAUNCH("hbm_copy", hbm_copy_kernel, dim3(stream_blocks(n16)), dim3(kStreamThreads), 0, stream,
               static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n16);
  return launched();
}

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* out, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  MLORA_LAUNCH("hbm_read", hbm_read_kernel, dim3(stream_blocks(n16)), dim3(kStreamThreads), 0, stream,
               static_cast<const u32x4*>(src), n16, out);
  return launched();
}

}  // namespace mlora
