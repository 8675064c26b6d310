// Streaming kernels of known traffic, used to calibrate achievable HBM
// bandwidth and the hardware byte counters: a copy (reads and writes
// exactly `bytes` each), a read (reads exactly `bytes`, writes one word
// per workgroup), and the same read through LDS DMA, the path by which the
// ring GEMMs fetch their operands.
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

// LDS-DMA read: every wave moves 1 KiB per instruction (16 bytes per lane)
// into one of its 8 LDS slots, at most 8 instructions in flight (a slot is
// reused only after its previous piece has landed); at the end the
// workgroup XORs its waves' slots' first 64 words into *out, so the loads
// have a consumer.  At most 512 workgroups (two per CU), each looping.
// The slots are zeroed by ordinary stores first: with the DMA as the only
// writer, the compiler took the final reads for reads of never-written
// memory, folded them away and then set up no LDS base for the DMA.
constexpr int kLdsSlots = 8, kLdsWaves = 4;
__global__ __launch_bounds__(64 * kLdsWaves) void hbm_read_lds_kernel(const void* __restrict__ src, uint32_t n_kib,
                                                                      uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[kLdsWaves][kLdsSlots][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)(n_kib * 1024u), 0x00020000);
  const uint32_t tw = gridDim.x * kLdsWaves;
#pragma unroll
  for (int sl = 0; sl < kLdsSlots; ++sl)
    *reinterpret_cast<uint4*>(&buf[wave][sl][4 * lane]) = make_uint4(0u, 0u, 0u, 0u);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  uint32_t k = 0;
  for (uint32_t pc = blockIdx.x * kLdsWaves + wave; pc < n_kib; pc += tw, ++k) {
    if (k >= kLdsSlots) __builtin_amdgcn_s_waitcnt((kLdsSlots - 1) | (7 << 4) | (15 << 8));  // vmcnt <= 7
    uint32_t* slot = &buf[wave][k % kLdsSlots][0];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, slot, 16, lane * 16, (int)(pc * 1024u), 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t x = 0;
#pragma unroll
  for (int sl = 0; sl < kLdsSlots; ++sl) x ^= buf[threadIdx.x >> 6][sl][lane];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  // one atomic per workgroup (same-address atomics serialize)
  __shared__ uint32_t red[kLdsWaves];
  if (lane == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(out, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

unsigned stream_blocks(size_t n16) {
  size_t blocks = (n16 + kStreamThreads - 1) / kStreamThreads;
  return (unsigned)(blocks > 8192 ? 8192 : blocks);
}

}  // namespace

hipError_t launch_hbm_read_lds(const void* src, size_t bytes, uint32_t* out, hipStream_t stream) {
  const size_t n_kib = bytes / 1024;
  if (n_kib == 0) return hipSuccess;
  if (bytes % 1024 != 0 || bytes > 0x7fffffffu) return hipErrorInvalidValue;
  const size_t want = (n_kib + kLdsWaves - 1) / kLdsWaves;
  const unsigned blocks = (unsigned)(want < 512 ? want : 512);
  MLORA_LAUNCH("hbm_read_lds", hbm_read_lds_kernel, dim3(blocks), dim3(64 * kLdsWaves), 0, stream, src,
               (uint32_t)n_kib, out);
  return launched();
}

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
