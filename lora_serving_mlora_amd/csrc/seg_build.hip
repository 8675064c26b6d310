// Segment builder kernels: the stable grouping of a batch's rows by adapter
// (group order and write-back rows of the M031 card's worked example,
// sections 02-03: P, R, Q; A's result to rows 0 and 2, B's to row 1), one
// wave for up to 64 rows, else one workgroup of 256 or 1024 threads in LDS.
// The sort itself is in seg_device.h, shared with the GEMM launches that
// build the segments beside their tiles.
#include "internal.h"
#include "seg_device.h"

namespace mlora {
namespace {

// NT threads (1, 4 or 16 waves, picked by batch size so that small decode
// batches do not pay for barriers across 16 waves)
template <int NT>
__global__ __launch_bounds__(NT) void seg_build_kernel(const int32_t* __restrict__ row_adapter, int n,
                                                       const int32_t* __restrict__ pool_rank, int max_adapters,
                                                       int passes, int cap, int32_t* __restrict__ ws) {
  extern __shared__ uint32_t lds[];
  __shared__ int s_wave[kMaxWaves];
  __shared__ int s_cnt[3];
  seg_build_block<NT>(row_adapter, n, pool_rank, max_adapters, passes, cap, ws, lds, s_wave, s_cnt);
}

// Batches of at most 64 rows (decode steps): one wave, one row per lane, no
// LDS passes and no barriers across waves.
__global__ __launch_bounds__(64) void seg_build_small(const int32_t* __restrict__ row_adapter, int n,
                                                      const int32_t* __restrict__ pool_rank, int max_adapters,
                                                      int32_t* __restrict__ ws) {
  __shared__ int s_sorted[65], s_rank[64];
  seg_build_wave(row_adapter, n, pool_rank, max_adapters, ws, s_sorted, s_rank);
}

template <int NT>
hipError_t launch_nt(const int32_t* row_adapter, int n, const int32_t* pool_rank, int max_adapters, int32_t* ws,
                     hipStream_t stream) {
  const int cap = ((n + 1) + 63) & ~63;
  const size_t lds = (size_t)(2 * cap + kRadix * (NT / 64)) * sizeof(uint32_t);
  if (lds > 64 * 1024) {
    // a batch near the row limit needs most of the 160 KiB of LDS of a CU;
    // the launch itself reports an error if the device cannot provide it
    static LdsLimit limit;
    if (limit.ensure({(const void*)seg_build_kernel<NT>}, lds) != hipSuccess) (void)hipGetLastError();
  }
  const int passes = n <= NT ? 0 : ((max_adapters + 1 < 256) ? 1 : 2);
  MLORA_LAUNCH("seg_build", seg_build_kernel<NT>, dim3(1), dim3(NT), lds, stream, row_adapter, n, pool_rank, max_adapters,
                     passes, cap, ws);
  return launched();
}

}  // namespace

hipError_t launch_seg_build(const int32_t* row_adapter, int n, const int32_t* pool_rank, int max_adapters,
                            int32_t* ws, hipStream_t stream) {
  if (n <= 64 && max_adapters <= 65533) {
    MLORA_LAUNCH("seg_build", seg_build_small, dim3(1), dim3(64), 0, stream, row_adapter, n, pool_rank, max_adapters, ws);
    return launched();
  }
  if (n <= 1024) return launch_nt<256>(row_adapter, n, pool_rank, max_adapters, ws, stream);
  return launch_nt<1024>(row_adapter, n, pool_rank, max_adapters, ws, stream);
}

}  // namespace mlora
