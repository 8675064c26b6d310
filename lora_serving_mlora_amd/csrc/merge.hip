// Merge and unmerge of one adapter into a base weight, in place:
//
//     W0[c][i] <- bf16( W0[c][i] + f * sum_q Up_a[c][q] Down_a[q][i] ),  f = sign * s_a
//
// The merged weight gives, for rows of that adapter, the same output as the
// base plus the low-rank term (M031 card, section 04: W_merged = W_base +
// scale * Up Down; airsota card, section three, derivation 2), at the cost of
// serving only that adapter with it; f = -s_a takes the term out again (up to
// the bf16 rounding of the two stores).
//
// The update reads and writes every element of W0 once and does rank
// multiply-adds per element, so it is bound by HBM traffic (4 bytes per
// element against 2 * rank flops: 8 flop/B at rank 16), not by arithmetic:
// plain vector FMAs, no matrix cores.  A workgroup owns 16 rows of W0 and
// 2048 columns (8 per thread).  It stages its rows' Up entries (16 x rank,
// gathered from the rank-major Up pages) in LDS; each thread loads its 16 W0
// pieces first (the HBM stream), then walks the ranks: one 16-byte Down
// piece (an L2 hit after the first workgroups: Down is rank x din) and 16
// LDS broadcasts per rank, 128 fp32 accumulators, summed in rank order.
#include "internal.h"

namespace mlora {
namespace {

constexpr int kMergeRows = 16;      // W0 rows per workgroup
constexpr int kMergeThreads = 256;  // 8 columns each: 2048 columns per workgroup

template <bool VEC>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(PoolView pv, int adapter, int proj, int rank, float f,
                                                              uint16_t* __restrict__ W) {
  __shared__ float up_s[kMergeRows][MLORA_MAX_RANK];
  const int din = pv.din, dout = pv.dout;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * kMergeRows;
  const int i0 = blockIdx.x * (kMergeThreads * 8) + tid * 8;
  const size_t pt = ((size_t)adapter * pv.n_proj + proj) * pv.max_rank;
  const int32_t* dpage = pv.down_page + pt;
  const int32_t* upage = pv.up_page + pt;

  // this thread's W0 pieces first: they are the bulk of the traffic
  const bool live = i0 < din;
  uint4 w[kMergeRows];
  if (VEC && live) {
#pragma unroll
    for (int c = 0; c < kMergeRows; ++c)
      if (c0 + c < dout) w[c] = *reinterpret_cast<const uint4*>(W + (size_t)(c0 + c) * din + i0);
  }
  // Up[c0 + c][q] for the workgroup's rows, from page q at offset c0 + c
  for (int e = tid; e < kMergeRows * rank; e += kMergeThreads) {
    const int c = e % kMergeRows, q = e / kMergeRows;
    up_s[c][q] = (c0 + c < dout) ? bf2f(pv.up[(size_t)upage[q] * dout + c0 + c]) : 0.f;
  }
  __syncthreads();
  if (!live) return;

  float acc[kMergeRows][8];
#pragma unroll
  for (int c = 0; c < kMergeRows; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  for (int q = 0; q < rank; ++q) {
    float d[8];
    load8<VEC>(pv.down + (size_t)dpage[q] * din, i0, din, d);
#pragma unroll
    for (int c = 0; c < kMergeRows; ++c) {
      const float u = up_s[c][q];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c][e] = fmaf(u, d[e], acc[c][e]);
    }
  }

#pragma unroll
  for (int c = 0; c < kMergeRows; ++c) {
    if (c0 + c >= dout) continue;
    uint16_t* wr = W + (size_t)(c0 + c) * din + i0;
    if (VEC) {
      const uint4 o = w[c];
      uint4 r;
      r.x = pack_bf2(fmaf(f, acc[c][0], lo_bf(o.x)), fmaf(f, acc[c][1], hi_bf(o.x)));
      r.y = pack_bf2(fmaf(f, acc[c][2], lo_bf(o.y)), fmaf(f, acc[c][3], hi_bf(o.y)));
      r.z = pack_bf2(fmaf(f, acc[c][4], lo_bf(o.z)), fmaf(f, acc[c][5], hi_bf(o.z)));
      r.w = pack_bf2(fmaf(f, acc[c][6], lo_bf(o.w)), fmaf(f, acc[c][7], hi_bf(o.w)));
      *reinterpret_cast<uint4*>(wr) = r;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (i0 + e < din) wr[e] = (uint16_t)f2bf(fmaf(f, acc[c][e], bf2f(wr[e])));
    }
  }
}

}  // namespace

hipError_t launch_merge(const PoolView& pv, int adapter, int proj, int rank, float f, uint16_t* W,
                        hipStream_t stream) {
  const dim3 grid((pv.din + kMergeThreads * 8 - 1) / (kMergeThreads * 8), (pv.dout + kMergeRows - 1) / kMergeRows);
  const bool vec = pv.din % 8 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(pv.down) % 16 == 0;
  if (vec)
    MLORA_LAUNCH("merge", (merge_kernel<true>), grid, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  else
    MLORA_LAUNCH("merge", (merge_kernel<false>), grid, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  return launched();
}

}  // namespace mlora
