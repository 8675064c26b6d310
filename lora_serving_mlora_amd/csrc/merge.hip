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
// plain vector FMAs, no matrix cores.  A workgroup owns 4 rows of W0 and
// 2048 columns (8 per thread): small, so the ~8 workgroups a CU holds are in
// different phases (loading, summing, storing) and the HBM stream does not
// stall while they all sum at once.  It stages its rows' Up entries (4 x rank,
// gathered from the rank-major Up pages) and the Down page ids in LDS; each
// thread loads its 4 W0 pieces first (the HBM stream), then walks the ranks
// eight at a time: eight 16-byte Down pieces in flight together (L2 hits
// after the first workgroups: Down is rank x din), 4 LDS broadcasts per
// rank, 32 fp32 accumulators, summed in rank order.
#include "internal.h"

namespace mlora {
namespace {

constexpr int kMergeRows = 4;       // W0 rows per workgroup
constexpr int kMergeThreads = 256;  // 8 columns each: 2048 columns per workgroup

template <bool VEC>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(PoolView pv, int adapter, int proj, int rank, float f,
                                                              uint16_t* __restrict__ W) {
  // Up entries of the workgroup's rows, ranks padded to a multiple of 8 with
  // zeros; Down page ids, the padding pointing at the last rank's page
  __shared__ float up_s[kMergeRows][MLORA_MAX_RANK];
  __shared__ int32_t dp_s[MLORA_MAX_RANK];
  const int din = pv.din, dout = pv.dout;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * kMergeRows;
  const int i0 = blockIdx.x * (kMergeThreads * 8) + tid * 8;
  const int rpad = (rank + 7) & ~7;
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
  if (tid < rpad) dp_s[tid] = dpage[min(tid, rank - 1)];
  for (int e = tid; e < kMergeRows * rpad; e += kMergeThreads) {
    const int c = e % kMergeRows, q = e / kMergeRows;
    up_s[c][q] = (q < rank && c0 + c < dout) ? bf2f(pv.up[(size_t)upage[q] * dout + c0 + c]) : 0.f;
  }
  __syncthreads();
  if (!live) return;

  float acc[kMergeRows][8];
#pragma unroll
  for (int c = 0; c < kMergeRows; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  // eight ranks per round: their Down pieces are in flight together
  for (int q0 = 0; q0 < rpad; q0 += 8) {
    float d[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) load8<VEC>(pv.down + (size_t)dp_s[q0 + j] * din, i0, din, d[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int c = 0; c < kMergeRows; ++c) {
        const float u = up_s[c][q0 + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = fmaf(u, d[j][e], acc[c][e]);
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
