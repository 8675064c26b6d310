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
// plain vector FMAs, no matrix cores.  (Ranks <= 16: merge_kernel_r16
// below.)  A workgroup owns 4 rows of W0 and
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

// Ranks <= 16 with 16-byte rows.  The vector ALU work (rank multiply-adds
// per element plus the bf16 unpacking, with no packed fp32 math) took as
// long as the HBM traffic, so this form sums the ranks in pairs with the
// bf16 dot instruction (two exact bf16 products and an fp32 add each): each
// thread loads its 8 columns of all 16 Down rows once, repacks them into
// rank pairs per column, and applies them to kMergeRows16 rows of W0, whose
// pieces it loads first; the rows' Up entries are staged in LDS as rank
// pairs.  Ranks past the adapter's weigh 0.
constexpr int kMergeRows16 = 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel_r16(PoolView pv, int adapter, int proj, int rank,
                                                                  float f, uint16_t* __restrict__ W) {
  __shared__ uint32_t up_p[kMergeRows16][8];  // (Up[c][2p], Up[c][2p+1]) as two bf16
  const int din = pv.din, dout = pv.dout;
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * kMergeRows16;
  const int i0 = blockIdx.x * (kMergeThreads * 8) + tid * 8;
  const size_t pt = ((size_t)adapter * pv.n_proj + proj) * pv.max_rank;
  const int32_t* dpage = pv.down_page + pt;
  const int32_t* upage = pv.up_page + pt;
  const bool live = i0 < din;
  const int nrows = min(kMergeRows16, dout - c0);

  uint4 w[kMergeRows16];
  uint4 d[16];
  if (live) {
#pragma unroll
    for (int c = 0; c < kMergeRows16; ++c)
      w[c] = *reinterpret_cast<const uint4*>(W + (size_t)(c0 + min(c, nrows - 1)) * din + i0);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      d[q] = *reinterpret_cast<const uint4*>(pv.down + (size_t)dpage[min(q, rank - 1)] * din + i0);
  }
  for (int e = tid; e < kMergeRows16 * 8; e += kMergeThreads) {
    const int c = e >> 3, q = 2 * (e & 7);
    const uint32_t lo = (q < rank && c < nrows) ? pv.up[(size_t)upage[q] * dout + c0 + c] : 0u;
    const uint32_t hi = (q + 1 < rank && c < nrows) ? pv.up[(size_t)upage[q + 1] * dout + c0 + c] : 0u;
    up_p[c][e & 7] = lo | (hi << 16);
  }
  __syncthreads();
  if (!live) return;

  // rank pairs per column: dl[p][j] = (D[2p][2j], D[2p+1][2j]), dh[p][j] =
  // (D[2p][2j+1], D[2p+1][2j+1]) for the thread's columns 2j, 2j+1
  uint32_t dl[8][4], dh[8][4];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t a[4] = {d[2 * p].x, d[2 * p].y, d[2 * p].z, d[2 * p].w};
    const uint32_t b[4] = {d[2 * p + 1].x, d[2 * p + 1].y, d[2 * p + 1].z, d[2 * p + 1].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dl[p][j] = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
      dh[p][j] = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
    }
  }
#pragma unroll
  for (int c = 0; c < kMergeRows16; ++c) {
    if (c >= nrows) continue;  // (not break: the loop must unroll, w[] stays in registers)
    uint32_t u[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) u[p] = up_p[c][p];
    float acc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo = 0.f, hi = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        lo = dot2_bf16(u[p], dl[p][j], lo);
        hi = dot2_bf16(u[p], dh[p][j], hi);
      }
      acc[2 * j] = lo;
      acc[2 * j + 1] = hi;
    }
    const uint4 o = w[c];
    uint4 r;
    r.x = pack_bf2(fmaf(f, acc[0], lo_bf(o.x)), fmaf(f, acc[1], hi_bf(o.x)));
    r.y = pack_bf2(fmaf(f, acc[2], lo_bf(o.y)), fmaf(f, acc[3], hi_bf(o.y)));
    r.z = pack_bf2(fmaf(f, acc[4], lo_bf(o.z)), fmaf(f, acc[5], hi_bf(o.z)));
    r.w = pack_bf2(fmaf(f, acc[6], lo_bf(o.w)), fmaf(f, acc[7], hi_bf(o.w)));
    *reinterpret_cast<uint4*>(W + (size_t)(c0 + c) * din + i0) = r;
  }
}

}  // namespace

hipError_t launch_merge(const PoolView& pv, int adapter, int proj, int rank, float f, uint16_t* W,
                        hipStream_t stream) {
  const dim3 grid((pv.din + kMergeThreads * 8 - 1) / (kMergeThreads * 8), (pv.dout + kMergeRows - 1) / kMergeRows);
  const bool vec = pv.din % 8 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(pv.down) % 16 == 0;
  if (vec && rank <= 16) {
    const dim3 grid16((pv.din + kMergeThreads * 8 - 1) / (kMergeThreads * 8),
                      (pv.dout + kMergeRows16 - 1) / kMergeRows16);
    MLORA_LAUNCH("merge", merge_kernel_r16, grid16, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  } else if (vec)
    MLORA_LAUNCH("merge", (merge_kernel<true>), grid, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  else
    MLORA_LAUNCH("merge", (merge_kernel<false>), grid, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  return launched();
}

}  // namespace mlora
