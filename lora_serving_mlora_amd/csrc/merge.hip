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
// element against 2 * rank flops: 8 flop/B at rank 16).  Rows of 16-byte
// pieces take merge_kernel_mfma below, which does the rank products on the
// matrix cores; the vector-ALU form here serves din % 8 != 0 and unaligned
// weights.  It gives a workgroup 4 rows of W0 and
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

// 16-byte rows (din % 8 == 0, aligned W0): the rank product on the matrix
// cores.  Up Down is a contraction over the ranks, 16 per 32x32x16
// MFMA, so a workgroup owns a 128 x 128 tile of W0 (rows c, columns i) and
// each of its four waves 32 rows of it.  Per 16 ranks the workgroup stages
// Down^T [i][q] and Up^T [c][q] of its tile in LDS (zeros past the rank and
// the matrix edges) and every wave runs one MFMA per 32x32 block with A =
// Down^T rows (M = i), B = Up^T rows (N = c), so that a lane's accumulator
// holds one row c and four consecutive columns i per group.  The W0 tile
// goes through LDS too: the wave's 32 rows are loaded as 16-byte row pieces
// (coalesced), stored with their 16-byte chunks XOR-swizzled by row, updated
// in place in the accumulator layout (8-byte pieces) and written back as the
// same row pieces.  At most 128 registers, so that four workgroups share a CU
// (four tiles of W0 in flight): 23.9 us at 4096 x 4096 and rank 16, as the
// vector-ALU form, and 38 / 58 us at ranks 64 / 128 against 51 / 87 us.
// (Persistent workgroups over several tiles, the next tile's W0 loaded during
// this one, held two per CU and took 26 / 51 / 82 us.)
constexpr int kMergeTile = 128;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void merge_kernel_mfma(
    PoolView pv, int adapter, int proj, int rank, float f, uint16_t* __restrict__ W) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kMergeTile * kMergeTile];  // W0 tile, swizzled rows
  __shared__ __attribute__((aligned(16))) uint16_t dT[kMergeTile * 16];          // Down^T [i][q]
  __shared__ __attribute__((aligned(16))) uint16_t uT[kMergeTile * 16];          // Up^T [c][q]
  const int din = pv.din, dout = pv.dout;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.x * kMergeTile, c0 = blockIdx.y * kMergeTile;
  const size_t pt = ((size_t)adapter * pv.n_proj + proj) * pv.max_rank;
  const int32_t* dpage = pv.down_page + pt;
  const int32_t* upage = pv.up_page + pt;
  char* wtb = reinterpret_cast<char*>(wt);

  // the wave's 32 rows of W0: 512 pieces of 16 bytes, 8 per lane, 16 lanes per row
  uint4 wv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = lane + 64 * k, r = 32 * wave + (e >> 4), ch = e & 15;
    const int c = c0 + r, i = i0 + 8 * ch;
    wv[k] = (c < dout && i < din) ? *reinterpret_cast<const uint4*>(W + (size_t)c * din + i) : make_uint4(0u, 0u, 0u, 0u);
  }

  floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  // staging: thread t fills row t & 127 of Down^T and of Up^T, ranks 8 (t >> 7) .. + 7
  const int sr = tid & 127, sq = 8 * (tid >> 7);
  for (int q0 = 0; q0 < rank; q0 += 16) {
    if (q0 > 0) __syncthreads();  // every wave is done with the previous ranks
    uint32_t hd[8], hu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = q0 + sq + e;
      hd[e] = (q < rank && i0 + sr < din) ? pv.down[(size_t)dpage[q] * din + i0 + sr] : 0u;
      hu[e] = (q < rank && c0 + sr < dout) ? pv.up[(size_t)upage[q] * dout + c0 + sr] : 0u;
    }
    if (q0 == 0) {
      // W0 rows into the wave's LDS rows (row r, chunk ch at physical chunk
      // ch ^ (r & 15)), their loads having gone out with the first ranks'
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = lane + 64 * k, r = 32 * wave + (e >> 4), ch = e & 15;
        *reinterpret_cast<uint4*>(wtb + r * 256 + ((ch ^ (r & 15)) << 4)) = wv[k];
      }
    }
    *reinterpret_cast<uint4*>(dT + sr * 16 + sq) =
        make_uint4(hd[0] | (hd[1] << 16), hd[2] | (hd[3] << 16), hd[4] | (hd[5] << 16), hd[6] | (hd[7] << 16));
    *reinterpret_cast<uint4*>(uT + sr * 16 + sq) =
        make_uint4(hu[0] | (hu[1] << 16), hu[2] | (hu[3] << 16), hu[4] | (hu[5] << 16), hu[6] | (hu[7] << 16));
    __syncthreads();
    const uint4 b = *reinterpret_cast<const uint4*>(uT + (32 * wave + (lane & 31)) * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 a = *reinterpret_cast<const uint4*>(dT + (32 * j + (lane & 31)) * 16 + 8 * (lane >> 5));
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       acc[j], 0, 0, 0);
    }
  }

  // update in the accumulator layout: row r = 32 wave + lane % 32, columns
  // 32 j + 8 g + 4 (lane / 32) + 0..3 (one 8-byte piece per group g)
  {
    const int r = 32 * wave + (lane & 31), h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        char* p = wtb + r * 256 + (((4 * j + g) ^ (r & 15)) << 4) + 8 * h;
        const uint2 o = *reinterpret_cast<const uint2*>(p);
        *reinterpret_cast<uint2*>(p) =
            make_uint2(pack_bf2(fmaf(f, acc[j][4 * g], lo_bf(o.x)), fmaf(f, acc[j][4 * g + 1], hi_bf(o.x))),
                       pack_bf2(fmaf(f, acc[j][4 * g + 2], lo_bf(o.y)), fmaf(f, acc[j][4 * g + 3], hi_bf(o.y))));
      }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = lane + 64 * k, r = 32 * wave + (e >> 4), ch = e & 15;
    const int c = c0 + r, i = i0 + 8 * ch;
    if (c < dout && i < din)
      *reinterpret_cast<uint4*>(W + (size_t)c * din + i) =
          *reinterpret_cast<const uint4*>(wtb + r * 256 + ((ch ^ (r & 15)) << 4));
  }
}

}  // namespace

hipError_t launch_merge(const PoolView& pv, int adapter, int proj, int rank, float f, uint16_t* W,
                        hipStream_t stream) {
  const bool vec = pv.din % 8 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (vec) {
    const dim3 grid((pv.din + kMergeTile - 1) / kMergeTile, (pv.dout + kMergeTile - 1) / kMergeTile);
    MLORA_LAUNCH("merge", merge_kernel_mfma, grid, dim3(256), 0, stream, pv, adapter, proj, rank, f, W);
  } else {
    const dim3 grid((pv.din + kMergeThreads * 8 - 1) / (kMergeThreads * 8), (pv.dout + kMergeRows - 1) / kMergeRows);
    MLORA_LAUNCH("merge", (merge_kernel<false>), grid, dim3(kMergeThreads), 0, stream, pv, adapter, proj, rank, f, W);
  }
  return launched();
}

}  // namespace mlora
