// Segment build of a batch of at most 64 rows by one wave: the stable
// grouping of rows by adapter of the M031 card's worked example (sections
// 02-03), for decode steps.  Shared by the segment builder's own small-batch
// kernel and by the decode GEMM launch, which can build the segments in one
// of its workgroups while the others stream W0.
#pragma once

#include "internal.h"

namespace mlora {
namespace {

// The row key that every per-row kernel reads: the adapter id for a row on
// a resident adapter, -1 for a base-only row, -2 for a row whose id is out of
// range or not resident.
__device__ __forceinline__ int row_key_of(int a, int rank_of_a, int max_adapters) {
  if (a == -1) return -1;
  if (a < -1 || a >= max_adapters) return -2;
  return rank_of_a > 0 ? a : -2;
}

// Writes the whole segment workspace `ws` for rows row_adapter[0, n), n <= 64.
// Every thread of the workgroup must call it (it has workgroup barriers);
// only the first wave does the work, one row per lane.  s_sorted (65 ints)
// and s_rank (64 ints) are LDS scratch of the caller's (the GEMM launch lends
// its dynamic LDS, so that its own buffers keep their alignment).  A row's sorted
// position is the number of rows with a smaller (key, row) pair, counted
// against every other lane's key broadcast from registers: the same stable
// order as the radix path of the large-batch builder.
__device__ __forceinline__ void seg_build_wave(const int32_t* __restrict__ row_adapter, int n,
                                               const int32_t* __restrict__ pool_rank, int max_adapters,
                                               int32_t* __restrict__ ws, int* s_sorted, int* s_rank) {
  // s_sorted: sorted keys, then segment offsets; s_rank: the resident table,
  // when it has at most 64 ids
  const int lane = threadIdx.x;
  const bool w0 = lane < 64;
  const bool valid = w0 && lane < n;
  const int A = max_adapters;
  const bool table = A <= 64;
  // row id and table entry travel in the same round trip
  const int a = valid ? row_adapter[lane] : -1;
  if (table && lane < A) s_rank[lane] = pool_rank[lane];
  __syncthreads();
  int key = A + 2, status = 0;  // lanes past n sort after everything
  if (valid) {
    const bool in_range = a >= 0 && a < A;
    const int rk = row_key_of(a, in_range ? (table ? s_rank[a] : pool_rank[a]) : 0, A);
    if (rk >= 0) {
      key = rk;
    } else if (rk == -1) {
      key = A;
    } else {
      key = A + 1;
      status = in_range ? MLORA_SEG_NOT_RESIDENT : MLORA_SEG_BAD_ID;
    }
    ws[MLORA_SEG_ROWKEY(n) + lane] = rk;
  }
  int pos = 0;
  for (int j = 0; j < 64; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    pos += (kj < key) || (kj == key && j < lane);
  }
  if (valid) {
    ws[MLORA_SEG_PERM(n) + pos] = lane;
    ws[MLORA_SEG_INV(n) + lane] = pos;
    s_sorted[pos] = key;
  }
  const unsigned long long act = __ballot(valid && key < A);
  const unsigned long long none = __ballot(valid && key == A);
  const unsigned long long bad = __ballot(valid && key == A + 1);
  int st = status;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) st |= __shfl_xor(st, m, 64);
  const int n_act = __popcll(act);
  __syncthreads();
  // segment starts among the active sorted positions
  const int kj = w0 && lane < n_act ? s_sorted[lane] : -1;
  const bool start = w0 && lane < n_act && (lane == 0 || s_sorted[lane - 1] != kj);
  const unsigned long long starts = __ballot(start);
  const int nseg = __popcll(starts);
  const int sidx = __popcll(starts & ((1ull << (lane & 63)) - 1ull));
  __syncthreads();
  if (start) {
    ws[MLORA_SEG_ADAPTER(n) + sidx] = kj;
    ws[MLORA_SEG_OFF(n) + sidx] = lane;
    s_sorted[sidx] = lane;
  }
  if (lane == 0) {
    ws[MLORA_SEG_OFF(n) + nseg] = n_act;
    s_sorted[nseg] = n_act;
  }
  __syncthreads();
  if (!w0) return;  // no barriers below
  // work items: ceil(len / ITEM_ROWS) per segment, in segment order
  int tiles = 0;
  if (lane < nseg) tiles = (s_sorted[lane + 1] - s_sorted[lane] + MLORA_ITEM_ROWS - 1) / MLORA_ITEM_ROWS;
  int incl = tiles;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const int n_items = __shfl(incl, 63, 64);
  int32_t* items = ws + MLORA_SEG_ITEMS(n);
  for (int t = 0; t < tiles; ++t) {
    items[2 * (incl - tiles + t)] = lane;
    items[2 * (incl - tiles + t) + 1] = s_sorted[lane] + t * MLORA_ITEM_ROWS;
  }
  if (lane == 0) {
    ws[MLORA_SEG_NSEG] = nseg;
    ws[MLORA_SEG_NACT] = n_act;
    ws[MLORA_SEG_NNONE] = __popcll(none);
    ws[MLORA_SEG_NBAD] = __popcll(bad);
    ws[MLORA_SEG_STATUS] = st;
    ws[MLORA_SEG_NITEMS] = n_items;
    ws[MLORA_SEG_NROWS] = n;
    ws[MLORA_SEG_MAXAD] = max_adapters;
  }
  // one tile per segment (a segment here has at most 64 rows)
  if (lane < nseg) {
    ws[MLORA_SEG_TILES(n) + 2 * lane] = lane;
    ws[MLORA_SEG_TILES(n) + 2 * lane + 1] = s_sorted[lane];
  }
  if (lane >= 8 && lane < MLORA_SEG_HEADER) ws[lane] = lane == MLORA_SEG_NTILES ? nseg : 0;
}

}  // namespace
}  // namespace mlora
