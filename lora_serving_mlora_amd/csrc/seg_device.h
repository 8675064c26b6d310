// Segment build: the stable grouping of a batch's rows by adapter of the
// M031 card's worked example (sections 02-03), as device functions shared by
// the segment builder's own kernels and by the GEMM launches that build the
// segments in one workgroup of their own while the others stream W0.
//
// Rows are sorted by key (adapter id for rows on a resident adapter, then the
// base-only rows, then rows with an invalid id), keeping the original order
// inside each key.  Up to 64 rows one wave does it (seg_build_wave); larger
// batches take one workgroup (seg_build_block): up to NT rows each row's
// place is counted directly, the number of smaller (key, row) pairs, all of
// which are distinct; larger batches take an LSD radix sort on 8-bit digits
// of the key (one pass when every key fits in 8 bits, two otherwise).  Each
// radix pass is stable by construction: every wave owns a contiguous range
// of entries, per-(digit, wave) counts are scanned digit-major, and inside a
// 64-entry slice a lane's place among equal digits is the popcount of the
// lower lanes holding the same digit (found with one ballot per digit bit),
// never an atomic's arrival order.  The result is bit-exact and identical run to run.
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

// Workgroup barrier for the builder's LDS data only: the builder writes its
// global outputs and never reads them back, so its barriers wait for the
// LDS operations in flight but not for those stores (a __syncthreads()
// would hold every wave until all its global stores were acknowledged).
__device__ __forceinline__ void seg_sync() {
  asm volatile("" ::: "memory");
  // s_waitcnt lgkmcnt(0) (vmcnt and expcnt not waited)
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
  seg_sync();
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
  seg_sync();
  // segment starts among the active sorted positions
  const int kj = w0 && lane < n_act ? s_sorted[lane] : -1;
  const bool start = w0 && lane < n_act && (lane == 0 || s_sorted[lane - 1] != kj);
  const unsigned long long starts = __ballot(start);
  const int nseg = __popcll(starts);
  const int sidx = __popcll(starts & ((1ull << (lane & 63)) - 1ull));
  seg_sync();
  if (start) {
    ws[MLORA_SEG_ADAPTER(n) + sidx] = kj;
    ws[MLORA_SEG_OFF(n) + sidx] = lane;
    s_sorted[sidx] = lane;
  }
  if (lane == 0) {
    ws[MLORA_SEG_OFF(n) + nseg] = n_act;
    s_sorted[nseg] = n_act;
  }
  seg_sync();
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
  const int n_items = __builtin_amdgcn_readlane(incl, 63);
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

// The valid lanes of the wave whose digit d (nbits <= 8 significant bits)
// equals this lane's: those that agree with it on each of those bits (one
// ballot per bit, whatever the number of distinct digits).
__device__ __forceinline__ unsigned long long same_digit_lanes(bool valid, int d, int nbits) {
  unsigned long long peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = ((d >> b) & 1) != 0;
    const unsigned long long m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Sum over the wave of v, 0 <= v < 32 (one ballot per bit).
__device__ __forceinline__ int wave_sum_small(int v) {
  int sum = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) sum += __popcll(__ballot(((v >> b) & 1) != 0)) << b;
  return sum;
}

constexpr int kRadix = 256;
constexpr int kMaxWaves = 16;

// Exclusive prefix sum of one int per thread over the whole block of NT
// threads; *total gets the block sum.  Every thread of the block must call it.
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  seg_sync();
  if (wave == 0) {
    int w = (lane < kWaves) ? s_wave[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kWaves) s_wave[lane] = w;
  }
  seg_sync();
  const int wave_prefix = wave ? s_wave[wave - 1] : 0;
  *total = s_wave[kWaves - 1];
  seg_sync();
  return wave_prefix + x - v;
}

// The segment build of a whole batch by one workgroup of NT threads (every
// thread must call it: it has workgroup barriers).  lds: 2 * cap + kRadix *
// NT / 64 words of LDS scratch (cap >= n + 1, a multiple of 64); s_wave:
// kMaxWaves ints; s_cnt: 3 ints (base-only rows, invalid rows, status bits).
// passes: 0 counts each row's place directly (n <= NT), else the number of
// 8-bit radix passes over the key.
template <int NT>
__device__ __forceinline__ void seg_build_block(const int32_t* __restrict__ row_adapter, int n,
                                                const int32_t* __restrict__ pool_rank, int max_adapters,
                                                int passes, int cap, int32_t* __restrict__ ws, uint32_t* lds,
                                                int* s_wave, int* s_cnt) {
  constexpr int kThreads = NT;
  constexpr int kWaves = NT / 64;

  uint32_t* bufA = lds;
  uint32_t* bufB = lds + cap;
  uint32_t* hist = lds + 2 * cap;  // [digit][wave]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t A = (uint32_t)max_adapters;
  int32_t* perm = ws + MLORA_SEG_PERM(n);
  int32_t* inv = ws + MLORA_SEG_INV(n);
  int32_t* seg_adapter = ws + MLORA_SEG_ADAPTER(n);
  int32_t* seg_off = ws + MLORA_SEG_OFF(n);
  int32_t* items = ws + MLORA_SEG_ITEMS(n);
  int32_t* row_key = ws + MLORA_SEG_ROWKEY(n);

  // The resident table (one rank per adapter id) is read into the free
  // buffer in the same round trip as the first row ids, so a row's residency
  // test is an LDS read instead of a second, dependent global load.  Used
  // when the table takes one load per thread and fits that buffer.
  const bool table = max_adapters <= kThreads && max_adapters <= cap;
  int32_t* rank_tab = reinterpret_cast<int32_t*>(bufB);
  const int a_first = tid < n ? row_adapter[tid] : -1;
  if (table && tid < max_adapters) rank_tab[tid] = pool_rank[tid];
  if (tid < 3) s_cnt[tid] = 0;
  seg_sync();

  // 1. key of every row, packed with its index: (key << 16) | row; a
  // thread's ids are fetched four rows at a time (one round trip each)
  int my_none = 0, my_bad = 0, my_status = 0;
  for (int k0 = tid; k0 < n; k0 += 4 * kThreads) {
    int ids[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * kThreads;
      ids[u] = k == tid ? a_first : (k < n ? row_adapter[k] : -1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * kThreads;
      if (k >= n) break;
      const int a = ids[u];
      uint32_t key;
      if (a == -1) {
        key = A;
        ++my_none;
      } else if (a < -1 || a >= max_adapters) {
        key = A + 1;
        ++my_bad;
        my_status |= MLORA_SEG_BAD_ID;
      } else if ((table ? rank_tab[a] : pool_rank[a]) <= 0) {
        key = A + 1;
        ++my_bad;
        my_status |= MLORA_SEG_NOT_RESIDENT;
      } else {
        key = (uint32_t)a;
      }
      bufA[k] = (key << 16) | (uint32_t)k;
      row_key[k] = key < A ? (int32_t)key : (key == A ? -1 : -2);
    }
  }
  // one LDS atomic per wave for each count (a thread has at most 16 rows)
  {
    const int w_none = wave_sum_small(my_none), w_bad = wave_sum_small(my_bad);
    const int w_status = (__ballot((my_status & MLORA_SEG_BAD_ID) != 0) ? MLORA_SEG_BAD_ID : 0) |
                         (__ballot((my_status & MLORA_SEG_NOT_RESIDENT) != 0) ? MLORA_SEG_NOT_RESIDENT : 0);
    if (lane == 0) {
      if (w_none) atomicAdd(&s_cnt[0], w_none);
      if (w_bad) atomicAdd(&s_cnt[1], w_bad);
      if (w_status) atomicOr(&s_cnt[2], w_status);
    }
  }
  seg_sync();

  // 2. stable sort of the packed (key, row) values, which are all distinct.
  // passes == 0 (at most one row per thread, up to 256 rows): a row's sorted
  // position is the number of smaller packed values.  Each wave reads 64 of
  // them at a time (one per lane) and broadcasts them lane by lane from
  // registers, so a comparison costs no LDS access.  Otherwise stable LSD
  // radix passes over the key's 8-bit digits.
  uint32_t* src = bufA;
  uint32_t* dst = bufB;
  if (passes == 0) {
    const uint32_t me = tid < n ? bufA[tid] : 0xffffffffu;
    int pos = 0;
    for (int base = 0; base < n; base += 64) {
      const uint32_t other = base + lane < n ? bufA[base + lane] : 0xffffffffu;  // above every packed value
#pragma unroll 16
      for (int l = 0; l < 64; ++l) pos += (int)((uint32_t)__builtin_amdgcn_readlane((int)other, l) < me);
    }
    if (tid < n) bufB[pos] = me;
    seg_sync();
    src = bufB;
    dst = bufA;
  }
  const int per = (((n + kWaves - 1) / kWaves) + 63) & ~63;
  const int beg = min(n, wave * per), end = min(n, wave * per + per);
  // significant bits of the largest key, A + 1 (the invalid rows' key)
  const int key_bits = 32 - __builtin_clz(A + 1u);
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 16 + 8 * pass;
    const int nbits = min(8, key_bits - 8 * pass);
    for (int i = tid; i < kRadix * kWaves; i += kThreads) hist[i] = 0;
    seg_sync();
    for (int i = beg + lane; i < end; i += 64) atomicAdd(&hist[((src[i] >> shift) & 255u) * kWaves + wave], 1u);
    seg_sync();
    {
      const uint32_t v0 = hist[4 * tid], v1 = hist[4 * tid + 1], v2 = hist[4 * tid + 2], v3 = hist[4 * tid + 3];
      int total;
      const uint32_t ex = (uint32_t)block_exclusive_scan<NT>((int)(v0 + v1 + v2 + v3), s_wave, &total);
      hist[4 * tid] = ex;
      hist[4 * tid + 1] = ex + v0;
      hist[4 * tid + 2] = ex + v0 + v1;
      hist[4 * tid + 3] = ex + v0 + v1 + v2;
    }
    seg_sync();
    for (int base = beg; base < end; base += 64) {
      const int i = base + lane;
      const bool valid = i < end;
      const uint32_t e = valid ? src[i] : 0u;
      const int d = (int)((e >> shift) & 255u);
      const unsigned long long peers = same_digit_lanes(valid, d, nbits);
      const unsigned long long below = peers & ((1ull << lane) - 1ull);
      if (valid) dst[hist[d * kWaves + wave] + (uint32_t)__popcll(below)] = e;
      // the lowest lane of each digit advances that digit's cursor (after
      // every lane of the wave has read it: LDS ops of one wave are ordered)
      if (valid && below == 0ull) hist[d * kWaves + wave] += (uint32_t)__popcll(peers);
    }
    seg_sync();
    uint32_t* t = src;
    src = dst;
    dst = t;
  }
  uint32_t* sorted = src;
  uint32_t* offs = dst;  // free buffer: segment offsets in LDS

  const int n_none = s_cnt[0], n_bad = s_cnt[1], status = s_cnt[2];
  const int n_act = n - n_none - n_bad;

  // 3. permutation and its inverse
  for (int j = tid; j < n; j += kThreads) {
    const int k = (int)(sorted[j] & 0xffffu);
    perm[j] = k;
    inv[k] = j;
  }

  // 4. segments: a new one starts wherever the key changes among active rows.
  // Each thread takes a run of E consecutive sorted positions, so one block
  // scan numbers them all.
  int nseg;
  {
    const int E = (n_act + kThreads - 1) / kThreads;
    const int j0 = tid * E, j1 = min(n_act, j0 + E);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += (j == 0) || ((sorted[j - 1] >> 16) != (sorted[j] >> 16));
    int total;
    int at = block_exclusive_scan<NT>(cnt, s_wave, &total);
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = sorted[j] >> 16;
      if ((j == 0) || ((sorted[j - 1] >> 16) != key)) {
        offs[at] = (uint32_t)j;
        seg_adapter[at] = (int32_t)key;
        seg_off[at] = j;
        ++at;
      }
    }
    nseg = total;
  }
  if (tid == 0) {
    offs[nseg] = (uint32_t)n_act;
    seg_off[nseg] = n_act;
  }
  seg_sync();

  // 5. work items: ceil(len / ITEM_ROWS) per segment, in segment order
  uint32_t* item_end = sorted;  // the sorted keys are no longer needed
  int n_items = 0;
  for (int base = 0; base < nseg; base += kThreads) {
    const int s = base + tid;
    int t = 0;
    if (s < nseg) t = (int)((offs[s + 1] - offs[s] + MLORA_ITEM_ROWS - 1) / MLORA_ITEM_ROWS);
    int total;
    const int ex = block_exclusive_scan<NT>(t, s_wave, &total);
    if (s < nseg) item_end[s] = (uint32_t)(n_items + ex + t);
    n_items += total;
  }
  seg_sync();
  for (int i = tid; i < n_items; i += kThreads) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)item_end[mid] > i) hi = mid; else lo = mid + 1;
    }
    const int first = lo ? (int)item_end[lo - 1] : 0;
    items[2 * i] = lo;
    items[2 * i + 1] = (int)offs[lo] + (i - first) * MLORA_ITEM_ROWS;
  }
  seg_sync();

  // 6. tiles: ceil(len / TILE_ROWS) per segment, in segment order
  int32_t* tiles = ws + MLORA_SEG_TILES(n);
  uint32_t* tile_end = sorted;
  int n_tiles = 0;
  for (int base = 0; base < nseg; base += kThreads) {
    const int s = base + tid;
    int t = 0;
    if (s < nseg) t = (int)((offs[s + 1] - offs[s] + MLORA_TILE_ROWS - 1) / MLORA_TILE_ROWS);
    int total;
    const int ex = block_exclusive_scan<NT>(t, s_wave, &total);
    if (s < nseg) tile_end[s] = (uint32_t)(n_tiles + ex + t);
    n_tiles += total;
  }
  seg_sync();
  for (int i = tid; i < n_tiles; i += kThreads) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)tile_end[mid] > i) hi = mid; else lo = mid + 1;
    }
    const int first = lo ? (int)tile_end[lo - 1] : 0;
    tiles[2 * i] = lo;
    tiles[2 * i + 1] = (int)offs[lo] + (i - first) * MLORA_TILE_ROWS;
  }
  if (tid == 0) {
    ws[MLORA_SEG_NSEG] = nseg;
    ws[MLORA_SEG_NACT] = n_act;
    ws[MLORA_SEG_NNONE] = n_none;
    ws[MLORA_SEG_NBAD] = n_bad;
    ws[MLORA_SEG_STATUS] = status;
    ws[MLORA_SEG_NITEMS] = n_items;
    ws[MLORA_SEG_NROWS] = n;
    ws[MLORA_SEG_MAXAD] = max_adapters;
    for (int h = 8; h < MLORA_SEG_HEADER; ++h) ws[h] = 0;
    ws[MLORA_SEG_NTILES] = n_tiles;
  }
}

}  // namespace
}  // namespace mlora
