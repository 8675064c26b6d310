// Segment builder: stable grouping of a batch's rows by adapter.
//
// Rows are sorted by key (adapter id for rows on a resident adapter, then the
// base-only rows, then rows with an invalid id), keeping the original order
// inside each key, which yields the group order and write-back rows of the
// M031 card's worked example (sections 02-03: P, R, Q; A's result to rows 0
// and 2, B's to row 1).  The whole batch is handled by one workgroup in LDS.
// Up to 256 rows, each row's place is counted directly: the number of
// smaller (key, row) pairs, all of which are distinct.  Larger batches take
// an LSD radix sort on 8-bit digits of the key (one pass when every key fits
// in 8 bits, two otherwise).  Each radix pass is stable by
// construction: every wave owns a contiguous range of entries, per-(digit,
// wave) counts are scanned digit-major, and inside a 64-entry slice a lane's
// place among equal digits is the popcount of the lower lanes holding the
// same digit (found with ballots), never an atomic's arrival order.  The
// result is bit-exact and identical run to run.
#include "internal.h"
#include "seg_wave.h"

namespace mlora {
namespace {

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
  __syncthreads();
  if (wave == 0) {
    int w = (lane < kWaves) ? s_wave[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kWaves) s_wave[lane] = w;
  }
  __syncthreads();
  const int wave_prefix = wave ? s_wave[wave - 1] : 0;
  *total = s_wave[kWaves - 1];
  __syncthreads();
  return wave_prefix + x - v;
}

// NT threads (1, 4 or 16 waves, picked by batch size so that small decode
// batches do not pay for barriers across 16 waves)
template <int NT>
__global__ __launch_bounds__(NT) void seg_build_kernel(const int32_t* __restrict__ row_adapter, int n,
                                                       const int32_t* __restrict__ pool_rank, int max_adapters,
                                                       int passes, int cap, int32_t* __restrict__ ws) {
  constexpr int kThreads = NT;
  constexpr int kWaves = NT / 64;
  extern __shared__ uint32_t lds[];
  __shared__ int s_wave[kMaxWaves];
  __shared__ int s_cnt[3];  // base-only rows, invalid rows, status bits

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
  __syncthreads();

  // 1. key of every row, packed with its index: (key << 16) | row
  int my_none = 0, my_bad = 0, my_status = 0;
  for (int k = tid; k < n; k += kThreads) {
    const int a = k == tid ? a_first : row_adapter[k];
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
  if (my_none) atomicAdd(&s_cnt[0], my_none);
  if (my_bad) atomicAdd(&s_cnt[1], my_bad);
  if (my_status) atomicOr(&s_cnt[2], my_status);
  __syncthreads();

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
      for (int l = 0; l < 64; ++l) pos += (int)(__builtin_amdgcn_readlane(other, l) < me);
    }
    if (tid < n) bufB[pos] = me;
    __syncthreads();
    src = bufB;
    dst = bufA;
  }
  const int per = (((n + kWaves - 1) / kWaves) + 63) & ~63;
  const int beg = min(n, wave * per), end = min(n, wave * per + per);
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 16 + 8 * pass;
    for (int i = tid; i < kRadix * kWaves; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int i = beg + lane; i < end; i += 64) atomicAdd(&hist[((src[i] >> shift) & 255u) * kWaves + wave], 1u);
    __syncthreads();
    {
      const uint32_t v0 = hist[4 * tid], v1 = hist[4 * tid + 1], v2 = hist[4 * tid + 2], v3 = hist[4 * tid + 3];
      int total;
      const uint32_t ex = (uint32_t)block_exclusive_scan<NT>((int)(v0 + v1 + v2 + v3), s_wave, &total);
      hist[4 * tid] = ex;
      hist[4 * tid + 1] = ex + v0;
      hist[4 * tid + 2] = ex + v0 + v1;
      hist[4 * tid + 3] = ex + v0 + v1 + v2;
    }
    __syncthreads();
    for (int base = beg; base < end; base += 64) {
      const int i = base + lane;
      const bool valid = i < end;
      const uint32_t e = valid ? src[i] : 0u;
      const int d = (int)((e >> shift) & 255u);
      // lanes holding the same digit as this lane
      unsigned long long peers = 0ull;
      unsigned long long todo = __ballot(valid);
      while (todo) {
        const int leader = __ffsll(todo) - 1;
        const int dl = __shfl(d, leader, 64);
        const unsigned long long m = __ballot(valid && d == dl);
        if (valid && d == dl) peers = m;
        todo &= ~m;
      }
      const unsigned long long below = peers & ((1ull << lane) - 1ull);
      if (valid) dst[hist[d * kWaves + wave] + (uint32_t)__popcll(below)] = e;
      // the lowest lane of each digit advances that digit's cursor (after
      // every lane of the wave has read it: LDS ops of one wave are ordered)
      if (valid && below == 0ull) hist[d * kWaves + wave] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
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

  // 4. segments: a new one starts wherever the key changes among active rows
  int nseg = 0;
  for (int base = 0; base < n_act; base += kThreads) {
    const int j = base + tid;
    int flag = 0;
    uint32_t key = 0;
    if (j < n_act) {
      key = sorted[j] >> 16;
      flag = (j == 0) || ((sorted[j - 1] >> 16) != key);
    }
    int total;
    const int ex = block_exclusive_scan<NT>(flag, s_wave, &total);
    if (flag) {
      offs[nseg + ex] = (uint32_t)j;
      seg_adapter[nseg + ex] = (int32_t)key;
      seg_off[nseg + ex] = j;
    }
    nseg += total;
  }
  if (tid == 0) {
    offs[nseg] = (uint32_t)n_act;
    seg_off[nseg] = n_act;
  }
  __syncthreads();

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
  __syncthreads();
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
  __syncthreads();

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
  __syncthreads();
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
    static size_t attr_bytes = 0;
    if (lds > attr_bytes) {
      if (hipFuncSetAttribute((const void*)seg_build_kernel<NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds) == hipSuccess)
        attr_bytes = lds;
      else
        (void)hipGetLastError();
    }
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
