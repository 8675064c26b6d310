// The low-rank branch of the multi-LoRA linear: for every row on an adapter,
// y += s_a * Up_a (Down_a x), with rows gathered by index through the
// segment permutation and results written back to their original rows
// (M031 card, section 02: group rows by adapter, run Down then Up per group,
// add the result at the original rows; wiblog article, Punica section:
// per-group BAx written back in the original order).
//
// Work is organised in items of up to MLORA_ITEM_ROWS rows of one segment
// (built by the segment builder), so adapters of different ranks and groups
// of any size share one launch: a one-token group is one item, a large group
// many.  Every kernel walks the item list with a grid-stride loop and exits
// on the device-side count, so no host synchronisation is needed.
//
// Decode-sized work is bound by reading the adapter pages from HBM, so these
// kernels use vector ALU dot products on 16-byte loads (8 bf16 per lane,
// coalesced along din or dout) rather than matrix cores:
//  * shrink: one wave per (item, 512-element slice of din); each lane keeps
//    a [rows x 16 ranks] block of partial dot products and the wave finishes
//    them with a butterfly reduce-scatter (6 xor-shuffle steps that halve
//    the live values each time, leaving one finished sum per lane) instead
//    of one full reduction per value.  Slices go to separate partial
//    buffers that the expand sums in a fixed order: no atomics.
//  * expand: one wave per (item, 512 columns of dout); t comes from the
//    partials, Up pages are read as rank-major rows (a page is one column of
//    Up), and each lane owns 8 output columns of each row of the item, so Y
//    is updated by read-modify-write with no atomics.
//  * fused: one 8-wave workgroup per item does the shrink over all of din
//    (per-wave butterfly, then a fixed-order sum of the 8 waves in LDS),
//    keeps t in LDS and runs the expand over all of dout: t never touches
//    HBM and the branch is one launch.
// Rows with an invalid adapter id are set to NaN by the expand and fused
// kernels (after the items).
#include "internal.h"
#include "row_kernels.h"

namespace mlora {
namespace {

constexpr int R = MLORA_ITEM_ROWS;  // rows per item
constexpr int G = 16;               // ranks per group (R * G = 64 = one value per lane after reduction)
static_assert(R * G == 64, "one reduced value per lane");

struct Item {
  int seg, j0, nr, adapter, rank;
  float scale;
};

__device__ __forceinline__ Item load_item(const PoolView& pv, const int32_t* __restrict__ ws, int n, int it) {
  const int32_t* items = ws + MLORA_SEG_ITEMS(n);
  Item m;
  m.seg = items[2 * it];
  m.j0 = items[2 * it + 1];
  const int end = ws[MLORA_SEG_OFF(n) + m.seg + 1];
  m.nr = min(R, end - m.j0);
  m.adapter = ws[MLORA_SEG_ADAPTER(n) + m.seg];
  m.rank = pv.rank[m.adapter];
  m.scale = pv.scale[m.adapter];
  return m;
}

// Butterfly reduce-scatter over the 64 lanes of a wave: on entry every lane
// holds 64 partial sums v[0..64); on exit lane l holds the full sum of
// index l.  Step m pairs lane l with l^m; the lane whose bit m is clear
// keeps the lower half of its live values and ships the upper half.
__device__ __forceinline__ float wave_reduce_scatter64(float (&v)[64]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const float send = upper ? v[i] : v[i + m];
      const float keep = upper ? v[i + m] : v[i];
      v[i] = keep + __shfl_xor(send, m, 64);
    }
  }
  return v[0];
}

// Partial dot products of one wave over din elements [k, k+8) for a rank
// group: acc[i*G + q] += Down[g0+q][k..k+8) . x_i[k..k+8).  Ranks past the
// adapter's rank read its last page instead (those sums are never stored),
// so all 16 page loads are issued back to back with no tests.
template <bool VEC>
__device__ __forceinline__ void shrink_step(const PoolView& pv, const int32_t* __restrict__ dpage, int g0, int rank,
                                            const float (&x)[R][8], int k, float (&acc)[64]) {
  float d[G][8];
#pragma unroll
  for (int q = 0; q < G; ++q) load8<VEC>(pv.down + (size_t)dpage[min(g0 + q, rank - 1)] * pv.din, k, pv.din, d[q]);
#pragma unroll
  for (int q = 0; q < G; ++q)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float s = acc[i * G + q];
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(d[q][e], x[i][e], s);
      acc[i * G + q] = s;
    }
}

// The item's rows at din elements [k, k+8); rows past nr repeat the last
// row (their results are never stored).
template <bool VEC>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ X, const int32_t* __restrict__ perm, int din,
                                          int j0, int nr, int k, float (&x)[R][8]) {
#pragma unroll
  for (int i = 0; i < R; ++i) load8<VEC>(X + (size_t)perm[j0 + min(i, nr - 1)] * din, k, din, x[i]);
}

// y_i[c..c+8) += sum_q ts[i][q] * Up^T[q][c..c+8) for the rows of an item,
// then read-modify-write of Y (bf16 RNE).  ts holds zeros from the rank up
// to the next multiple of G, so ranks are walked in full groups of G page
// loads (pages past the rank are clamped to the last one and weigh zero).
template <bool VEC>
__device__ __forceinline__ void expand_cols(const PoolView& pv, const int32_t* __restrict__ upage, int rank,
                                            const float (*ts)[MLORA_MAX_RANK], const int32_t* __restrict__ perm,
                                            int j0, int nr, int c, uint16_t* __restrict__ Y) {
  const int dout = pv.dout;
  float acc[R][8];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int g0 = 0; g0 < rank; g0 += G) {
    float u[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q) load8<VEC>(pv.up + (size_t)upage[min(g0 + q, rank - 1)] * dout, c, dout, u[q]);
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float t = ts[i][g0 + q];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(t, u[q][e], acc[i][e]);
      }
  }
  float yo[R][8];
  uint16_t* y[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    y[i] = Y + (size_t)perm[j0 + min(i, nr - 1)] * dout;
    load8<VEC>(y[i], c, dout, yo[i]);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i >= nr) continue;
    if (VEC) {
      uint4 w;
      w.x = pack_bf2(yo[i][0] + acc[i][0], yo[i][1] + acc[i][1]);
      w.y = pack_bf2(yo[i][2] + acc[i][2], yo[i][3] + acc[i][3]);
      w.z = pack_bf2(yo[i][4] + acc[i][4], yo[i][5] + acc[i][5]);
      w.w = pack_bf2(yo[i][6] + acc[i][6], yo[i][7] + acc[i][7]);
      *reinterpret_cast<uint4*>(y[i] + c) = w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < dout) y[i][c + e] = (uint16_t)f2bf(yo[i][e] + acc[i][e]);
    }
  }
}

// NaN over columns [c, c+8) of an invalid row.
template <bool VEC>
__device__ __forceinline__ void nan_cols(uint16_t* __restrict__ y, int c, int dout) {
  if (VEC) {
    *reinterpret_cast<uint4*>(y + c) = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < dout) y[c + e] = 0x7fc0;
  }
}

// ---------------------------------------------------------------------------
// shrink: grid (items, n_chunks), one wave per block
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(64) void shrink_kernel(PoolView pv, int proj, const uint16_t* __restrict__ X,
                                                    const int32_t* __restrict__ ws, int n, float* __restrict__ T,
                                                    int chunk_elems) {
  const int lane = threadIdx.x;
  const int n_items = ws[MLORA_SEG_NITEMS];
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  const int c = blockIdx.y;
  const int k_beg = c * chunk_elems;
  const int k_end = min(pv.din, k_beg + chunk_elems);
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const Item m = load_item(pv, ws, n, it);
    const int32_t* dpage = pv.down_page + ((size_t)m.adapter * pv.n_proj + proj) * pv.max_rank;
    for (int g0 = 0; g0 < m.rank; g0 += G) {
      float acc[64];
#pragma unroll
      for (int v = 0; v < 64; ++v) acc[v] = 0.f;
      for (int k = k_beg + lane * 8; k < k_end; k += 512) {
        float x[R][8];
        load_rows<VEC>(X, perm, pv.din, m.j0, m.nr, k, x);
        shrink_step<VEC>(pv, dpage, g0, m.rank, x, k, acc);
      }
      const float tot = wave_reduce_scatter64(acc);
      const int i = lane / G, q = g0 + lane % G;
      if (i < m.nr && q < m.rank) T[((size_t)c * n + m.j0 + i) * pv.max_rank + q] = tot;
    }
  }
}

// ---------------------------------------------------------------------------
// expand: grid (items + invalid rows, column chunks of 512), one wave
// ---------------------------------------------------------------------------
// over (when not null): nothing to do unless *over is nonzero.
template <bool VEC>
__global__ __launch_bounds__(64) void expand_kernel(PoolView pv, int proj, const float* __restrict__ T, int n_chunks,
                                                    const int32_t* __restrict__ ws, uint16_t* __restrict__ Y, int n,
                                                    const int32_t* __restrict__ over) {
  if (over != nullptr && *over == 0) return;
  __shared__ float ts[R][MLORA_MAX_RANK];
  const int lane = threadIdx.x;
  const int n_items = ws[MLORA_SEG_NITEMS];
  const int n_bad = ws[MLORA_SEG_NBAD];
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  const int c = blockIdx.y * 512 + lane * 8;
  for (int it = blockIdx.x; it < n_items + n_bad; it += gridDim.x) {
    if (it < n_items) {
      const Item m = load_item(pv, ws, n, it);
      const int rpad = (m.rank + G - 1) / G * G;
      for (int idx = lane; idx < R * rpad; idx += 64) {
        const int i = idx / rpad, q = idx % rpad;
        float s = 0.f;
        if (i < m.nr && q < m.rank) {
          const float* tp = T + ((size_t)(m.j0 + i)) * pv.max_rank + q;
          const size_t cs = (size_t)n * pv.max_rank;
#pragma unroll 8
          for (int ch = 0; ch < n_chunks; ++ch) s += tp[ch * cs];
        }
        ts[i][q] = m.scale * s;
      }
      __syncthreads();
      if (c < pv.dout) {
        const int32_t* upage = pv.up_page + ((size_t)m.adapter * pv.n_proj + proj) * pv.max_rank;
        expand_cols<VEC>(pv, upage, m.rank, ts, perm, m.j0, m.nr, c, Y);
      }
      __syncthreads();
    } else if (c < pv.dout) {
      nan_cols<VEC>(Y + (size_t)perm[n - n_bad + (it - n_items)] * pv.dout, c, pv.dout);
    }
  }
}

// ---------------------------------------------------------------------------
// fused: one 512-thread workgroup per item.  The shrink runs one row of the
// item at a time with the per-row body (8 waves over din, 16 ranks per
// reduction group: few live registers, so nothing spills), the scaled t of
// the item's rows stays in LDS, then the expand runs over all of dout.
// ---------------------------------------------------------------------------
constexpr int kFusedThreads = kRowThreads;

// The first expand pass of a thread (columns c..c+8, ranks below G) with its
// Up pieces already in registers (bf16 pairs as loaded); later rank groups
// are loaded here.  Then read-modify-write of Y, as expand_cols.
__device__ __forceinline__ void expand_cols_pre(const PoolView& pv, const int32_t* __restrict__ upage, int rank,
                                                const float (*ts)[MLORA_MAX_RANK], const int32_t* __restrict__ perm,
                                                int j0, int nr, int c, const uint4 (&u0)[G],
                                                uint16_t* __restrict__ Y) {
  const int dout = pv.dout;
  float acc[R][8];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const uint32_t w[4] = {u0[q].x, u0[q].y, u0[q].z, u0[q].w};
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float t = ts[i][q];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[i][2 * h] = fmaf(t, lo_bf(w[h]), acc[i][2 * h]);
        acc[i][2 * h + 1] = fmaf(t, hi_bf(w[h]), acc[i][2 * h + 1]);
      }
    }
  }
  for (int g0 = G; g0 < rank; g0 += G) {
    float u[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q) load8<true>(pv.up + (size_t)upage[min(g0 + q, rank - 1)] * dout, c, dout, u[q]);
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float t = ts[i][g0 + q];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(t, u[q][e], acc[i][e]);
      }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i >= nr) continue;
    uint16_t* y = Y + (size_t)perm[j0 + i] * dout;
    const uint4 o = *reinterpret_cast<const uint4*>(y + c);
    uint4 w;
    w.x = pack_bf2(lo_bf(o.x) + acc[i][0], hi_bf(o.x) + acc[i][1]);
    w.y = pack_bf2(lo_bf(o.y) + acc[i][2], hi_bf(o.y) + acc[i][3]);
    w.z = pack_bf2(lo_bf(o.z) + acc[i][4], hi_bf(o.z) + acc[i][5]);
    w.w = pack_bf2(lo_bf(o.w) + acc[i][6], hi_bf(o.w) + acc[i][7]);
    *reinterpret_cast<uint4*>(y + c) = w;
  }
}

// One step of the reduce-scatter of G partial sums over a wave (as in
// shrink_row_to): lanes with bit MSK set keep the upper LEN values, the
// others the lower LEN, each adding its partner's copy.
template <int MSK, int LEN>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[G], int lane) {
  const bool upper = (lane & MSK) != 0;
#pragma unroll
  for (int j = 0; j < LEN; ++j) {
    const float send = upper ? v[j] : v[j + LEN];
    const float keep = upper ? v[j + LEN] : v[j];
    v[j] = keep + __shfl_xor(send, MSK, 64);
  }
}

// Fast form of one item (rank <= G, din and dout <= 8 * kFusedThreads, 16-byte
// aligned rows): each thread owns 8 elements of din for the shrink and 8
// columns of dout for the expand, and every load of the item goes out before
// any arithmetic waits for one: the X rows and the Down rows first, then the
// Up pieces and the Y pieces of the read-modify-write.  Loads return in
// issue order, so the Down stream is not queued behind the Up stream, and
// the Y read is not a round trip of its own at the end.  The arithmetic is
// that of shrink_row_to and expand_cols_pre.
// row0: the item's first original row when the caller already has it, else
// -1 (read from perm here).
__device__ __forceinline__ void fused_item_fast(const PoolView& pv, const Item& m, const int32_t* __restrict__ dpage,
                                                const int32_t* __restrict__ upage, const uint16_t* __restrict__ X,
                                                const int32_t* __restrict__ perm, uint16_t* __restrict__ Y,
                                                float (*ts)[MLORA_MAX_RANK], float (*red)[G], int row0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = tid * 8;  // this thread's din elements and dout columns
  const bool kin = k0 < pv.din, cin = k0 < pv.dout;
  // page ids and rows are uniform over the workgroup (scalar registers)
  int dp[G], up[G], row[R];
#pragma unroll
  for (int q = 0; q < G; ++q) {
    dp[q] = __builtin_amdgcn_readfirstlane(dpage[min(q, pv.max_rank - 1)]);
    up[q] = __builtin_amdgcn_readfirstlane(upage[min(q, pv.max_rank - 1)]);
  }
#pragma unroll
  for (int q = 1; q < G; ++q) {  // pages past the rank: the first page, weighed 0
    dp[q] = dp[q] < 0 ? dp[0] : dp[q];
    up[q] = up[q] < 0 ? up[0] : up[q];
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    row[i] = (i == 0 && row0 >= 0) ? row0 : __builtin_amdgcn_readfirstlane(perm[m.j0 + min(i, m.nr - 1)]);
  // the first row's X and Y pieces go out with the weights; an item's
  // further rows (same adapter) load theirs when they come up
  // loads are unconditional (threads past din or dout read the last piece;
  // their X piece is zeroed, their expand is never stored), so every load
  // is a plain global load from a uniform base
  const int kc = min(k0, pv.din - 8), cc = min(k0, pv.dout - 8);
  uint4 d[G], u[G];
  uint4 x0 = *reinterpret_cast<const uint4*>(X + (size_t)row[0] * pv.din + kc);
#pragma unroll
  for (int q = 0; q < G; ++q) d[q] = *reinterpret_cast<const uint4*>(pv.down + (size_t)dp[q] * pv.din + kc);
#pragma unroll
  for (int q = 0; q < G; ++q) u[q] = *reinterpret_cast<const uint4*>(pv.up + (size_t)up[q] * pv.dout + cc);
  const uint4 y0 = *reinterpret_cast<const uint4*>(Y + (size_t)row[0] * pv.dout + cc);
  if (!kin) x0 = make_uint4(0u, 0u, 0u, 0u);
  // shrink, row by row: partial dot products of 8 din elements, the
  // reduce-scatter of shrink_row_to, then the 8 waves summed in order
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i >= m.nr) break;
    uint4 xi = x0;
    if (i > 0) {
      xi = *reinterpret_cast<const uint4*>(X + (size_t)row[i] * pv.din + kc);
      if (!kin) xi = make_uint4(0u, 0u, 0u, 0u);
    }
    const uint32_t xw[4] = {xi.x, xi.y, xi.z, xi.w};
    float v[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const uint32_t dw[4] = {d[q].x, d[q].y, d[q].z, d[q].w};
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        s = fmaf(lo_bf(dw[h]), lo_bf(xw[h]), s);
        s = fmaf(hi_bf(dw[h]), hi_bf(xw[h]), s);
      }
      v[q] = s;
    }
    reduce_scatter_step<32, 8>(v, lane);
    reduce_scatter_step<16, 4>(v, lane);
    reduce_scatter_step<8, 2>(v, lane);
    reduce_scatter_step<4, 1>(v, lane);
    float tot = v[0];
    tot += __shfl_xor(tot, 2, 64);
    tot += __shfl_xor(tot, 1, 64);
    if ((lane & 3) == 0) red[wave][lane >> 2] = tot;
    __syncthreads();
    if (tid < G) {
      float sum = red[0][tid];
#pragma unroll
      for (int w = 1; w < kFusedThreads / 64; ++w) sum += red[w][tid];
      ts[i][tid] = tid < m.rank ? m.scale * sum : 0.f;  // zeros past the rank
    }
    __syncthreads();
  }
  if (!cin) return;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i >= m.nr) break;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const uint32_t w[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
      const float t = ts[i][q];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[2 * h] = fmaf(t, lo_bf(w[h]), acc[2 * h]);
        acc[2 * h + 1] = fmaf(t, hi_bf(w[h]), acc[2 * h + 1]);
      }
    }
    const uint4 o = i == 0 ? y0 : *reinterpret_cast<const uint4*>(Y + (size_t)row[i] * pv.dout + cc);
    uint4 w;
    w.x = pack_bf2(lo_bf(o.x) + acc[0], hi_bf(o.x) + acc[1]);
    w.y = pack_bf2(lo_bf(o.y) + acc[2], hi_bf(o.y) + acc[3]);
    w.z = pack_bf2(lo_bf(o.z) + acc[4], hi_bf(o.z) + acc[5]);
    w.w = pack_bf2(lo_bf(o.w) + acc[6], hi_bf(o.w) + acc[7]);
    *reinterpret_cast<uint4*>(Y + (size_t)row[i] * pv.dout + k0) = w;
  }
}

// Batches whose every item takes the fast form (the pool's largest rank at
// most G; din, dout <= 8 * kFusedThreads; 16-byte aligned rows): the fused
// kernel without the general form's registers.
__global__ __launch_bounds__(kFusedThreads) void fused_fast_kernel(PoolView pv, int proj,
                                                                   const uint16_t* __restrict__ X,
                                                                   const int32_t* __restrict__ ws,
                                                                   uint16_t* __restrict__ Y, int n) {
  __shared__ float ts[R][MLORA_MAX_RANK];
  __shared__ float red[kFusedThreads / 64][G];
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  // The first item's entries are read together with the counts, and so are
  // the entries of segment b and sorted position b (b = this workgroup):
  // when the item is (segment b, first position b), as every item is where
  // each row has an adapter of its own, its adapter, end and first row
  // arrive two dependent loads earlier than through load_item.  (Indices are
  // clamped to the arrays; the values are used only when the item matches.)
  const int b = blockIdx.x;
  const int bi = min(b, MLORA_SEG_MAX_ITEMS(n) - 1), bs = min(b, n - 1);
  const int g_seg = ws[MLORA_SEG_ITEMS(n) + 2 * bi], g_j0 = ws[MLORA_SEG_ITEMS(n) + 2 * bi + 1];
  const int g_ad = ws[MLORA_SEG_ADAPTER(n) + bs], g_end = ws[MLORA_SEG_OFF(n) + bs + 1], g_row = perm[bs];
  const int n_items = ws[MLORA_SEG_NITEMS];
  const int n_bad = ws[MLORA_SEG_NBAD];
  for (int it = b; it < n_items + n_bad; it += gridDim.x) {
    if (it < n_items) {
      Item m;
      int row0 = -1;
      if (it == b && g_seg == b && g_j0 == b) {
        m.seg = b;
        m.j0 = b;
        m.nr = min(R, g_end - b);
        m.adapter = g_ad;
        m.rank = pv.rank[g_ad];
        m.scale = pv.scale[g_ad];
        row0 = g_row;
      } else {
        m = load_item(pv, ws, n, it);
      }
      const size_t pt = ((size_t)m.adapter * pv.n_proj + proj) * pv.max_rank;
      fused_item_fast(pv, m, pv.down_page + pt, pv.up_page + pt, X, perm, Y, ts, red, row0);
      __syncthreads();
    } else {
      uint16_t* y = Y + (size_t)perm[n - n_bad + (it - n_items)] * pv.dout;
      for (int c = threadIdx.x * 8; c < pv.dout; c += kFusedThreads * 8) nan_cols<true>(y, c, pv.dout);
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kFusedThreads) void fused_kernel(PoolView pv, int proj, const uint16_t* __restrict__ X,
                                                              const int32_t* __restrict__ ws,
                                                              uint16_t* __restrict__ Y, int n) {
  __shared__ float ts[R][MLORA_MAX_RANK];
  const int tid = threadIdx.x;
  const int n_items = ws[MLORA_SEG_NITEMS];
  const int n_bad = ws[MLORA_SEG_NBAD];
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  for (int it = blockIdx.x; it < n_items + n_bad; it += gridDim.x) {
    if (it < n_items) {
      const Item m = load_item(pv, ws, n, it);
      const size_t pt = ((size_t)m.adapter * pv.n_proj + proj) * pv.max_rank;
      const int32_t* upage = pv.up_page + pt;
      const int rpad = (m.rank + G - 1) / G * G;
      // VEC: the Up pieces of this thread's first columns and first 16 ranks
      // do not depend on t, so they are fetched before the shrink and arrive
      // while it runs (pages past the rank fall back to the first one and
      // weigh zero)
      const int c0 = tid * 8;
      uint4 u0[G];
      if (VEC && c0 < pv.dout) {
        int pg[G];
#pragma unroll
        for (int q = 0; q < G; ++q) pg[q] = upage[min(q, pv.max_rank - 1)];
#pragma unroll
        for (int q = 1; q < G; ++q) pg[q] = pg[q] < 0 ? pg[0] : pg[q];
#pragma unroll
        for (int q = 0; q < G; ++q) u0[q] = *reinterpret_cast<const uint4*>(pv.up + (size_t)pg[q] * pv.dout + c0);
      }
      for (int i = 0; i < R; ++i) {
        if (i < m.nr)
          shrink_row_to<VEC>(pv, pv.down_page + pt, m.rank, m.scale, X + (size_t)perm[m.j0 + i] * pv.din, ts[i]);
        // zeros past the rank up to the group size the expand walks
        for (int q = m.rank + tid; q < rpad; q += kFusedThreads) ts[i][q] = 0.f;
      }
      __syncthreads();
      int c = c0;
      if (VEC && c < pv.dout) {
        expand_cols_pre(pv, upage, m.rank, ts, perm, m.j0, m.nr, c, u0, Y);
        c += kFusedThreads * 8;
      }
      for (; c < pv.dout; c += kFusedThreads * 8) expand_cols<VEC>(pv, upage, m.rank, ts, perm, m.j0, m.nr, c, Y);
      __syncthreads();
    } else {
      uint16_t* y = Y + (size_t)perm[n - n_bad + (it - n_items)] * pv.dout;
      for (int c = tid * 8; c < pv.dout; c += kFusedThreads * 8) nan_cols<VEC>(y, c, pv.dout);
    }
  }
}

// ---------------------------------------------------------------------------
// shrink_rows (decode): one 8-wave workgroup per row (body in row_kernels.h)
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void shrink_rows_kernel(PoolView pv, int proj, const uint16_t* __restrict__ X,
                                                                  const int32_t* __restrict__ row_key, int n,
                                                                  float* __restrict__ T) {
  for (int k = blockIdx.x; k < n; k += gridDim.x)
    shrink_row_body<VEC>(pv, proj, X, row_key, k, T, row_desc(T, n, pv.max_rank));
}

// ---------------------------------------------------------------------------
// shrink_tiles (large groups): one 4-wave workgroup per (64-row segment
// tile, din slice).  At prefill sizes a group holds hundreds of rows and the
// shrink is a real contraction (ranks up to 64 and more need more flops per
// byte than the vector ALU gives at HBM speed), so it runs on the matrix
// cores: v_mfma_f32_16x16x32_bf16 with A = 16 gathered X rows and B = 16
// Down rank rows.  Each wave takes all 64 rows of the tile and up to 64
// ranks over its own quarter of the slice, so every X element and every
// Down element of the slice is read exactly once by the workgroup, straight
// from global memory into MFMA operands; the four quarters are summed
// through LDS in a fixed order.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

constexpr int kTileWaves = 4;
constexpr int kTileRB = MLORA_TILE_ROWS / 16;  // 16-row MFMA blocks per tile

// Two MFMA operand fragments from 128-byte row pieces: `lo` holds rows
// l & 7, `hi` rows 8 + (l & 7), 16-byte chunk l >> 3 of a 64-element K
// segment.  f0 takes chunk 2g for lane group g = l >> 4 (the even chunks),
// f1 the odd chunks; lanes 0-7 of each 16-lane row carry rows 0-7 and lanes
// 8-15 rows 8-15, as the MFMA operand layout wants.  One DPP move per dword.
__device__ __forceinline__ void frag_pair(const uint4& lo, const uint4& hi, uint4& f0, uint4& f1) {
  f0.x = __builtin_amdgcn_update_dpp((int)lo.x, (int)hi.x, 0x118, 0xf, 0xc, false);  // row_shr:8 into lanes 8-15
  f0.y = __builtin_amdgcn_update_dpp((int)lo.y, (int)hi.y, 0x118, 0xf, 0xc, false);
  f0.z = __builtin_amdgcn_update_dpp((int)lo.z, (int)hi.z, 0x118, 0xf, 0xc, false);
  f0.w = __builtin_amdgcn_update_dpp((int)lo.w, (int)hi.w, 0x118, 0xf, 0xc, false);
  f1.x = __builtin_amdgcn_update_dpp((int)hi.x, (int)lo.x, 0x108, 0xf, 0x3, false);  // row_shl:8 into lanes 0-7
  f1.y = __builtin_amdgcn_update_dpp((int)hi.y, (int)lo.y, 0x108, 0xf, 0x3, false);
  f1.z = __builtin_amdgcn_update_dpp((int)hi.z, (int)lo.z, 0x108, 0xf, 0x3, false);
  f1.w = __builtin_amdgcn_update_dpp((int)hi.w, (int)lo.w, 0x108, 0xf, 0x3, false);
}

template <int NG>  // rank groups of 16 in this pass
__device__ __forceinline__ void shrink_tile_pass(const PoolView& pv, const uint16_t* __restrict__ X,
                                                 const int32_t* __restrict__ perm, int j0, int jend, int q0,
                                                 int rank, const int32_t* __restrict__ dpage, int k0, int k1,
                                                 float* __restrict__ Tc, floatx4* __restrict__ red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int din = pv.din;
  // this wave's quarter of the slice in 64-wide segments; the last wave also
  // takes a trailing 32-wide step
  const int segs = (k1 - k0) / 64;
  const int kb = k0 + 64 * ((segs * wave) / kTileWaves);
  const int km = k0 + 64 * ((segs * (wave + 1)) / kTileWaves);
  const int ke = wave == kTileWaves - 1 ? k1 : km;
  // X: 128-byte pieces of rows 8h + (l & 7) of each 16-row block (for the
  // segment loop) and the plain fragment rows l & 15 (for the 32-wide tail)
  const uint16_t* xp[kTileRB][2];
  const uint16_t* xt[kTileRB];
#pragma unroll
  for (int rb = 0; rb < kTileRB; ++rb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = min(j0 + 16 * rb + 8 * h + (lane & 7), jend - 1);  // rows past the tile repeat its last row
      xp[rb][h] = X + (size_t)perm[j] * din + (lane >> 3) * 8;
    }
    xt[rb] = X + (size_t)perm[min(j0 + 16 * rb + (lane & 15), jend - 1)] * din + (lane >> 4) * 8;
  }
  // Down: rank rows q0 + 16g + (l & 15); ranks past the adapter's repeat its last
  const uint16_t* dr[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int pg = dpage[min(q0 + 16 * g + (lane & 15), rank - 1)];
    dr[g] = pv.down + (size_t)pg * din + (lane >> 4) * 8;
  }
  floatx4 acc[kTileRB][NG];
#pragma unroll
  for (int rb = 0; rb < kTileRB; ++rb)
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[rb][g] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k = kb; k < km; k += 64) {
    uint4 xa[kTileRB][2], d0[NG], d1[NG];
#pragma unroll
    for (int rb = 0; rb < kTileRB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) xa[rb][h] = *reinterpret_cast<const uint4*>(xp[rb][h] + k);
    // B chunks matching f0 (chunk 2g of the segment) and f1 (chunk 2g + 1)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      d0[g] = *reinterpret_cast<const uint4*>(dr[g] + k + (lane >> 4) * 8);
      d1[g] = *reinterpret_cast<const uint4*>(dr[g] + k + (lane >> 4) * 8 + 8);
    }
#pragma unroll
    for (int rb = 0; rb < kTileRB; ++rb) {
      uint4 f0, f1;
      frag_pair(xa[rb][0], xa[rb][1], f0, f1);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        acc[rb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f0), as_bf16x8(d0[g]), acc[rb][g], 0, 0, 0);
        acc[rb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f1), as_bf16x8(d1[g]), acc[rb][g], 0, 0, 0);
      }
    }
  }
  for (int k = km; k < ke; k += 32) {
    uint4 a[kTileRB], b[NG];
#pragma unroll
    for (int rb = 0; rb < kTileRB; ++rb) a[rb] = *reinterpret_cast<const uint4*>(xt[rb] + k);
#pragma unroll
    for (int g = 0; g < NG; ++g) b[g] = *reinterpret_cast<const uint4*>(dr[g] + k);
#pragma unroll
    for (int rb = 0; rb < kTileRB; ++rb)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        acc[rb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb]), as_bf16x8(b[g]), acc[rb][g], 0, 0, 0);
  }
  // quarters -> LDS, then wave w sums row block w over the quarters in order
#pragma unroll
  for (int rb = 0; rb < kTileRB; ++rb)
#pragma unroll
    for (int g = 0; g < NG; ++g) red[((wave * kTileRB + rb) * NG + g) * 64 + lane] = acc[rb][g];
  __syncthreads();
  const int rb = wave;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    floatx4 sum = red[((0 * kTileRB + rb) * NG + g) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kTileWaves; ++w) sum += red[((w * kTileRB + rb) * NG + g) * 64 + lane];
    // C[(l >> 4) * 4 + v][l & 15]: row of the block, rank of the group
    const int q = q0 + 16 * g + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int jj = j0 + 16 * rb + (lane >> 4) * 4 + v;
      if (jj < jend && q < rank) Tc[(size_t)jj * pv.max_rank + q] = sum[v];
    }
  }
  __syncthreads();  // red is reused by the next pass
}

__global__ __launch_bounds__(64 * kTileWaves) void shrink_tiles_kernel(PoolView pv, int proj,
                                                                       const uint16_t* __restrict__ X,
                                                                       const int32_t* __restrict__ ws, int n,
                                                                       float* __restrict__ T, int chunk_elems) {
  __shared__ floatx4 red[kTileWaves * kTileRB * 4 * 64];  // 64 KiB
  const int n_tiles = ws[MLORA_SEG_NTILES];
  const int32_t* tiles = ws + MLORA_SEG_TILES(n);
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  const int c = blockIdx.y;
  const int k0 = min(c * chunk_elems, pv.din), k1 = min(k0 + chunk_elems, pv.din);
  float* Tc = T + (size_t)c * n * pv.max_rank;
  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int seg = __builtin_amdgcn_readfirstlane(tiles[2 * t]);
    const int j0 = __builtin_amdgcn_readfirstlane(tiles[2 * t + 1]);
    const int jend = min(j0 + MLORA_TILE_ROWS, __builtin_amdgcn_readfirstlane(ws[MLORA_SEG_OFF(n) + seg + 1]));
    const int adapter = __builtin_amdgcn_readfirstlane(ws[MLORA_SEG_ADAPTER(n) + seg]);
    const int rank = __builtin_amdgcn_readfirstlane(pv.rank[adapter]);
    const int32_t* dpage = pv.down_page + ((size_t)adapter * pv.n_proj + proj) * pv.max_rank;
    for (int q0 = 0; q0 < rank; q0 += 64) {
      const int rem = rank - q0;
      if (rem > 32)
        shrink_tile_pass<4>(pv, X, perm, j0, jend, q0, rank, dpage, k0, k1, Tc, red);
      else if (rem > 16)
        shrink_tile_pass<2>(pv, X, perm, j0, jend, q0, rank, dpage, k0, k1, Tc, red);
      else
        shrink_tile_pass<1>(pv, X, perm, j0, jend, q0, rank, dpage, k0, k1, Tc, red);
    }
  }
}

// ---------------------------------------------------------------------------
// lora_prep: the operands of the large-batch GEMM's low-rank term.
// (Columns per gather block: small enough that the LDS tile lets the
// launch's blocks all be resident at once.)
// Every block first sums r_pad (rank rounded up to 16) over the batch's
// segments: when the sum, rounded up to 64, is at most txw, the batch takes
// the rank-concatenated form (Tx, Ux: extra K stages of the GEMM), else the
// epilogue form (tb, upt).  Adapter a's ranks start at koff[a] = the sum of
// r_pad over the segments before a's, in both forms.
// Blocks [0, nt): t per original row, the scaled sum of the shrink's din
// slices in slice order (the same arithmetic the expand applies), rounded
// to bf16: compact and zero-padded to wt (epilogue form), or at the
// adapter's columns of a Kx-wide row, zeros elsewhere and NaN for a row with
// an invalid id (concatenated form).  Block 0 records Kx (0: epilogue form).
// Blocks [nt, ...): one per (segment, kPrepCols columns): the adapter's Up
// columns, ranks contiguous and zeros past the rank, as a [dout][r_pad] block
// at koff * dout (epilogue form) or at columns koff .. koff + r_pad - 1 of
// the [dout][txw] rows of Ux, the last segment's blocks also zeroing the
// columns up to Kx (concatenated form); koff recorded per adapter id.  In
// the epilogue form a block that would end past upt_units rank rows writes
// nothing, and the first column block of the last segment (of the first,
// with no segment) records in *over whether the batch's blocks overran.
// ---------------------------------------------------------------------------
constexpr int kPrepCols = 64;
constexpr int kConcatSegs = kMaxConcatRanks / 16;  // segments of a concatenated batch, at most

__device__ __forceinline__ int rank_pad16(int r) { return (r + 15) & ~15; }

// The sum of the shrink's n_chunks din slices of one t entry (slice stride
// cs), in slice order.  Up to 8 slices the loads are all issued before the
// first add (a load-add loop would wait out one round trip per slice).
__device__ __forceinline__ float sum_slices(const float* __restrict__ p, size_t cs, int n_chunks) {
  float v = 0.f;
  if (n_chunks <= 8) {
    float x[8];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) x[ch] = p[(size_t)min(ch, n_chunks - 1) * cs];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch)
      if (ch < n_chunks) v += x[ch];
  } else {
    for (int ch = 0; ch < n_chunks; ++ch) v += p[(size_t)ch * cs];
  }
  return v;
}

__global__ __launch_bounds__(256) void lora_prep_kernel(PoolView pv, int proj, const int32_t* __restrict__ ws, int n,
                                                        const float* __restrict__ Ts, int n_chunks,
                                                        uint16_t* __restrict__ tb, int wt, int nt,
                                                        int32_t* __restrict__ koff_out, uint16_t* __restrict__ upt,
                                                        long upt_units, int32_t* __restrict__ over,
                                                        uint16_t* __restrict__ tx, int txw, int32_t* __restrict__ kx_out) {
  const int tid = threadIdx.x;
  const int nseg = ws[MLORA_SEG_NSEG];
  const int32_t* seg_adapter = ws + MLORA_SEG_ADAPTER(n);
  const int chunks = (pv.dout + kPrepCols - 1) / kPrepCols;
  const bool tpart = (int)blockIdx.x < nt;
  const int sidx = tpart ? 0 : (blockIdx.x - nt) / chunks, cc = tpart ? 0 : (blockIdx.x - nt) % chunks;
  // r_pad over all segments, and over those before this block's (each
  // thread sums every 256th, then block sums); the first kConcatSegs
  // segments' adapters and r_pad kept for the concatenated form's rows
  __shared__ int part[2][4];
  __shared__ int tab_ad[kConcatSegs], tab_rank[kConcatSegs];
  __shared__ float tab_scale[kConcatSegs];
  int all = 0, before = 0;
  for (int s2 = tid; s2 < nseg; s2 += 256) {
    const int ad = seg_adapter[s2];
    const int rk = pv.rank[ad], rp = rank_pad16(rk);
    if (s2 < kConcatSegs) {
      tab_ad[s2] = ad;
      tab_rank[s2] = rk;
      tab_scale[s2] = pv.scale[ad];
    }
    all += rp;
    before += s2 < sidx ? rp : 0;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    all += __shfl_xor(all, m, 64);
    before += __shfl_xor(before, m, 64);
  }
  if ((tid & 63) == 0) {
    part[0][tid >> 6] = all;
    part[1][tid >> 6] = before;
  }
  __syncthreads();
  const int total = part[0][0] + part[0][1] + part[0][2] + part[0][3];
  const int koff = part[1][0] + part[1][1] + part[1][2] + part[1][3];
  const int kx = (tx != nullptr && total > 0 && ((total + 63) & ~63) <= txw) ? (total + 63) & ~63 : 0;
  const size_t cs = (size_t)n * pv.max_rank;

  if (tpart) {
    if (blockIdx.x == 0 && tid == 0 && kx_out != nullptr) *kx_out = kx;
    if (kx) {
      // (kx > 0: at most kConcatSegs segments, all in the table)
      const int32_t* row_key = ws + MLORA_SEG_ROWKEY(n);
      const int32_t* inv = ws + MLORA_SEG_INV(n);
      const int per_row = kx / 8;
      for (long idx = (long)blockIdx.x * 256 + tid; idx < (long)n * per_row; idx += (long)nt * 256) {
        const int r = (int)(idx / per_row), c0 = (int)(idx % per_row) * 8;
        const int key = row_key[r];
        const int j = inv[r];
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = key == -2 ? 0x7fc0u : 0u;
        if (key >= 0) {
          // the adapter's rank, scale and first column (r_pad of the segments before its own)
          int ko = 0, run = 0, rank = 0;
          float sc = 0.f;
          for (int s2 = 0; s2 < nseg; ++s2) {
            if (tab_ad[s2] == key) {
              ko = run;
              rank = tab_rank[s2];
              sc = tab_scale[s2];
            }
            run += rank_pad16(tab_rank[s2]);
          }
          const float* tp = Ts + (size_t)j * pv.max_rank;
          if (n_chunks <= 8) {
            // all 8 x n_chunks loads first, then the sums in slice order
            float x[8][8];
#pragma unroll
            for (int ch = 0; ch < 8; ++ch)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int q = c0 + e - ko;
                x[ch][e] = (q >= 0 && q < rank && ch < n_chunks) ? tp[(size_t)ch * cs + q] : 0.f;
              }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q = c0 + e - ko;
              float v = 0.f;
#pragma unroll
              for (int ch = 0; ch < 8; ++ch)
                if (ch < n_chunks) v += x[ch][e];
              if (q >= 0 && q < rank) h[e] = f2bf(v * sc);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q = c0 + e - ko;
              if (q >= 0 && q < rank) h[e] = f2bf(sum_slices(tp + q, cs, n_chunks) * sc);
            }
          }
        }
        *reinterpret_cast<uint4*>(tx + (size_t)r * txw + c0) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
      return;
    }
    const int n_act = ws[MLORA_SEG_NACT];
    const int32_t* perm = ws + MLORA_SEG_PERM(n);
    const int32_t* row_key = ws + MLORA_SEG_ROWKEY(n);
    for (int idx = blockIdx.x * 256 + tid; idx < n_act * wt; idx += nt * 256) {
      const int j = idx / wt, q = idx % wt;
      const int row = perm[j];
      const int key = row_key[row];  // >= 0: sorted positions below n_act are rows on resident adapters
      float v = 0.f;
      if (q < pv.rank[key]) v = sum_slices(Ts + (size_t)j * pv.max_rank + q, cs, n_chunks) * pv.scale[key];
      tb[(size_t)row * wt + q] = (uint16_t)f2bf(v);
    }
    return;
  }
  __shared__ __attribute__((aligned(16))) uint16_t tile[MLORA_MAX_RANK][kPrepCols];  // Up rows of the block's columns
  if (nseg == 0 && sidx == 0 && cc == 0 && tid == 0) *over = 0;
  if (sidx >= nseg) return;
  const int a = seg_adapter[sidx];
  const int rank = pv.rank[a], rp = rank_pad16(rank);
  const bool fits = kx > 0 || koff + rp <= upt_units;
  if (cc == 0 && tid == 0) {
    koff_out[a] = koff;
    if (sidx == nseg - 1) *over = fits ? 0 : 1;
  }
  if (!fits) return;
  const int c0 = cc * kPrepCols, ncol = min(kPrepCols, pv.dout - c0);
  const int32_t* upage = pv.up_page + ((size_t)a * pv.n_proj + proj) * pv.max_rank;
  // rank rows in: 8 columns per thread-chunk (one 16-byte load when the
  // row pieces are aligned and whole), rows past the rank are zero
  const bool vec = (pv.dout % 8) == 0 && (reinterpret_cast<uintptr_t>(pv.up) % 16) == 0;
  for (int idx = tid; idx < rp * (kPrepCols / 8); idx += 256) {
    const int q = idx / (kPrepCols / 8), cl = (idx % (kPrepCols / 8)) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (q < rank && cl < ncol) {
      const uint16_t* src = pv.up + (size_t)upage[q] * pv.dout + c0 + cl;
      if (vec && cl + 8 <= ncol) {
        v = *reinterpret_cast<const uint4*>(src);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = cl + e < ncol ? src[e] : 0u;
        v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
    }
    *reinterpret_cast<uint4*>(&tile[q][cl]) = v;
  }
  __syncthreads();
  // columns out, 8 ranks per 16-byte store: the block [dout][rp] at
  // koff * dout, or columns koff.. of the txw-wide rows
  const int stride = kx ? txw : rp;
  uint16_t* dst = kx ? upt + (size_t)c0 * txw + koff : upt + (size_t)koff * pv.dout + (size_t)c0 * rp;
  for (int idx = tid; idx < ncol * (rp / 8); idx += 256) {
    const int cl = idx / (rp / 8), q0 = (idx % (rp / 8)) * 8;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = tile[q0 + e][cl];
    *reinterpret_cast<uint4*>(dst + (size_t)cl * stride + q0) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  }
  if (kx && sidx == nseg - 1) {
    // zeros from the last adapter's columns up to Kx
    const int tail = (kx - total) / 8;
    for (int idx = tid; idx < ncol * tail; idx += 256) {
      const int cl = idx / tail, q0 = total + (idx % tail) * 8;
      *reinterpret_cast<uint4*>(upt + (size_t)(c0 + cl) * txw + q0) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

bool vec_ok(const PoolView& pv, const void* a, const void* b) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                      reinterpret_cast<uintptr_t>(pv.down) | reinterpret_cast<uintptr_t>(pv.up);
  return (pv.din % 8 == 0) && (pv.dout % 8 == 0) && (p % 16 == 0);
}

// The kernels walk items (and invalid rows) with grid-stride loops, so the
// grid only has to be large enough to fill the chip: at most one block per
// possible item, capped at 1024.
int item_grid(int n) {
  const int upper = MLORA_SEG_MAX_ITEMS(n);
  return upper < 1024 ? upper : 1024;
}

}  // namespace

bool shrink_uses_tiles(const PoolView& pv, int n, const void* X) {
  return n >= kShrinkTilesMinRows && pv.din % 32 == 0 && vec_ok(pv, X, X);
}

int shrink_tile_cap(const PoolView& pv, int n) {
  // tiles <= ceil(n_act / TILE_ROWS) + nseg, nseg <= min(n, max_adapters)
  return (n + MLORA_TILE_ROWS - 1) / MLORA_TILE_ROWS + (n < pv.max_adapters ? n : pv.max_adapters);
}

hipError_t launch_shrink(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, int n, float* T,
                         int n_chunks, int chunk_elems, hipStream_t stream) {
  if (shrink_uses_tiles(pv, n, X)) {
    const int cap = shrink_tile_cap(pv, n);
    const dim3 grid(cap < 4096 ? cap : 4096, n_chunks), block(64 * kTileWaves);
    MLORA_LAUNCH("shrink_tiles", shrink_tiles_kernel, grid, block, 0, stream, pv, proj, X, ws, n, T, chunk_elems);
    return launched();
  }
  const dim3 grid(item_grid(n), n_chunks), block(64);
  if (vec_ok(pv, X, X))
    MLORA_LAUNCH("shrink", (shrink_kernel<true>), grid, block, 0, stream, pv, proj, X, ws, n, T, chunk_elems);
  else
    MLORA_LAUNCH("shrink", (shrink_kernel<false>), grid, block, 0, stream, pv, proj, X, ws, n, T, chunk_elems);
  return launched();
}

hipError_t launch_shrink_rows(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, int n, float* T,
                              hipStream_t stream) {
  const dim3 grid(n < 1024 ? n : 1024), block(kRowThreads);
  const int32_t* row_key = ws + MLORA_SEG_ROWKEY(n);
  if (vec_ok(pv, X, X))
    MLORA_LAUNCH("shrink_rows", (shrink_rows_kernel<true>), grid, block, 0, stream, pv, proj, X, row_key, n, T);
  else
    MLORA_LAUNCH("shrink_rows", (shrink_rows_kernel<false>), grid, block, 0, stream, pv, proj, X, row_key, n, T);
  return launched();
}

hipError_t launch_expand(const PoolView& pv, int proj, const float* T, int n_chunks, const int32_t* ws, uint16_t* Y,
                         int n, hipStream_t stream) {
  const dim3 grid(item_grid(n), (pv.dout + 511) / 512), block(64);
  const int32_t* none = nullptr;
  if (vec_ok(pv, Y, Y))
    MLORA_LAUNCH("expand", (expand_kernel<true>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n, none);
  else
    MLORA_LAUNCH("expand", (expand_kernel<false>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n, none);
  return launched();
}

hipError_t launch_expand_over(const PoolView& pv, int proj, const float* T, int n_chunks, const int32_t* ws,
                              uint16_t* Y, int n, const int32_t* over, hipStream_t stream) {
  const dim3 grid(item_grid(n), (pv.dout + 511) / 512), block(64);
  if (vec_ok(pv, Y, Y))
    MLORA_LAUNCH("expand_over", (expand_kernel<true>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n, over);
  else
    MLORA_LAUNCH("expand_over", (expand_kernel<false>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n,
                 over);
  return launched();
}

hipError_t launch_fused(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, uint16_t* Y, int n,
                        hipStream_t stream) {
  if (n <= 0) return hipSuccess;  // (the fast form's first-item reads index sorted position min(b, n - 1))
  const dim3 grid(item_grid(n)), block(kFusedThreads);
  if (vec_ok(pv, X, Y) && pv.max_rank <= G && pv.din <= 8 * kFusedThreads && pv.dout <= 8 * kFusedThreads)
    MLORA_LAUNCH("fused", fused_fast_kernel, grid, block, 0, stream, pv, proj, X, ws, Y, n);
  else if (vec_ok(pv, X, Y))
    MLORA_LAUNCH("fused", (fused_kernel<true>), grid, block, 0, stream, pv, proj, X, ws, Y, n);
  else
    MLORA_LAUNCH("fused", (fused_kernel<false>), grid, block, 0, stream, pv, proj, X, ws, Y, n);
  return launched();
}

hipError_t launch_lora_prep(const PoolView& pv, int proj, const int32_t* ws, int n, const float* Ts, int n_chunks,
                            uint16_t* tb, int wt, int32_t* koff, uint16_t* upt, long upt_units, int32_t* over,
                            uint16_t* tx, int txw, int32_t* kx, hipStream_t stream) {
  if (tx != nullptr && (txw % 64 != 0 || txw > kMaxConcatRanks || (long)txw > upt_units))
    return hipErrorInvalidValue;
  const long total = (long)n * wt;
  const int nt = (int)((total + 255) / 256 < 1024 ? (total + 255) / 256 : 1024);
  const long segs = n < pv.max_adapters ? n : pv.max_adapters;  // segments of the batch, at most
  const long blocks = (nt > 0 ? nt : 1) + segs * ((pv.dout + kPrepCols - 1) / kPrepCols);
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  MLORA_LAUNCH("lora_prep", lora_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pv, proj, ws, n, Ts,
               n_chunks, tb, wt, nt > 0 ? nt : 1, koff, upt, upt_units, over, tx, txw, kx);
  return launched();
}

}  // namespace mlora
