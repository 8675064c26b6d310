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
template <bool VEC>
__global__ __launch_bounds__(64) void expand_kernel(PoolView pv, int proj, const float* __restrict__ T, int n_chunks,
                                                    const int32_t* __restrict__ ws, uint16_t* __restrict__ Y, int n) {
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
// fused: one 512-thread workgroup per item
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = 64 * kFusedWaves;

template <bool VEC>
__global__ __launch_bounds__(kFusedThreads) void fused_kernel(PoolView pv, int proj, const uint16_t* __restrict__ X,
                                                              const int32_t* __restrict__ ws,
                                                              uint16_t* __restrict__ Y, int n) {
  __shared__ float red[kFusedWaves][64];
  __shared__ float ts[R][MLORA_MAX_RANK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_items = ws[MLORA_SEG_NITEMS];
  const int n_bad = ws[MLORA_SEG_NBAD];
  const int32_t* perm = ws + MLORA_SEG_PERM(n);
  for (int it = blockIdx.x; it < n_items + n_bad; it += gridDim.x) {
    if (it < n_items) {
      const Item m = load_item(pv, ws, n, it);
      const size_t pt = ((size_t)m.adapter * pv.n_proj + proj) * pv.max_rank;
      const int32_t* dpage = pv.down_page + pt;
      const int32_t* upage = pv.up_page + pt;
      for (int g0 = 0; g0 < m.rank; g0 += G) {
        float acc[64];
#pragma unroll
        for (int v = 0; v < 64; ++v) acc[v] = 0.f;
        for (int k = tid * 8; k < pv.din; k += kFusedThreads * 8) {
          float x[R][8];
          load_rows<VEC>(X, perm, pv.din, m.j0, m.nr, k, x);
          shrink_step<VEC>(pv, dpage, g0, m.rank, x, k, acc);
        }
        red[wave][lane] = wave_reduce_scatter64(acc);
        __syncthreads();
        if (tid < 64) {
          float s = red[0][tid];
#pragma unroll
          for (int w = 1; w < kFusedWaves; ++w) s += red[w][tid];
          const int i = tid / G, q = g0 + tid % G;
          ts[i][q] = (q < m.rank) ? m.scale * s : 0.f;
        }
        __syncthreads();
      }
      for (int c = tid * 8; c < pv.dout; c += kFusedThreads * 8)
        expand_cols<VEC>(pv, upage, m.rank, ts, perm, m.j0, m.nr, c, Y);
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
  for (int k = blockIdx.x; k < n; k += gridDim.x) shrink_row_body<VEC>(pv, proj, X, row_key, k, T);
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

hipError_t launch_shrink(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, int n, float* T,
                         int n_chunks, int chunk_elems, hipStream_t stream) {
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
  if (vec_ok(pv, Y, Y))
    MLORA_LAUNCH("expand", (expand_kernel<true>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n);
  else
    MLORA_LAUNCH("expand", (expand_kernel<false>), grid, block, 0, stream, pv, proj, T, n_chunks, ws, Y, n);
  return launched();
}

hipError_t launch_fused(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, uint16_t* Y, int n,
                        hipStream_t stream) {
  const dim3 grid(item_grid(n)), block(kFusedThreads);
  if (vec_ok(pv, X, Y))
    MLORA_LAUNCH("fused", (fused_kernel<true>), grid, block, 0, stream, pv, proj, X, ws, Y, n);
  else
    MLORA_LAUNCH("fused", (fused_kernel<false>), grid, block, 0, stream, pv, proj, X, ws, Y, n);
  return launched();
}

}  // namespace mlora
