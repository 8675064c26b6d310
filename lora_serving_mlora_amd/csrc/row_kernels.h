// Device code shared by the per-row kernels: the per-row shrink body and the
// per-row low-rank term of 8 output columns.
#pragma once

#include "internal.h"

namespace mlora {
namespace {

// The low-rank term of row r at columns [c0, c0+8): sum_q t_q Up_a[c][q],
// with T [M][max_rank] holding t with the scale folded in.  Zero for a
// base-only row or a row past M, NaN for a row with an invalid id.  Ranks
// past the adapter's rank read its last column with weight 0, so each group
// of 8 page loads goes out at once.
template <bool VEC>
__device__ __forceinline__ void lora_delta8(const PoolView& pv, int proj, const int32_t* __restrict__ row_key,
                                            const float* __restrict__ T, int r, int M, int c0, int N,
                                            float (&acc8)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  const int key = (r < M && c0 < N) ? row_key[r] : -1;
  if (key >= 0) {
    const int rank = pv.rank[key];
    const int32_t* upage = pv.up_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank;
    const float* tr = T + (size_t)r * pv.max_rank;
    // t rows of 8 ranks as two 16-byte loads when they are aligned
    const bool tvec = (pv.max_rank & 7) == 0;
    // page indices and t are read without waiting for the rank: entries past
    // it fall back to the group's first page and weigh zero (a select, so an
    // unwritten t past the rank never reaches the sum)
    int q0 = 0;
    do {
      float u8[8][8], tv[8], tq[8];
      int pg[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) pg[q] = upage[min(q0 + q, pv.max_rank - 1)];
#pragma unroll
      for (int q = 1; q < 8; ++q) pg[q] = pg[q] < 0 ? pg[0] : pg[q];
#pragma unroll
      for (int q = 0; q < 8; ++q) load8<VEC>(pv.up + (size_t)pg[q] * pv.dout, c0, N, u8[q]);
      if (tvec) {
        // q0 + 7 < max_rank here: q0 < rank <= max_rank and both multiples of 8
        const float4 a = *reinterpret_cast<const float4*>(tr + q0);
        const float4 b = *reinterpret_cast<const float4*>(tr + q0 + 4);
        tv[0] = a.x; tv[1] = a.y; tv[2] = a.z; tv[3] = a.w;
        tv[4] = b.x; tv[5] = b.y; tv[6] = b.z; tv[7] = b.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) tv[q] = tr[min(q0 + q, pv.max_rank - 1)];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) tq[q] = (q0 + q < rank) ? tv[q] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = fmaf(tq[q], u8[q][e], acc8[e]);
      q0 += 8;
    } while (q0 < rank);
  } else if (key == -2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = __uint_as_float(0x7fc00000u);
  }
}

// The low-rank term of row r at columns [c0, c0+8) as lora_delta8, with the
// key, rank, scale and Up page ids taken from the row's descriptor: they
// are loaded together, so the Up loads wait for one dependent load.  Ranks
// go in rounds of QG (8 or 16): each round's QG page loads go out at once,
// so a rank-16 row takes one round with QG = 16; QG = 8 keeps the register
// count low where many waves must share each SIMD.  The sum over ranks runs
// in rank order either way.  PARTS: T holds tp partial slices
// [tp][M][max_rank] (K ranges of the shrink), summed here in slice order and
// then scaled; otherwise T [M][max_rank] holds t with the scale folded in.
template <bool VEC, bool PARTS = false, int QG = 8>
__device__ __forceinline__ void lora_delta8_desc(const PoolView& pv, const int32_t* __restrict__ desc,
                                                 const float* __restrict__ T, int r, int M, int c0, int N,
                                                 float (&acc8)[8], int tp = 1) {
  static_assert(QG == 8 || QG == 16, "rank rounds of 8 or 16");
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  if (r >= M || c0 >= N) return;
  const int words = row_desc_words(pv.max_rank);
  const int32_t* d = desc + (size_t)r * words;
  const int key = d[0];
  const int rank = d[1];
  const float tscale = PARTS ? __int_as_float(d[2]) : 1.f;
  if (!PARTS) tp = 1;
  if (key >= 0) {
    const float* tr = T + (size_t)r * pv.max_rank;
    const size_t tstride = (size_t)M * pv.max_rank;
    const bool tvec = (pv.max_rank & 7) == 0;  // rows of T 16-byte aligned
    int q0 = 0;
    do {
      float u8[QG][8], tv[QG], tq[QG];
#pragma unroll
      for (int q = 0; q < QG; ++q) load8<VEC>(pv.up + (size_t)d[4 + min(q0 + q, pv.max_rank - 1)] * pv.dout, c0, N,
                                              u8[q]);
      if (tvec && q0 + QG <= pv.max_rank) {
#pragma unroll
        for (int q = 0; q < QG; ++q) tv[q] = 0.f;
#pragma unroll 4
        for (int p = 0; p < tp; ++p) {
#pragma unroll
          for (int h = 0; h < QG / 4; ++h) {
            const float4 a = *reinterpret_cast<const float4*>(tr + p * tstride + q0 + 4 * h);
            tv[4 * h] += a.x; tv[4 * h + 1] += a.y; tv[4 * h + 2] += a.z; tv[4 * h + 3] += a.w;
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < QG; ++q) {
          const int qq = min(q0 + q, pv.max_rank - 1);
          tv[q] = tr[qq];
          for (int p = 1; p < tp; ++p) tv[q] += tr[p * tstride + qq];
        }
      }
#pragma unroll
      for (int q = 0; q < QG; ++q) tq[q] = (q0 + q < rank) ? tscale * tv[q] : 0.f;
#pragma unroll
      for (int q = 0; q < QG; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = fmaf(tq[q], u8[q][e], acc8[e]);
      q0 += QG;
    } while (q0 < rank);
  } else if (key == -2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = __uint_as_float(0x7fc00000u);
  }
}

// ---------------------------------------------------------------------------
// shrink_rows (decode): one 8-wave workgroup per row, rows read by index in
// original order; T[k][q] = s_a * (Down_a x_k)[q].  Each lane holds the
// partial dot products of its 8 din elements for a group of 16 ranks; a
// 4-step reduce-scatter (xor 32, 16, 8, 4: 16 values -> 1 per lane) plus two
// xor steps finishes each wave, then the 8 waves are summed in LDS in order.
// ---------------------------------------------------------------------------
constexpr int kRowWaves = 8;
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kRowGroup = 16;  // ranks per reduction group

// One row: out[q] = scale * (Down x)[q] for q < rank, with x the row at xr
// and Down reached through the page table dpage (rank >= 1).  Called by all
// 64 * NW threads of a workgroup (uniform control flow, block barriers
// inside); `out` may be global or LDS memory.
template <bool VEC, int NW = kRowWaves>
__device__ __forceinline__ void shrink_row_to(const PoolView& pv, const int32_t* __restrict__ dpage, int rank,
                                              float scale, const uint16_t* __restrict__ xr, float* __restrict__ out) {
  __shared__ float red[NW][kRowGroup];
  constexpr int G = kRowGroup;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The page table is read without waiting for the rank: entries past the
  // rank hold -1 and are replaced by the group's first page (their sums are
  // never stored), and the first group runs before the rank is known.
  int g0 = 0;
  do {
    int pg[G];
#pragma unroll
    for (int q = 0; q < G; ++q) pg[q] = dpage[min(g0 + q, pv.max_rank - 1)];
#pragma unroll
    for (int q = 1; q < G; ++q) pg[q] = pg[q] < 0 ? pg[0] : pg[q];
    float v[G];
#pragma unroll
    for (int q = 0; q < G; ++q) v[q] = 0.f;
    for (int kk = tid * 8; kk < pv.din; kk += 64 * NW * 8) {
      float x[8], d[G][8];
      load8<VEC>(xr, kk, pv.din, x);
#pragma unroll
      for (int q = 0; q < G; ++q) load8<VEC>(pv.down + (size_t)pg[q] * pv.din, kk, pv.din, d[q]);
#pragma unroll
      for (int q = 0; q < G; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q] = fmaf(d[q][e], x[e], v[q]);
    }
    // reduce-scatter 16 -> 1: after the steps lane l holds index l >> 2
#pragma unroll
    for (int m = 32, len = G / 2; m >= 4; m >>= 1, len >>= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < len; ++i) {
        const float send = upper ? v[i] : v[i + len];
        const float keep = upper ? v[i + len] : v[i];
        v[i] = keep + __shfl_xor(send, m, 64);
      }
    }
    float tot = v[0];
    tot += __shfl_xor(tot, 2, 64);
    tot += __shfl_xor(tot, 1, 64);
    if ((lane & 3) == 0) red[wave][lane >> 2] = tot;
    __syncthreads();
    if (tid < G && g0 + tid < rank) {
      float sum = red[0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][tid];
      out[g0 + tid] = scale * sum;
    }
    __syncthreads();
    g0 += G;
  } while (g0 < rank);
}

// Row k's descriptor (row_desc_words(max_rank) words at desc + k * words),
// one word per thread of the calling workgroup (which has at least that many
// threads); key is the row's key, uniform.
__device__ __forceinline__ void write_row_desc(const PoolView& pv, int proj, int key, int k,
                                               int32_t* __restrict__ desc) {
  const int tid = threadIdx.x;
  const int words = row_desc_words(pv.max_rank);
  if (tid < words) {
    int32_t v = 0;
    if (tid == 0) {
      v = key;
    } else if (key >= 0) {
      if (tid == 1) {
        v = pv.rank[key];
      } else if (tid == 2) {
        v = __float_as_int(pv.scale[key]);
      } else if (tid >= 4) {
        const int32_t* upage = pv.up_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank;
        const int32_t pg = upage[tid - 4];
        v = pg < 0 ? upage[0] : pg;
      }
    }
    desc[(size_t)k * words + tid] = v;
  }
}

// One row k: T[k][q] = s_a (Down_a x_k)[q] and the row's descriptor; called
// by all 64 * NW threads of a workgroup (uniform control flow, block
// barriers inside).
template <bool VEC, int NW = kRowWaves>
__device__ __forceinline__ void shrink_row_body(const PoolView& pv, int proj, const uint16_t* __restrict__ X,
                                                const int32_t* __restrict__ row_key, int k, float* __restrict__ T,
                                                int32_t* __restrict__ desc) {
  const int key = row_key[k];
  write_row_desc(pv, proj, key, k, desc);
  if (key < 0) return;  // base-only or invalid: no low-rank term
  shrink_row_to<VEC, NW>(pv, pv.down_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank, pv.rank[key],
                         pv.scale[key], X + (size_t)k * pv.din, T + (size_t)k * pv.max_rank);
}

}  // namespace
}  // namespace mlora
