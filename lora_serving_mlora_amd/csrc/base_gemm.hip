// Base GEMM of the multi-LoRA linear: Y = X W0^T for the whole batch at once
// (the shared-base step of the M031 card, section 02; the airsota card's
// trade-off item 2 notes this product runs on the matrix cores).
//
// bf16 operands, fp32 accumulation on CDNA4 MFMA, bf16 (RNE) output.  Both
// operands are K-contiguous ("NT"), which is the natural MFMA operand form:
// every lane feeds 8 consecutive K elements (one 16-byte load) of one row.
//
// Two kernels:
//  * gemm_skinny - decode batches (M <= 64).  The product is bound by
//    streaming W0 from HBM, so each workgroup owns 16 output columns and all
//    rows; its 8 waves split K, each lane loads its MFMA operands straight
//    from global memory (no LDS staging: every W0 byte is used once), and the
//    8 partial 16x16 tiles per row block are summed in LDS in a fixed order.
//  * gemm_tiled  - larger batches.  128x128 output tile per workgroup of 4
//    waves (2x2, 64x64 each = 2x2 MFMA 32x32x16 tiles), K in steps of 64
//    staged through LDS with a register-staged double buffer; LDS rows are
//    XOR-swizzled in 16-byte chunks so that the 128-bit fragment reads of
//    sixteen consecutive lanes hit sixteen different bank groups (no bank
//    conflicts).
#include <stdlib.h>

#include "internal.h"
#include "row_kernels.h"
#include "seg_device.h"

namespace mlora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive bf16 of a row as one 16-byte word; zero past `limit`.
// VEC: row base and k are 16-byte aligned, so a full chunk is one load.
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ row, int k, int limit) {
  if (VEC && k + 8 <= limit) return *reinterpret_cast<const uint4*>(row + k);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = (k + 2 * e < limit) ? row[k + 2 * e] : 0u;
    const uint32_t hi = (k + 2 * e + 1 < limit) ? row[k + 2 * e + 1] : 0u;
    w[e] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// skinny: M <= 16*MB rows, 16 columns per workgroup, K split over the waves
//
// Rows past M and columns past N read a clamped (valid) row instead: MFMA
// output (i, j) depends only on A row i and B column j, and those outputs are
// never stored.  So the main loop has no bounds tests at all and every load
// of an unrolled group is in flight at once; only a K tail that does not
// fill a whole 32-wide step takes element loads.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;

template <int MB>
__device__ __forceinline__ void skinny_step(const uint16_t* __restrict__ wrow, const uint16_t* const (&xrow)[MB],
                                            int k, floatx4 (&acc)[MB]) {
  const uint4 b = *reinterpret_cast<const uint4*>(wrow + k);
  uint4 a[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const uint4*>(xrow[mb] + k);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[mb]), as_bf16x8(b), acc[mb], 0, 0, 0);
}

// The K loop of one skinny workgroup: wave `wave` of kSkinnyWaves takes the
// 32-wide K steps wave, wave + 8, ...; acc[mb] is its partial 16x16 tile.
template <int MB, bool VEC>
__device__ __forceinline__ void skinny_kloop(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, int M,
                                             int K, int N, int n0, int lane, int wave, floatx4 (&acc)[MB]) {
  const int kl = (lane >> 4) * 8;  // this lane's K offset inside a 32-wide step
  const uint16_t* wrow = W + (size_t)min(n0 + (lane & 15), N - 1) * K + kl;
  const uint16_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xrow[mb] = X + (size_t)min(mb * 16 + (lane & 15), M - 1) * K + kl;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Each wave owns a contiguous range of 32-wide K steps.  In batches of 16
  // steps, all 16 W0 loads of the batch are issued at once (the HBM stream:
  // one round trip per batch instead of one per step), then the X fragments
  // (L2-resident, tiny) follow in groups of 4 steps, the next group issued
  // before the MFMAs of the current one.
  const int nfull = VEC ? K / 32 : 0;  // steps whose 32 K values all exist
  const int per = (nfull + kSkinnyWaves - 1) / kSkinnyWaves;
  const int s_beg = min(nfull, wave * per), s_end = min(nfull, s_beg + per);
  int s = VEC ? s_beg : wave;  // without VEC every step is a tail step, shared round-robin
  if (VEC) {
    for (; s + 16 <= s_end; s += 16) {
      uint4 wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) wv[j] = *reinterpret_cast<const uint4*>(wrow + (s + j) * 32);
      uint4 xa[2][4][MB];
      auto xload = [&](int g, uint4 (&x)[4][MB]) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) x[u][mb] = *reinterpret_cast<const uint4*>(xrow[mb] + (s + 4 * g + u) * 32);
      };
      xload(0, xa[0]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g + 1 < 4) xload(g + 1, xa[(g + 1) & 1]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[g & 1][u][mb]), as_bf16x8(wv[4 * g + u]),
                                                              acc[mb], 0, 0, 0);
      }
    }
    for (; s < s_end; ++s) skinny_step<MB>(wrow, xrow, s * 32, acc);
    s = nfull + wave;  // the K tail below is shared round-robin
  }
  // K tail (and every step when rows are not 16-byte aligned): element loads
  const int nsteps = (K + 31) / 32;
  for (; s < nsteps; s += kSkinnyWaves) {
    const int k = s * 32;
    const int lim = K - k - kl;  // valid elements of this lane's chunk
    const uint4 b = load_chunk<false>(wrow + k, 0, lim);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint4 a = load_chunk<false>(xrow[mb] + k, 0, lim);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc[mb], 0, 0, 0);
    }
  }
}

template <int MB, bool VEC>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ W,
                                                                  uint16_t* __restrict__ Y, int M, int K, int N) {
  __shared__ floatx4 red[kSkinnyWaves][MB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  floatx4 acc[MB];
  skinny_kloop<MB, VEC>(X, W, M, K, N, n0, lane, wave, acc);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  // output tile element (row (lane/16)*4 + v, column lane%16) of row block mb;
  // thread t sums the waves' partials in wave order
  for (int t = threadIdx.x; t < MB * 64; t += 64 * kSkinnyWaves) {
    const int mb = t >> 6, l = t & 63;
    floatx4 sum = red[0][mb][l];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) sum += red[w][mb][l];
    const int c = n0 + (l & 15);
    if (c < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = mb * 16 + (l >> 4) * 4 + v;
        if (r < M) Y[(size_t)r * N + c] = (uint16_t)f2bf(sum[v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// skinny + low-rank expand (decode): the 8 GEMM waves stream W0 while 2 more
// waves of the same workgroup compute, for the workgroup's 16 columns, every
// row's delta sum_q T[r][q] Up_a[c][q] (T = s * Down x per original row, from
// the per-row shrink); the delta is added when the partial tiles are summed,
// so Y is written once and the branch costs no extra pass over Y.
// ---------------------------------------------------------------------------
constexpr int kLoraWaves = 2;

template <int MB, bool VEC>
__global__ __launch_bounds__(64 * (kSkinnyWaves + kLoraWaves)) void gemm_skinny_lora(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int K, int N,
    PoolView pv, int proj, const int32_t* __restrict__ row_key, const float* __restrict__ T) {
  __shared__ floatx4 red[kSkinnyWaves][MB][64];
  __shared__ float delta[MB * 16][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  if (wave < kSkinnyWaves) {
    floatx4 acc[MB];
    skinny_kloop<MB, VEC>(X, W, M, K, N, n0, lane, wave, acc);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  } else {
    // task (row r, 8-column half h) per thread
    const int u = threadIdx.x - 64 * kSkinnyWaves;
    for (int task = u; task < MB * 16 * 2; task += 64 * kLoraWaves) {
      const int r = task >> 1, h = task & 1;
      float acc8[8];
      lora_delta8<VEC>(pv, proj, row_key, T, r, M, n0 + 8 * h, N, acc8);
#pragma unroll
      for (int e = 0; e < 8; ++e) delta[r][8 * h + e] = acc8[e];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < MB * 64; t += 64 * (kSkinnyWaves + kLoraWaves)) {
    const int mb = t >> 6, l = t & 63;
    floatx4 sum = red[0][mb][l];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) sum += red[w][mb][l];
    const int c = n0 + (l & 15);
    if (c < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = mb * 16 + (l >> 4) * 4 + v;
        if (r < M) Y[(size_t)r * N + c] = (uint16_t)f2bf(sum[v] + delta[r][l & 15]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// ksplit: medium batches (65 .. 1024 rows).  A 128 x 32 output tile per
// workgroup, so even a 256-row batch launches 256+ workgroups; its 4 waves
// split K (steps of 16, interleaved), each computing the whole tile over its
// share with MFMA 32x32x16 on operands loaded straight into registers, two
// groups of 4 steps in flight; the 4 partial tiles are summed in LDS in a
// fixed order.  Rows past M / columns past N read clamped rows (never
// stored); a K tail shorter than a 16-wide step takes element loads.
// ---------------------------------------------------------------------------
constexpr int kKsWaves = 4;
constexpr int kKsLoraWaves = 8;  // one (row, 8-column) task of the 128 x 32 tile per thread
constexpr int KS_MB = 4;         // 32-row blocks per tile (128 rows)

template <bool VEC, bool LORA>
__global__ __launch_bounds__(64 * (kKsWaves + (LORA ? kKsLoraWaves : 0))) void gemm_ksplit(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int K, int N,
    PoolView pv, int proj, const int32_t* __restrict__ row_key, const float* __restrict__ T) {
  __shared__ float red[kKsWaves - 1][KS_MB][16][64];  // partials of waves 1..3, [mb][v][lane]
  __shared__ float delta[LORA ? 32 * KS_MB : 1][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * (32 * KS_MB);
  if (LORA && wave >= kKsWaves) {
    // the tile's low-rank term: task (row, 8-column quarter) per thread
    const int u = threadIdx.x - 64 * kKsWaves;
    for (int task = u; task < 32 * KS_MB * 4; task += 64 * kKsLoraWaves) {
      const int r = task >> 2, h = task & 3;
      float acc8[8];
      lora_delta8<VEC>(pv, proj, row_key, T, m0 + r, M, n0 + 8 * h, N, acc8);
#pragma unroll
      for (int e = 0; e < 8; ++e) delta[r][8 * h + e] = acc8[e];
    }
    __syncthreads();
    return;
  }
  const int kl = (lane >> 5) * 8;
  const uint16_t* wrow = W + (size_t)min(n0 + (lane & 31), N - 1) * K + kl;
  const uint16_t* xrow[KS_MB];
#pragma unroll
  for (int mb = 0; mb < KS_MB; ++mb) xrow[mb] = X + (size_t)min(m0 + mb * 32 + (lane & 31), M - 1) * K + kl;
  floatx16 acc[KS_MB];
#pragma unroll
  for (int mb = 0; mb < KS_MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mb][v] = 0.f;

  // Each wave owns a contiguous range of 16-wide K steps.  In batches of 16
  // steps, the 16 W0 loads of the batch go out at once (the HBM stream);
  // the X fragments (4 per step, L2-resident) follow in groups of 2 steps,
  // the next group issued before the MFMAs of the current one.
  const int nfull = VEC ? K / 16 : 0;
  const int per = (nfull + kKsWaves - 1) / kKsWaves;
  const int s_beg = min(nfull, wave * per), s_end = min(nfull, s_beg + per);
  int s = VEC ? s_beg : wave;  // without VEC every step is a tail step, shared round-robin
  if (VEC) {
    for (; s + 16 <= s_end; s += 16) {
      uint4 wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) wv[j] = *reinterpret_cast<const uint4*>(wrow + (s + j) * 16);
      uint4 xa[2][2][KS_MB];
      auto xload = [&](int g, uint4 (&x)[2][KS_MB]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mb = 0; mb < KS_MB; ++mb) x[u][mb] = *reinterpret_cast<const uint4*>(xrow[mb] + (s + 2 * g + u) * 16);
      };
      xload(0, xa[0]);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g + 1 < 8) xload(g + 1, xa[(g + 1) & 1]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mb = 0; mb < KS_MB; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xa[g & 1][u][mb]), as_bf16x8(wv[2 * g + u]),
                                                              acc[mb], 0, 0, 0);
      }
    }
    for (; s < s_end; ++s) {
      const int k = s * 16;
      const uint4 b = *reinterpret_cast<const uint4*>(wrow + k);
#pragma unroll
      for (int mb = 0; mb < KS_MB; ++mb) {
        const uint4 a = *reinterpret_cast<const uint4*>(xrow[mb] + k);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[mb], 0, 0, 0);
      }
    }
    s = nfull + wave;  // the K tail below is shared round-robin
  }
  const int nsteps = (K + 15) / 16;
  for (; s < nsteps; s += kKsWaves) {
    const int k = s * 16;
    const int lim = K - k - kl;
    const uint4 b = load_chunk<false>(wrow + k, 0, lim);
#pragma unroll
    for (int mb = 0; mb < KS_MB; ++mb) {
      const uint4 a = load_chunk<false>(xrow[mb] + k, 0, lim);
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[mb], 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < KS_MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[wave - 1][mb][v][lane] = acc[mb][v];
  }
  __syncthreads();
  if (wave == 0) {
    // C layout of a 32x32 tile: lane l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4
    const int c = n0 + (lane & 31);
#pragma unroll
    for (int mb = 0; mb < KS_MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float sum = acc[mb][v];
#pragma unroll
        for (int w = 0; w < kKsWaves - 1; ++w) sum += red[w][mb][v][lane];
        const int rl = mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int r = m0 + rl;
        if (LORA) sum += delta[rl][lane & 31];
        if (r < M && c < N) Y[(size_t)r * N + c] = (uint16_t)f2bf(sum);
      }
  }
}

// ---------------------------------------------------------------------------
// tiled: 128 x 128 x 64 tiles, 4 waves, MFMA 32x32x16
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kTiledThreads = 256;
constexpr int kChunksPerRow = BK / 8;                          // 16-byte chunks per LDS row
constexpr int kLoadsA = BM * kChunksPerRow / kTiledThreads;    // 4
constexpr int kLoadsB = BN * kChunksPerRow / kTiledThreads;    // 4

// 128-byte LDS rows, chunks XOR-swizzled by (row >> 1) & 7: a 128-bit LDS
// read is served 16 lanes (256 bytes) per cycle, and the 16 consecutive
// rows of a fragment read then land in 16 distinct 16-byte slots of the
// 256-byte window (row & 7 would put rows r and r + 8 on the same banks).
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// PART: split-K form - workgroup z covers K tiles [z*kt_per, (z+1)*kt_per)
// and stores its fp32 partial tile to part[z][M][N] (summed by finish_part).
template <bool VEC, bool PART = false>
__global__ __launch_bounds__(kTiledThreads) void gemm_tiled(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ W,
                                                            uint16_t* __restrict__ Y, int M, int K, int N,
                                                            float* __restrict__ part = nullptr, int kt_per = 0) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // global chunk assignment: chunk c = tid + i*256 -> (row c/8, kchunk c%8).
  // Rows past M / N read a clamped row (their outputs are never stored), so a
  // K tile that lies wholly inside K is loaded with no tests at all.
  uint4 ra[kLoadsA], rb[kLoadsB];
  const uint16_t* pa[kLoadsA];
  const uint16_t* pb[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int c = tid + i * kTiledThreads;
    pa[i] = X + (size_t)min(m0 + (c >> 3), M - 1) * K + (c & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int c = tid + i * kTiledThreads;
    pb[i] = W + (size_t)min(n0 + (c >> 3), N - 1) * K + (c & 7) * 8;
  }
  const int nk_full = VEC ? K / BK : 0;
  auto gload = [&](int kt) {
    const int kbase = kt * BK;
    if (kt < nk_full) {
#pragma unroll
      for (int i = 0; i < kLoadsA; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + kbase);
#pragma unroll
      for (int i = 0; i < kLoadsB; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + kbase);
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsA; ++i) {
        const int c = tid + i * kTiledThreads;
        ra[i] = load_chunk<false>(pa[i] + kbase, 0, K - kbase - (c & 7) * 8);
      }
#pragma unroll
      for (int i = 0; i < kLoadsB; ++i) {
        const int c = tid + i * kTiledThreads;
        rb[i] = load_chunk<false>(pb[i] + kbase, 0, K - kbase - (c & 7) * 8);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int c = tid + i * kTiledThreads;
      *reinterpret_cast<uint4*>(&As[buf][swz(c >> 3, c & 7)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
      const int c = tid + i * kTiledThreads;
      *reinterpret_cast<uint4*>(&Bs[buf][swz(c >> 3, c & 7)]) = rb[i];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk_all = (K + BK - 1) / BK;
  const int kt0 = PART ? blockIdx.z * kt_per : 0;
  const int nk = PART ? min(nk_all, kt0 + kt_per) : nk_all;
  gload(kt0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 31;        // fragment row (A) / column (B) inside a 32-wide tile
  const int fk = lane >> 5;        // which 8-wide half of a 16-wide k step
  for (int kt = kt0; kt < nk; ++kt) {
    const int buf = (kt - kt0) & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kc = kk * 2 + fk;
      uint4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + fr;
        fa[i] = *reinterpret_cast<const uint4*>(&As[buf][swz(r, kc)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + fr;
        fb[j] = *reinterpret_cast<const uint4*>(&Bs[buf][swz(r, kc)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 32x32 tile: lane l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = n0 + wn * 64 + j * 32 + (lane & 31);
      if (c >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < M) {
          if (PART)
            part[((size_t)blockIdx.z * M + r) * N + c] = acc[i][j][v];
          else
            Y[(size_t)r * N + c] = (uint16_t)f2bf(acc[i][j][v]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// ring: TM x TN output tiles (256 x 256 for large batches, 128 x 128 with
// split-K for medium ones), 4 waves of (TM/2) x (TN/2), MFMA 32x32x16.  K
// advances in 32-deep tiles through an LDS ring of NS = 4 stages (32 KiB
// each for 256 x 256, 16 KiB for 128 x 128, so two medium workgroups fit a
// CU).  Tiles are moved global -> LDS
// by LDS DMA (buffer_load ... lds: each lane's 16 bytes land at a fixed LDS
// slot, so the XOR swizzle is applied by choosing which global chunk each
// lane fetches), and the DMA of tile kt+NS-1 is issued while tile kt is
// consumed, so NS-1 tiles are always in flight.  Inside a stage the
// fragment reads of the second 16-deep step overlap the MFMAs of the first.
// Workgroups are mapped to tiles so that the tiles dispatched to one XCD
// (block ids congruent mod 8) are contiguous: along N within one or two
// bands of X rows for large products (they share X rows in that XCD's L2),
// along M within a W column block for split-K medium ones (W is then read
// from HBM once and X, a few MiB, is what each XCD re-reads).  Needs K a
// multiple of 32 * NS (per split) and 16-byte aligned rows; rows past M or
// N read zeros (buffer bounds).
// ---------------------------------------------------------------------------
constexpr int kRingKAlign = 128;  // K (per split) must be a multiple of two 64-deep stages
constexpr int kRingThreads = 256;
constexpr int kGroupM = 4;  // row bands per tile group (large products)

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those make every wave wait for all of its outstanding DMAs (vmcnt(0)),
// which would expose the latency the stage ring is there to hide.  Each
// wave waits for exactly the DMA it needs before arriving (explicit
// s_waitcnt), and LDS is coherent inside the CU; the empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate for "vmcnt <= v" (expcnt and lgkmcnt not waited)
constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

struct RingCtx {
  __amdgpu_buffer_rsrc_t rsa, rsb;
  int voff, voff64, row_bytes, wave, wm, wn, fr, fk;
  // rank-concatenated stages (kt >= kmain): Tx and Ux rows, xrow_bytes long
  __amdgpu_buffer_rsrc_t rsx, rsu;
  int voffx, xrow_bytes, kmain;
};

// ---------------------------------------------------------------------------
// ring64: the same pipelined ring with 64-deep stages.  A DMA instruction then
// covers 8 tile rows x 128 contiguous bytes (8 whole cache lines) instead of
// 16 rows x 64 bytes (16 half lines): the per-CU memory pipe handles cache
// lines at a fixed rate, so the same bytes reach LDS in about half the time.
// LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by (row >> 1) & 7,
// so the 16 lanes of a fragment read (16 consecutive rows, one logical
// chunk) cover all 16 slots of a 256-byte window.  Large products use
// 256 x 128 tiles with 3 stages (48 KiB each), medium split-K ones 128 x 128
// tiles with 4 stages (32 KiB each).
// ---------------------------------------------------------------------------
constexpr int GBK64 = 64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__shared__ __attribute__((aligned(16))) uint16_t m64_a0[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_a1[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_a2[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_a3[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_b0[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_b1[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_b2[128 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t m64_b3[128 * GBK64];

// LDS element offset of 16-byte chunk `chunk` (0..7) of 128-byte row `row`
__device__ __forceinline__ int swz8(int row, int chunk) { return row * GBK64 + ((chunk ^ ((row >> 1) & 7)) << 3); }

// DMA of 64-deep K tile kt into (da, db): instruction j of this wave covers
// tile rows 8i..8i+7, i = wave + 4j; lane L fills row L >> 3 of the group,
// physical chunk L & 7 (voff64: the logical chunk that slot holds, which
// depends on the row's parity group, the same for all i of a wave).
// EXT: tiles kt >= kmain come from the rank-concatenated operands (tile
// kt - kmain of Tx and Ux), chosen by selects, not a branch, so the DMAs stay
// in the block the callers' schedule interleaves with the MFMAs.
template <int TM, int TN, bool EXT = false>
__device__ __forceinline__ void ring64_issue(const RingCtx& c, uint16_t* __restrict__ da, uint16_t* __restrict__ db,
                                             int kt) {
  __amdgpu_buffer_rsrc_t ra = c.rsa, rb = c.rsb;
  int voff = c.voff64, rbytes = c.row_bytes, ko = kt * GBK64 * 2;
  if constexpr (EXT) {
    const bool x = kt >= c.kmain;
    ra = x ? c.rsx : c.rsa;
    rb = x ? c.rsu : c.rsb;
    voff = x ? c.voffx : c.voff64;
    rbytes = x ? c.xrow_bytes : c.row_bytes;
    ko = (x ? kt - c.kmain : kt) * GBK64 * 2;
  }
#pragma unroll
  for (int j = 0; j < TM / 32; ++j) {
    const int i = c.wave + 4 * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, da + i * 8 * GBK64, 16, voff, i * 8 * rbytes + ko, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < TN / 32; ++j) {
    const int i = c.wave + 4 * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, db + i * 8 * GBK64, 16, voff, i * 8 * rbytes + ko, 0, 0);
  }
}

// fragments of one 64-deep stage: four 16-deep quarters
template <int TM, int TN>
struct Ring64Frags {
  uint4 a[4][TM / 64], b[4][TN / 64];
};

template <int TM, int TN>
__device__ __forceinline__ void ring64_read(const RingCtx& c, const uint16_t* __restrict__ ra,
                                            const uint16_t* __restrict__ rb, Ring64Frags<TM, TN>& f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int i = 0; i < TM / 64; ++i)
      f.a[q][i] = *reinterpret_cast<const uint4*>(ra + swz8(c.wm * (TM / 2) + i * 32 + c.fr, 2 * q + c.fk));
#pragma unroll
    for (int j = 0; j < TN / 64; ++j)
      f.b[q][j] = *reinterpret_cast<const uint4*>(rb + swz8(c.wn * (TN / 2) + j * 32 + c.fr, 2 * q + c.fk));
  }
}

// Step k of an NS-stage ring: MFMAs of stage k on cf, reads of stage k+1
// (ra, rb) into nf, DMA of stage k+NS into the buffer of stage k (da, db);
// then wait until stage k+2 has landed and the own reads are done, and sync
template <int TM, int TN, int NS>
__device__ __forceinline__ void ring64_step(const RingCtx& c, const uint16_t* __restrict__ ra,
                                            const uint16_t* __restrict__ rb, uint16_t* __restrict__ da,
                                            uint16_t* __restrict__ db, int kt, int kend,
                                            const Ring64Frags<TM, TN>& cf, Ring64Frags<TM, TN>& nf,
                                            floatx16 (&acc)[TM / 64][TN / 64]) {
  constexpr int MI = TM / 64, NJ = TN / 64;
  constexpr int kDma = (TM + TN) / 32, kReads = 4 * (MI + NJ), kMfma = 4 * MI * NJ;
  static_assert(kDma <= kReads && kMfma >= kReads, "one DMA per read group, at least one MFMA per group");
  ring64_issue<TM, TN>(c, da, db, min(kt + NS, kend - 1));
  ring64_read<TM, TN>(c, ra, rb, nf);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cf.b[q][j]), as_bf16x8(cf.a[q][i]), acc[i][j], 0,
                                                            0, 0);
#pragma unroll
  for (int r = 0; r < kReads; ++r) {
    if (r < kDma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                // one fragment read
    if (r < kMfma % kReads)
      __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kReads + 1, 0);  // MFMAs
    else
      __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kReads, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kDma) & ~(15 << 8));  // + lgkmcnt(0)
  ring_barrier();
}

// K tiles [kt0, kend) through 4 stages (any count >= 1; later steps of the
// last round skipped by nested uniform branches)
template <int TM, int TN>
__device__ __forceinline__ void ring64_loop4(const RingCtx& c, uint16_t* __restrict__ a0, uint16_t* __restrict__ a1,
                                             uint16_t* __restrict__ a2, uint16_t* __restrict__ a3,
                                             uint16_t* __restrict__ b0, uint16_t* __restrict__ b1,
                                             uint16_t* __restrict__ b2, uint16_t* __restrict__ b3, int kt0, int kend,
                                             floatx16 (&acc)[TM / 64][TN / 64]) {
  constexpr int n = (TM + TN) / 32;
  ring64_issue<TM, TN>(c, a0, b0, kt0);
  ring64_issue<TM, TN>(c, a1, b1, min(kt0 + 1, kend - 1));
  ring64_issue<TM, TN>(c, a2, b2, min(kt0 + 2, kend - 1));
  ring64_issue<TM, TN>(c, a3, b3, min(kt0 + 3, kend - 1));
  Ring64Frags<TM, TN> f0, f1;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * n));  // stage kt0 has landed
  ring_barrier();
  ring64_read<TM, TN>(c, a0, b0, f0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * n) & ~(15 << 8));  // stage kt0+1 landed, own reads done
  ring_barrier();
  for (int kt = kt0; kt < kend; kt += 4) {
    ring64_step<TM, TN, 4>(c, a1, b1, a0, b0, kt, kend, f0, f1, acc);
    if (kt + 1 < kend) {
      ring64_step<TM, TN, 4>(c, a2, b2, a1, b1, kt + 1, kend, f1, f0, acc);
      if (kt + 2 < kend) {
        ring64_step<TM, TN, 4>(c, a3, b3, a2, b2, kt + 2, kend, f0, f1, acc);
        if (kt + 3 < kend) ring64_step<TM, TN, 4>(c, a0, b0, a3, b3, kt + 3, kend, f1, f0, acc);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// 256 x 256 tiles with 64-deep stages: two 64 KiB stages fill the LDS, so the
// ring is double-buffered and pipelined at half-stage granularity (two
// 16-deep quarters per register set): the MFMAs of one half run while the
// other half, or the first half of the next stage, is read.  One barrier
// per stage, after the second half has been read: every wave is then done
// with the stage's buffer, which receives the DMA of stage k+2, and stage
// k+1 has landed (the only DMA in flight was waited for).
__shared__ __attribute__((aligned(16))) uint16_t h64_a0[256 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t h64_a1[256 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t h64_b0[256 * GBK64];
__shared__ __attribute__((aligned(16))) uint16_t h64_b1[256 * GBK64];

template <int TM, int TN>
struct RingHalf {
  uint4 a[2][TM / 64], b[2][TN / 64];
};

template <int TM, int TN>
__device__ __forceinline__ void ring64_read_half(const RingCtx& c, const uint16_t* __restrict__ ra,
                                                 const uint16_t* __restrict__ rb, int h, RingHalf<TM, TN>& f) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int i = 0; i < TM / 64; ++i)
      f.a[q][i] = *reinterpret_cast<const uint4*>(ra + swz8(c.wm * (TM / 2) + i * 32 + c.fr, 4 * h + 2 * q + c.fk));
#pragma unroll
    for (int j = 0; j < TN / 64; ++j)
      f.b[q][j] = *reinterpret_cast<const uint4*>(rb + swz8(c.wn * (TN / 2) + j * 32 + c.fr, 4 * h + 2 * q + c.fk));
  }
}

template <int TM, int TN>
__device__ __forceinline__ void ring64_mfma_half(const RingHalf<TM, TN>& f, floatx16 (&acc)[TM / 64][TN / 64]) {
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < TM / 64; ++i)
#pragma unroll
      for (int j = 0; j < TN / 64; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f.b[q][j]), as_bf16x8(f.a[q][i]), acc[i][j], 0, 0, 0);
}

// stage k in (ca, cb), the other buffer (oa, ob) holds stage k+1 (landed
// before this call); h0 holds the first half of stage k
template <int TM, int TN, bool EXT>
__device__ __forceinline__ void ring64x2_stage(const RingCtx& c, uint16_t* __restrict__ ca, uint16_t* __restrict__ cb,
                                               const uint16_t* __restrict__ oa, const uint16_t* __restrict__ ob,
                                               int kt, int kend, RingHalf<TM, TN>& h0, RingHalf<TM, TN>& h1,
                                               floatx16 (&acc)[TM / 64][TN / 64]) {
  constexpr int MI = TM / 64, NJ = TN / 64;
  constexpr int kReads = 2 * (MI + NJ), kMfma = 2 * MI * NJ, kDma = (TM + TN) / 32;
  static_assert(kDma <= kReads && kMfma % kReads == 0, "schedule pattern");
  // first half: MFMAs on h0, reads of the second half into h1
  ring64_read_half<TM, TN>(c, ca, cb, 1, h1);
  ring64_mfma_half<TM, TN>(h0, acc);
#pragma unroll
  for (int r = 0; r < kReads; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kReads, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // every wave is done with this buffer; stage k+1 (the one DMA in flight) has landed
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~(15 << 8));
  ring_barrier();
  // second half: DMA of stage k+2 into this buffer, MFMAs on h1, reads of
  // the next stage's first half into h0
  ring64_issue<TM, TN, EXT>(c, ca, cb, min(kt + 2, kend - 1));
  ring64_read_half<TM, TN>(c, oa, ob, 0, h0);
  ring64_mfma_half<TM, TN>(h1, acc);
#pragma unroll
  for (int r = 0; r < kReads; ++r) {
    if (r < kDma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kReads, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// EXT: K tiles [kt0, c.kmain) of X and W, then [c.kmain, kend) of the
// rank-concatenated operands (kend - kt0 may then be odd; c.kmain - kt0 >= 2)
template <int TM, int TN, bool EXT = false>
__device__ __forceinline__ void ring64x2_loop(const RingCtx& c, uint16_t* __restrict__ a0, uint16_t* __restrict__ a1,
                                              uint16_t* __restrict__ b0, uint16_t* __restrict__ b1, int kt0, int kend,
                                              floatx16 (&acc)[TM / 64][TN / 64]) {
  constexpr int n = (TM + TN) / 32;
  ring64_issue<TM, TN>(c, a0, b0, kt0);
  ring64_issue<TM, TN>(c, a1, b1, min(kt0 + 1, (EXT ? c.kmain : kend) - 1));
  RingHalf<TM, TN> h0, h1;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(n));  // stage kt0 has landed
  ring_barrier();
  ring64_read_half<TM, TN>(c, a0, b0, 0, h0);
  for (int kt = kt0; kt < kend; kt += 2) {  // (without EXT kend - kt0 is even: K is a multiple of 128)
    ring64x2_stage<TM, TN, EXT>(c, a0, b0, a1, b1, kt, kend, h0, h1, acc);
    if (!EXT || kt + 1 < kend) ring64x2_stage<TM, TN, EXT>(c, a1, b1, a0, b0, kt + 1, kend, h0, h1, acc);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// The low-rank term added in the GEMM's registers (prefill): for every row
// of the tile on a resident adapter a, acc[row][col] += sum_q t[row][q] *
// Up_a[col][q].  Rows of one tile carry different adapters, so each wave
// walks the distinct adapters among its own rows (smallest first, a wave
// min-reduction per step) and, per 16 ranks, runs one more 32x32x16 MFMA
// step per accumulator with A = t of the rows on that adapter (zero for the
// others) and B = the adapter's Up columns.  Both operands are prepared per
// batch in MFMA-friendly form (lora_prep): t as bf16 [M][wt] per original
// row, Up as a [dout][r_pad] block per adapter (ranks contiguous), so each
// fragment is one 16-byte load.  The expand then costs a few percent more
// MFMA work instead of a read-modify-write of all of Y.
// A uniform read of pool metadata that the kernel never writes, through the
// constant address space, so it becomes a scalar load (it does not wait on
// the vector loads in flight).
__device__ __forceinline__ int32_t uniform_load(const int32_t* p, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// The wave owns MI x NJ blocks of 32 x 32 outputs: rows wr + 32 i, columns
// wc + 32 j (wr, wc absolute).
template <int MI, int NJ>
__device__ __forceinline__ void ring_lora_epilogue(int wr, int wc, int M, int N, const PoolView& pv,
                                                   const int32_t* __restrict__ row_key, const LoraOperands& lo,
                                                   floatx16 (&acc)[MI][NJ], int (&key)[MI]) {
  // kBad: the pseudo adapter of rows with an invalid id, walked after the
  // real ones; its step multiplies NaN into those rows' accumulators
  constexpr int kNone = 0x7fffffff, kBad = 0x7ffffffe, kBatch = 4;
  const int lane = threadIdx.x & 63, half = lane >> 5;
  int pend[MI];
  int trow[MI];  // element offset of the lane's t piece (rows past M read row M-1: never stored)
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wr + i * 32 + (lane & 31);
    key[i] = r < M ? row_key[r] : -1;
    if (key[i] == -2) key[i] = kBad;
    pend[i] = (key[i] >= 0) ? key[i] : kNone;
    trow[i] = min(r, M - 1) * lo.wt + 8 * half;
  }
  int col[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) col[j] = min(wc + j * 32 + (lane & 31), N - 1);
  // the wave's next adapter (smallest pending key), taken off the pending set
  auto next_key = [&]() {
    int a = pend[0];
#pragma unroll
    for (int i = 1; i < MI; ++i) a = min(a, pend[i]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a = min(a, __shfl_xor(a, m, 64));
    a = __builtin_amdgcn_readfirstlane(a);
#pragma unroll
    for (int i = 0; i < MI; ++i) pend[i] = pend[i] == a ? kNone : pend[i];
    return a;
  };
  int a = next_key(), rank = 0, koff = 0, q0 = 0;
  auto adapter_meta = [&]() {
    if (a == kBad) {
      rank = 16;  // one step, no memory of its own
      koff = 0;
    } else if (a != kNone) {
      rank = uniform_load(pv.rank, a);
      koff = uniform_load(lo.koff, a);
    }
  };
  adapter_meta();
  // Steps (adapter, 16 ranks) in batches of kBatch: all loads of a batch go
  // out together, then its MFMAs run.  A batch is always full: slots past
  // the last step load valid addresses and are zeroed (branch-free), so the
  // loads of the whole batch can be issued back to back.  (One flat loop: a
  // nested loop made the register allocator move the accumulators out of
  // the AGPRs.)
  while (a != kNone) {
    int sa[kBatch], sq[kBatch], sb[kBatch], sr[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      sa[k] = a;  // kNone for an empty slot: matches no row
      sq[k] = 0;
      sb[k] = 0;
      sr[k] = 16;
      if (a != kNone) {
        const int rp = (rank + 15) & ~15;
        sq[k] = q0;
        sr[k] = rp;
        sb[k] = koff * N + q0;  // element offset of (col 0, rank q0) in the adapter's block
        q0 += 16;
        if (q0 >= rank) {
          a = next_key();
          q0 = 0;
          adapter_meta();
        }
      }
    }
    uint4 fa[kBatch][MI], fb[kBatch][NJ];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[k][i] = *reinterpret_cast<const uint4*>(lo.tb + trow[i] + sq[k]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[k][j] = *reinterpret_cast<const uint4*>(lo.upt + sb[k] + col[j] * sr[k] + 8 * half);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      // A = t of the rows on this step's adapter, zero for the others (NaN
      // for the invalid rows' step); B of an empty or invalid-row slot is
      // zeroed (its memory may hold anything; NaN times zero stays NaN)
      const bool bad = sa[k] == kBad;
      const uint32_t live = (sa[k] != kNone && !bad) ? 0xffffffffu : 0u;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint32_t m = key[i] == sa[k] ? 0xffffffffu : 0u;
        const uint32_t nan = bad ? 0x7fc07fc0u : 0u;
        fa[k][i] = make_uint4(((fa[k][i].x & live) | nan) & m, ((fa[k][i].y & live) | nan) & m,
                              ((fa[k][i].z & live) | nan) & m, ((fa[k][i].w & live) | nan) & m);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[k][j] = make_uint4(fb[k][j].x & live, fb[k][j].y & live, fb[k][j].z & live, fb[k][j].w & live);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fb[k][j]), as_bf16x8(fa[k][i]), acc[i][j],
                                                              0, 0, 0);
    }
  }
}

// LORA (whole-K form only): the low-rank term of every row is added as
// extra K tiles over the rank-concatenated operands (when lora_prep wrote
// Kx > 0) or else in the epilogue (ring_lora_epilogue); rows with an invalid
// id become NaN.
// CO (medium split-K tiles only): the per-row shrink T[k] = s_a Down_a x_k
// runs in n_shrink workgroups of its own ahead of the tiles, and the tiles
// take the ring with two 32 KiB stages, so a shrink workgroup and a tile
// workgroup fit on one CU together (64 KiB of LDS each, at most 256
// registers per lane) and the shrink's Down reads overlap the tiles' work
// instead of following it.  (Run by the tile workgroups after their tiles,
// the shrink's latency showed in full.)
// The per-row shrink of row k with its key taken from the batch's adapter
// ids and the resident table (the same key the segment workspace holds).
template <bool VEC, int NW>
__device__ __forceinline__ void shrink_row_body_ids(const PoolView& pv, int proj, const uint16_t* __restrict__ X,
                                                    const int32_t* __restrict__ ids, int k, float* __restrict__ T,
                                                    int32_t* __restrict__ desc) {
  const int a = ids[k];
  const int rk = (a >= 0 && a < pv.max_adapters) ? pv.rank[a] : 0;
  const int key = row_key_of(a, rk, pv.max_adapters);
  write_row_desc(pv, proj, key, k, desc);
  if (key < 0) return;  // base-only or invalid: no low-rank term
  shrink_row_to<VEC, NW>(pv, pv.down_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank, rk, pv.scale[key],
                         X + (size_t)k * pv.din, T + (size_t)k * pv.max_rank);
}

// The store of a wave's MI x NJ accumulator blocks (rows wr + 32 i, columns
// wc + 32 j) through LDS, `st` being the wave's own buffer of at least
// MI 32 rows x NJ 32 elements (bf16 Y, or fp32 partials `pt` when PART).
// Rows of the buffer are RB bytes, CH 16-byte chunks, XOR-swizzled by
// row % CH so that both the scattered piece writes and the row reads spread
// over the banks.  Each read pass covers 64 / CH rows, one 16-byte piece per
// lane; pieces past N, and every piece when N or the output is not aligned
// to 16 bytes per piece, go out element by element.  The 16-byte pieces are
// non-temporal stores: every CU writes its tile at about the same moment,
// and streaming them past the L2 shortened the medium split-K launches by
// 3-14 % (their finish pass reads the partials back a little slower).
template <int MI, int NJ, bool PART>
__device__ __forceinline__ void ring_store_tile(int wave, int wr, int wc, int M, int N, uint16_t* __restrict__ Y,
                                                float* __restrict__ pt, floatx16 (&acc)[MI][NJ], uint16_t* st16) {
  constexpr int ES = PART ? 4 : 2;  // bytes per element
  constexpr int RB = NJ * 32 * ES, CH = RB / 16, EPC = 16 / ES, RPP = 64 / CH;
  static_assert(CH == 8 || CH == 16, "rows of 128 or 256 bytes");
  char* st = reinterpret_cast<char*>(st16);
  const int lane = threadIdx.x & 63, h = lane >> 5, lr = lane & 31;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int R = i * 32 + lr, off = (j * 32 + 8 * g + 4 * h) * ES;
        char* d = st + R * RB + (((off >> 4) ^ (R % CH)) << 4) + (off & 15);
        const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1], v2 = acc[i][j][4 * g + 2],
                    v3 = acc[i][j][4 * g + 3];
        if constexpr (PART)
          *reinterpret_cast<float4*>(d) = make_float4(v0, v1, v2, v3);
        else
          *reinterpret_cast<uint2*>(d) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
      }
  // the wave's own LDS writes before its reads: DS instructions of a wave
  // complete in order, the fence keeps the compiler from reordering them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int cc = lane % CH, rr = lane / CH;
  const int col = wc + cc * EPC;
  const bool vec = N % EPC == 0 && (PART ? reinterpret_cast<uintptr_t>(pt) : reinterpret_cast<uintptr_t>(Y)) % 16 == 0;
#pragma unroll
  for (int p = 0; p < MI * 32 / RPP; ++p) {
    const int R = p * RPP + rr, row = wr + R;
    const uint4 v = *reinterpret_cast<const uint4*>(st + R * RB + ((cc ^ (R % CH)) << 4));
    if (row >= M || col >= N) continue;
    if (vec) {
      void* dst = PART ? static_cast<void*>(pt + (size_t)row * N + col) : static_cast<void*>(Y + (size_t)row * N + col);
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, static_cast<u32x4*>(dst));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (col + e < N) {
          if constexpr (PART)
            pt[(size_t)row * N + col + e] = __uint_as_float(w[e]);
          else
            Y[(size_t)row * N + col + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// IDS (co-resident form only): the shrink workgroups take each row's key
// from the adapter ids `ids`, and the first workgroup dispatched, (0, 0),
// builds the batch's segment workspace seg_ws (seg_passes radix passes) in
// the LDS its ring would use, while the rows go to the other n_shrink - 1
// (seg_rows: to all n_shrink, that workgroup's share last).
// S4 (co-resident mapping, split-K partials): the tiles run over the 4-stage
// ring (128 KiB of LDS) and the launch has no shrink workgroups.
template <int TM, int TN, bool PART, bool LORA, bool CO, bool IDS = false, bool S4 = false>
__device__ __forceinline__ void gemm_ring_body(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y,
    float* __restrict__ part, int M, int K, int N, int tiles_n, int n_tiles, int per_xcd, int kt_per, PoolView pv,
    const int32_t* __restrict__ row_key, LoraOperands lo, int proj, float* __restrict__ Trows, int n_shrink,
    const int32_t* __restrict__ ids = nullptr, int32_t* __restrict__ seg_ws = nullptr,
    int seg_passes = 0, int seg_rows = 0) {
  static_assert(!(PART && LORA), "the low-rank epilogue needs the whole K range");
  static_assert(!CO || (TM == 128 && TN == 128), "co-resident form: 128x128 tiles");
  static_assert(!(TM == 256) || TN == 256, "large form: 256x256 tiles");
  static_assert(!PART || CO, "split-K partials: the co-resident form");
  static_assert(!IDS || CO, "the id-based form is the co-resident one");
  constexpr int MI = TM / 64, NJ = TN / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (CO) {
    if ((int)blockIdx.x < n_shrink) {
      {
        if constexpr (IDS) {
          if (blockIdx.x == 0) {
            // up to 1024 rows: 2 * 1088 + 4 * kRadix words of scratch
            static_assert((2 * 1088 + kRadix * (kRingThreads / 64)) * 4 <= sizeof(m64_a0), "segment scratch");
            static_assert(kMaxWaves + 3 <= sizeof(m64_a1) / 4, "segment scratch");
            const int cap = ((M + 1) + 63) & ~63;
            seg_build_block<kRingThreads>(ids, M, pv.rank, pv.max_adapters, seg_passes, cap, seg_ws,
                                          reinterpret_cast<uint32_t*>(m64_a0), reinterpret_cast<int*>(m64_a1),
                                          reinterpret_cast<int*>(m64_a1) + kMaxWaves);
          }
          // the rows: over the other workgroups, or (seg_rows) over all of
          // them, the segment build's taking the last share
          if (blockIdx.x != 0 || seg_rows) {
            const int nw = seg_rows ? n_shrink : n_shrink - 1;
            const int i0 = seg_rows ? ((int)blockIdx.x + n_shrink - 1) % n_shrink : (int)blockIdx.x - 1;
            for (int k = i0; k < M; k += nw)
              shrink_row_body_ids<true, kRingThreads / 64>(pv, proj, X, ids, k, Trows,
                                                           row_desc(Trows, M, pv.max_rank));
          }
        } else {
          for (int k = blockIdx.x; k < M; k += n_shrink)
            shrink_row_body<true, kRingThreads / 64>(pv, proj, X, row_key, k, Trows, row_desc(Trows, M, pv.max_rank));
        }
      }
      return;
    }
  }
  // the tile workgroups follow the shrink workgroups in a one-dimensional
  // grid, K slice by K slice (no idle shrink slots per slice to dispatch);
  // n_shrink and per_xcd * 8 are multiples of 8, so a workgroup's XCD is
  // bx & 7 either way
  const int b = (int)blockIdx.x - (CO ? n_shrink : 0);
  const int ks = PART ? b / (per_xcd * 8) : 0;
  const int bx = PART ? b % (per_xcd * 8) : b;
  const int t = (bx & 7) * per_xcd + (bx >> 3);
  if (t >= n_tiles) return;
  // large: groups of kGroupM row bands walked column by column, so the
  // ~32 tiles an XCD runs at once form a kGroupM x 8 block that shares X and
  // W slices in its L2 (row-band major order re-fetched every W tile for
  // each band); split-K medium: column major, so the few row tiles of a W
  // column block run on one XCD and W crosses HBM once
  const int tiles_m = n_tiles / tiles_n;
  int mt, nt;
  if (PART) {
    mt = t % tiles_m;
    nt = t / tiles_m;
  } else {
    const int g = t / (kGroupM * tiles_n), r = t % (kGroupM * tiles_n);
    const int gm = min(kGroupM, tiles_m - g * kGroupM);
    mt = g * kGroupM + r % gm;
    nt = r / gm;
  }
  const int m0 = mt * TM, n0 = nt * TN;
  RingCtx c;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: DMA offsets stay scalar
  c.fr = lane & 31;
  c.fk = lane >> 5;
  c.wm = c.wave >> 1;
  c.wn = c.wave & 1;
  c.row_bytes = K * 2;
  c.rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X + (size_t)m0 * K), (short)0,
                                            (M - m0) * c.row_bytes, 0x00020000);
  c.rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W + (size_t)n0 * K), (short)0,
                                            (N - n0) * c.row_bytes, 0x00020000);
  // lane L fills LDS slot (row L >> 2 of its 16-row group, physical chunk
  // L & 3), which holds logical chunk (L & 3) ^ ((row >> 2) & 3)
  c.voff = (lane >> 2) * c.row_bytes + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  // 64-deep stages: lane L fills LDS slot (row L >> 3 of its 8-row group,
  // physical chunk L & 7); the group's rows 8i + (L >> 3) have (row >> 1) & 7
  // = (4 (i & 1) + (L >> 4)) & 7, and i & 1 = wave & 1 for every group of a wave
  c.voff64 = (lane >> 3) * c.row_bytes + (((lane & 7) ^ ((4 * (c.wave & 1) + (lane >> 4)) & 7)) << 4);

  floatx16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int kt0 = PART ? ks * kt_per : 0;
  int kend = PART ? kt0 + kt_per : K / GBK64;
  // LORA: a batch in the rank-concatenated form (kx > 0) runs kx / 64 more
  // K tiles from Tx and Ux, and no epilogue
  int kx = 0;
  c.kmain = kend;
  c.rsx = c.rsa;
  c.rsu = c.rsb;
  c.voffx = c.voff64;
  c.xrow_bytes = c.row_bytes;
  if constexpr (LORA) {
    if (lo.kx != nullptr) {
      kx = uniform_load(lo.kx, 0);
      c.xrow_bytes = lo.txw * 2;
      c.rsx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(lo.tx + (size_t)m0 * lo.txw), (short)0,
                                                (M - m0) * c.xrow_bytes, 0x00020000);
      c.rsu = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(lo.upt + (size_t)n0 * lo.txw), (short)0,
                                                (N - n0) * c.xrow_bytes, 0x00020000);
      c.voffx = (lane >> 3) * c.xrow_bytes + (((lane & 7) ^ ((4 * (c.wave & 1) + (lane >> 4)) & 7)) << 4);
      kend += kx / GBK64;
    }
  }
  if constexpr (S4) {
    static_assert(CO && PART && !LORA, "the 4-stage form: split-K partials of 128x128 tiles");
    ring64_loop4<TM, TN>(c, m64_a0, m64_a1, m64_a2, m64_a3, m64_b0, m64_b1, m64_b2, m64_b3, kt0, kend, acc);
  } else if constexpr (CO) {
    ring64x2_loop<TM, TN, LORA>(c, m64_a0, m64_a1, m64_b0, m64_b1, kt0, kend, acc);
  } else if constexpr (TM == 256) {
    ring64x2_loop<TM, TN, LORA>(c, h64_a0, h64_a1, h64_b0, h64_b1, kt0, kend, acc);
  } else {
    ring64_loop4<TM, TN>(c, m64_a0, m64_a1, m64_a2, m64_a3, m64_b0, m64_b1, m64_b2, m64_b3, kt0, kend, acc);
  }

  int key[MI];  // low-rank epilogue: the keys of the lane's A-fragment rows
  if constexpr (LORA) {
    __builtin_amdgcn_sched_barrier(0);
    // (left out when the batch's Up blocks overran the operand buffer: a
    // separate expand then adds the term)
    if (kx == 0 && (lo.over == nullptr || uniform_load(lo.over, 0) == 0))
      ring_lora_epilogue<MI, NJ>(m0 + c.wm * (TM / 2), n0 + c.wn * (TN / 2), M, N, pv, row_key, lo, acc, key);
  }

  // Output through LDS.  The ring's MFMAs take the W0 fragment as A and the
  // X fragment as B, so each 32x32 accumulator block is the transposed
  // output: lane l holds output row l % 32 and columns 8 (v / 4) + 4 (l / 32)
  // + v % 4, four consecutive columns per v / 4, one 8-byte (bf16) or 16-byte
  // (fp32 partials) piece.  Straight to memory every store instruction would
  // scatter over 32 rows; instead each wave writes its (MI 32) x (NJ 32)
  // block into a ring buffer of its own (idle once every wave has passed the
  // barrier below: the rings' DMAs were waited for) and reads it back as
  // 16-byte row pieces, so one store instruction covers whole rows.
  static_assert(MI * 32 * NJ * 32 * (PART ? 4 : 2) <= (TM == 256 ? sizeof(h64_a0) : sizeof(m64_a0)),
                "a wave's output block fits its ring buffer");
  ring_barrier();
  ring_store_tile<MI, NJ, PART>(c.wave, m0 + c.wm * (TM / 2), n0 + c.wn * (TN / 2), M, N, Y,
                                PART ? part + (size_t)ks * M * N : nullptr, acc,
                                TM == 256 ? (c.wave == 0 ? h64_a0 : c.wave == 1 ? h64_a1 : c.wave == 2 ? h64_b0 : h64_b1)
                                          : (c.wave == 0 ? m64_a0 : c.wave == 1 ? m64_a1 : c.wave == 2 ? m64_b0 : m64_b1));
}

// one workgroup per CU: 256x256 tiles (large products, with or without the
// low-rank term) or whole-K 128x128 tiles over a 4-stage ring (plain
// medium GEMM)
template <int TM, int TN, bool LORA>
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_ring(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int K, int N,
    int tiles_n, int n_tiles, int per_xcd, PoolView pv, const int32_t* __restrict__ row_key, LoraOperands lo) {
  gemm_ring_body<TM, TN, false, LORA, false>(X, W, Y, nullptr, M, K, N, tiles_n, n_tiles, per_xcd, 0, pv, row_key, lo,
                                             0, nullptr, 0);
}

// two workgroups per CU on whole-K 128x128 tiles (plain GEMM, Y in bf16)
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_ring_co_whole(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int K, int N,
    int tiles_n, int n_tiles, int per_xcd) {
  gemm_ring_body<128, 128, false, false, true>(X, W, Y, nullptr, M, K, N, tiles_n, n_tiles, per_xcd, 0, PoolView{},
                                               nullptr, LoraOperands{}, 0, nullptr, 0);
}

// the same with the low-rank term
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_ring_co_lora(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int K, int N,
    int tiles_n, int n_tiles, int per_xcd, PoolView pv, const int32_t* __restrict__ row_key, LoraOperands lo) {
  gemm_ring_body<128, 128, false, true, true>(X, W, Y, nullptr, M, K, N, tiles_n, n_tiles, per_xcd, 0, pv, row_key,
                                              lo, 0, nullptr, 0);
}

__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_ring_co(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y,
    float* __restrict__ part, int M, int K, int N, int tiles_n, int n_tiles, int per_xcd, int kt_per, PoolView pv,
    const int32_t* __restrict__ row_key, int proj, float* __restrict__ Trows, int n_shrink) {
  gemm_ring_body<128, 128, true, false, true>(X, W, Y, part, M, K, N, tiles_n, n_tiles, per_xcd, kt_per, pv, row_key,
                                              LoraOperands{}, proj, Trows, n_shrink);
}

// the same, with the row keys from the adapter ids and the segment build in
// workgroup (0, 0)
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_ring_co_ids(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y,
    float* __restrict__ part, int M, int K, int N, int tiles_n, int n_tiles, int per_xcd, int kt_per, PoolView pv,
    int proj, float* __restrict__ Trows, int n_shrink, const int32_t* __restrict__ ids, int32_t* __restrict__ seg_ws,
    int seg_passes, int seg_rows) {
  gemm_ring_body<128, 128, true, false, true, true>(X, W, Y, part, M, K, N, tiles_n, n_tiles, per_xcd, kt_per, pv,
                                                    nullptr, LoraOperands{}, proj, Trows, n_shrink, ids, seg_ws,
                                                    seg_passes, seg_rows);
}

// Medium products without the low-rank term, from kMidS4Rows rows: split-K
// 128x128 tiles over the 4-stage ring (128 KiB of LDS, one workgroup per
// CU), three stages of lookahead where the co-resident form has one.
// Against that form: 24.1 against 32.4 us at 512 x 4096 x 4096, 40.5
// against 58.6 us at 1024 rows; no gain at 256 rows.  (The layer with its
// per-row shrink keeps the co-resident form: the shrink workgroups no
// longer fit beside 128 KiB tiles, and run on a second stream they started
// only as the tiles ended, the cross-stream waits costing about 10 us each.)
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_ring_split4(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ part, int M, int K, int N,
    int tiles_n, int n_tiles, int per_xcd, int kt_per) {
  gemm_ring_body<128, 128, true, false, true, false, true>(X, W, nullptr, part, M, K, N, tiles_n, n_tiles, per_xcd,
                                                           kt_per, PoolView{}, nullptr, LoraOperands{}, 0, nullptr, 0);
}


// Large products: 256x256 tiles, one workgroup per CU, unless too few tiles
// fill the chip's 256 slots; then 128x128 tiles two workgroups per CU
// (measured ~8 % slower per tile-flop at full occupancy, so they win when
// they fill the machine clearly better: 2048x4096x4096 in 64 us against 91).
bool big_prefers_co(int M, int N) {
  const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
  const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  const double e256 = (double)t256 / (((t256 + 255) / 256) * 256);
  const double e128 = (double)t128 / (((t128 + 511) / 512) * 512);
  return e128 > 1.08 * e256;
}

hipError_t launch_big(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, hipStream_t st) {
  if (big_prefers_co(M, N)) {
    const int tiles_n = (N + 127) / 128, n_tiles = ((M + 127) / 128) * tiles_n;
    const int per_xcd = (n_tiles + 7) / 8;
    MLORA_LAUNCH("gemm_big", gemm_ring_co_whole, dim3(per_xcd * 8), dim3(kRingThreads), 0, st, X, W, Y, M, K, N,
                 tiles_n, n_tiles, per_xcd);
    return launched();
  }
  const int tiles_n = (N + 255) / 256, n_tiles = ((M + 255) / 256) * tiles_n;
  const int per_xcd = (n_tiles + 7) / 8;
  MLORA_LAUNCH("gemm_big", (gemm_ring<256, 256, false>), dim3(per_xcd * 8), dim3(kRingThreads), 0, st, X, W, Y, M, K,
               N, tiles_n, n_tiles, per_xcd, PoolView{}, (const int32_t*)nullptr, LoraOperands{});
  return launched();
}

template <bool VEC>
hipError_t launch_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, hipStream_t st) {
  if (M <= 64) {
    const dim3 grid((N + 15) / 16), block(64 * kSkinnyWaves);
    if (M <= 16) MLORA_LAUNCH("gemm_skinny", (gemm_skinny<1, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 32) MLORA_LAUNCH("gemm_skinny", (gemm_skinny<2, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 48) MLORA_LAUNCH("gemm_skinny", (gemm_skinny<3, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else MLORA_LAUNCH("gemm_skinny", (gemm_skinny<4, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
  } else if (VEC && M <= 1024 && K % (GBK64 * 4) == 0 && (long)M * K * 2 < (1L << 31) &&
             (long)N * K * 2 < (1L << 31)) {
    // medium batches without scratch for split-K partials: 128x128 ring
    // tiles over the whole K, Y written once in bf16
    const int tiles_n = (N + 127) / 128, n_tiles = ((M + 127) / 128) * tiles_n;
    const int per_xcd = (n_tiles + 7) / 8;
    MLORA_LAUNCH("gemm_mid", (gemm_ring<128, 128, false>), dim3(per_xcd * 8), dim3(kRingThreads), 0, st, X, W, Y, M,
                 K, N, tiles_n, n_tiles, per_xcd, PoolView{}, (const int32_t*)nullptr, LoraOperands{});
    return launched();
  } else if (M <= 1024 && (long)((M + 127) / 128) * ((N + 31) / 32) >= 128) {
    const dim3 grid((N + 31) / 32, (M + 32 * KS_MB - 1) / (32 * KS_MB)), block(64 * kKsWaves);
    MLORA_LAUNCH("gemm_ksplit", (gemm_ksplit<VEC, false>), grid, block, 0, st, X, W, Y, M, K, N, PoolView{}, 0, nullptr,
                       nullptr);
  } else if (VEC && K % kRingKAlign == 0 && (long)M * N >= 2048L * 2048L && (long)M * K * 2 < (1L << 31) &&
             (long)N * K * 2 < (1L << 31)) {
    return launch_big(X, W, Y, M, K, N, st);
  } else {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(kTiledThreads);
    MLORA_LAUNCH("gemm_tiled", (gemm_tiled<VEC>), grid, block, 0, st, X, W, Y, M, K, N, nullptr, 0);
    return launched();
  }
  return launched();
}

// ---------------------------------------------------------------------------
// decode: split-K skinny GEMM with the low-rank expand, for M <= 64.
//
// Every workgroup reading all of X made X (L2-resident, but read 256 times)
// cost as much as streaming W0 from HBM.  Here a workgroup owns 64 columns
// and one of S slices of K (at most 1024 deep, a whole number of 128-wide
// units; S = 4 up to din 4096, then one slice per 1024): its X slice
// (M x slice) is brought into LDS once by LDS DMA and shared by the 4
// column-group waves, so each X byte is read by N/64 workgroups instead of
// N/16, while 64 * S workgroups still cover the chip.  8 GEMM waves = 4
// column groups x 2 halves of the slice (the halves take alternate 64-wide
// segments); each wave issues all 16 of its W0 loads at once.  The slice's
// fp32 partial goes to `part` and a second kernel (finish_part) sums the S
// partials in slice order, adds the low-rank term and writes Y:
// deterministic.  (Finishing in the last workgroup of a column block behind
// an atomic counter cost more: the device-scope release/acquire writes back
// and invalidates the L2s.)  The per-row shrink of the batch rides along as
// extra work of the same workgroups: independent work, and one launch less
// per step.
// LDS: X slice [M][xs_stride] in 1 KiB blocks whose 16-byte chunks are
// XOR-swizzled by (row & 15), so the 16 rows an MFMA fragment read touches
// hit 16 different chunk positions.
// ---------------------------------------------------------------------------
constexpr int kDecCols = 64, kDecWaves = 8;
constexpr int kDecMinSlices = 4, kDecMaxDepth = 1024, kDecUnit = 128;

// Number of K slices of the decode form for din K (a multiple of kDecUnit,
// at most kDecMaxSlices * kDecMaxDepth).
int dec_slices(int K) {
  const int s = (K + kDecMaxDepth - 1) / kDecMaxDepth;
  return s > kDecMinSlices ? s : kDecMinSlices;
}
// Slice s of S over U units: units [U s / S, U (s + 1) / S), so slices differ
// by at most one unit.
__host__ __device__ __forceinline__ int dec_slice_unit(int U, int S, int s) { return (int)(((long)U * s) / S); }
// LDS row stride of the X slice: the deepest slice rounded up to 1 KiB blocks.
int dec_xs_stride(int K, int S) {
  const int units = (K / kDecUnit + S - 1) / S;
  return (units * kDecUnit + 511) / 512 * 512;
}
constexpr int kMidMaxSplit = 8;

// Row r's key and its adapter's rank (0 for a key < 0) from the batch's
// adapter ids and the resident table; every value is wave-uniform, so the
// loads are scalar and never wait for the vector loads in flight.
struct KeyRank {
  int key, rank;
};
__device__ __forceinline__ KeyRank key_rank_from_ids(const int32_t* __restrict__ ids, const PoolView& pv, int r) {
  const int a = __builtin_amdgcn_readfirstlane(ids[r]);
  int rk = 0;
  if (a >= 0 && a < pv.max_adapters) rk = __builtin_amdgcn_readfirstlane(pv.rank[a]);
  const int key = __builtin_amdgcn_readfirstlane(row_key_of(a, rk, pv.max_adapters));
  return {key, key >= 0 ? rk : 0};
}

// IDS: the row keys come from the adapter ids `ids` and the resident table
// instead of a built workspace, and one workgroup past the GEMM's builds
// that workspace (seg_ws) beside it.
template <int MB, bool IDS>
__global__ __launch_bounds__(64 * kDecWaves) void gemm_decode(const uint16_t* __restrict__ X,
                                                             const uint16_t* __restrict__ W, int M, int K, int N,
                                                             int S, int xs_stride, PoolView pv, int proj,
                                                             const int32_t* __restrict__ row_key,
                                                             float* __restrict__ Tp, float* __restrict__ part,
                                                             int shrink, const int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ seg_ws) {
  extern __shared__ __attribute__((aligned(16))) uint16_t dec_lds[];
  if (IDS && (int)blockIdx.x == ((N + kDecCols - 1) / kDecCols) * S) {
    int* scratch_lds = reinterpret_cast<int*>(dec_lds);  // 516 bytes of at least 4 KiB (the reduction area alone)
    seg_build_wave(ids, M, pv.rank, pv.max_adapters, seg_ws, scratch_lds, scratch_lds + 65);
    return;
  }
  uint16_t* xs = dec_lds;                                                      // [M][xs_stride]
  floatx4* red = reinterpret_cast<floatx4*>(dec_lds + (size_t)M * xs_stride);  // [4][MB][64]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ncb = (N + kDecCols - 1) / kDecCols;
  const int cb = blockIdx.x % ncb, kq = blockIdx.x / ncb;
  const int n0 = cb * kDecCols;
  const int cg = wave & 3, kh = wave >> 2;
  // this workgroup's slice: [k0, k0 + Kq), nseg 128-wide units; each half
  // of the waves takes one 64-wide segment of every unit (nseg <= 8)
  const int U = K / kDecUnit;
  const int u0 = dec_slice_unit(U, S, kq), nseg = dec_slice_unit(U, S, kq + 1) - u0;
  const int k0 = u0 * kDecUnit, Kq = nseg * kDecUnit;

  // X slice -> LDS first (an L2 hit for all but the first workgroups of a
  // slice): instruction (row r, 1 KiB block b); lane l fetches logical
  // chunk l ^ (r & 15) of the block into physical chunk l.  In the last
  // block of a slice that is not a whole number of blocks, lanes whose
  // chunk lies past the slice fetch nothing (those LDS chunks are never
  // read), so no load leaves the slice.
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), (short)0, M * K * 2, 0x00020000);
  const int blocks = (Kq + 511) / 512;
  for (int i = wave; i < M * blocks; i += kDecWaves) {
    const int r = i / blocks, bl = i % blocks;
    if (bl * 64 + (lane ^ (r & 15)) < Kq / 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, xs + (size_t)r * xs_stride + bl * 512, 16,
                                               (lane ^ (r & 15)) * 16, (r * K + k0 + bl * 512) * 2, 0, 0);
  }
  // then W0, all 16 loads of the wave at once.  Instruction 2s+h reads rows
  // 8h + (l & 7) of the column group, 16-byte chunk l >> 3 of the wave's
  // half of unit s: 128 contiguous bytes per row (64-byte row pieces cost
  // 30 % more HBM time), next to the other half's 128.  Segments are
  // consumed as they land (the compiler's waits count the loads in issue
  // order).
  const size_t kbase = (size_t)k0 + kh * 64 + (lane >> 3) * 8;
  const uint16_t* w0p = W + (size_t)min(n0 + 16 * cg + (lane & 7), N - 1) * K + kbase;
  const uint16_t* w1p = W + (size_t)min(n0 + 16 * cg + 8 + (lane & 7), N - 1) * K + kbase;
  uint4 wv[16];
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    wv[2 * sg] = *reinterpret_cast<const uint4*>(w0p + min(sg, nseg - 1) * kDecUnit);
    wv[2 * sg + 1] = *reinterpret_cast<const uint4*>(w1p + min(sg, nseg - 1) * kDecUnit);
  }
  // The per-row shrink rides along: this workgroup computes the slice-kq
  // partial of T for rows cb, cb + ncb, ... from the X slice it already
  // holds.  Key, rank and pages are uniform (scalar loads, which do not wait
  // for the vector loads in flight); the first 16 ranks of the first row
  // are fetched now: each wave takes ranks wave and wave + 8, each lane the
  // 16-byte chunks lane and lane + 64 of the slice (nch chunks in all; a
  // lane past them re-reads the last one and adds nothing).
  const int nch = Kq / 8;
  // halves (at most half as many rows as column blocks): each row's shrink
  // is shared by two column blocks, 8 of every 16 ranks each, one rank per
  // wave, so that every workgroup carries the same shrink work
  const bool halves = shrink && 2 * M <= ncb;
  const int srow = halves ? (cb >> 1) : cb, hq = halves ? 8 * (cb & 1) : 0;
  int key0 = -1, rank0 = 0;
  uint4 dn[2][2];
  if (shrink && srow < M) {
    if (IDS) {
      const KeyRank kr = key_rank_from_ids(ids, pv, srow);
      key0 = kr.key;
      rank0 = kr.rank;
    } else {
      key0 = __builtin_amdgcn_readfirstlane(row_key[srow]);
    }
    if (key0 >= 0) {
      if (!IDS) rank0 = __builtin_amdgcn_readfirstlane(pv.rank[key0]);
      const int32_t* dpage = pv.down_page + ((size_t)key0 * pv.n_proj + proj) * pv.max_rank;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (halves && i > 0) break;
        int pg = dpage[min(hq + wave + 8 * i, pv.max_rank - 1)];
        pg = pg < 0 ? dpage[0] : pg;
        const uint16_t* dr = pv.down + (size_t)pg * pv.din + k0;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          dn[i][cc] = *reinterpret_cast<const uint4*>(dr + min(lane + 64 * cc, nch - 1) * 8);
      }
    }
  }
  // the X slice has landed once at most the 16 W0 loads and the 4 Down
  // loads issued after it are in flight (the barrier carries no fence, so
  // it does not wait for the W0 loads too)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
  ring_barrier();

  floatx4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    if (sg < nseg) {
      // two MFMA B fragments from the pair of loads of segment sg, with one
      // DPP move per dword: f0 = K chunks 0,2,4,6 of the segment (lane group
      // g = l >> 4 takes chunk 2g), f1 = chunks 1,3,5,7.  Column n < 8 is
      // row n (first load), n >= 8 row n (second load), as MFMA wants.
      const uint4 A = wv[2 * sg], B = wv[2 * sg + 1];
      uint4 f0, f1;
      f0.x = __builtin_amdgcn_update_dpp((int)A.x, (int)B.x, 0x118, 0xf, 0xc, false);  // row_shr:8 into lanes 8-15
      f0.y = __builtin_amdgcn_update_dpp((int)A.y, (int)B.y, 0x118, 0xf, 0xc, false);
      f0.z = __builtin_amdgcn_update_dpp((int)A.z, (int)B.z, 0x118, 0xf, 0xc, false);
      f0.w = __builtin_amdgcn_update_dpp((int)A.w, (int)B.w, 0x118, 0xf, 0xc, false);
      f1.x = __builtin_amdgcn_update_dpp((int)B.x, (int)A.x, 0x108, 0xf, 0x3, false);  // row_shl:8 into lanes 0-7
      f1.y = __builtin_amdgcn_update_dpp((int)B.y, (int)A.y, 0x108, 0xf, 0x3, false);
      f1.z = __builtin_amdgcn_update_dpp((int)B.z, (int)A.z, 0x108, 0xf, 0x3, false);
      f1.w = __builtin_amdgcn_update_dpp((int)B.w, (int)A.w, 0x108, 0xf, 0x3, false);
#pragma unroll
      for (int odd = 0; odd < 2; ++odd) {
        const int c = (2 * sg + kh) * 8 + 2 * (lane >> 4) + odd;  // logical 16-byte chunk in the slice row
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = min(mb * 16 + (lane & 15), M - 1);
          const uint4 a = *reinterpret_cast<const uint4*>(xs + (size_t)r * xs_stride + (c >> 6) * 512 +
                                                          (((c & 63) ^ (r & 15)) << 3));
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(odd ? f1 : f0), acc[mb], 0, 0, 0);
        }
      }
    }
  }

  if (halves) {
    if (srow < M) {
      const int r = srow, key = key0, rank = rank0;
      if (kq == 0 && hq == 0) write_row_desc(pv, proj, key, r, row_desc(Tp, M, pv.max_rank));
      if (key >= 0) {
        const int32_t* dpage = pv.down_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank;
        uint4 d[2] = {dn[0][0], dn[0][1]};
        for (int q0 = 0; q0 < rank; q0 += 16) {
          if (q0 > 0) {
            int pg = dpage[min(q0 + hq + wave, pv.max_rank - 1)];
            pg = pg < 0 ? dpage[0] : pg;
            const uint16_t* dr = pv.down + (size_t)pg * pv.din + k0;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
              d[cc] = *reinterpret_cast<const uint4*>(dr + min(lane + 64 * cc, nch - 1) * 8);
          }
          float v = 0.f;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int c = lane + 64 * cc;  // logical chunk of row r's slice
            if (c < nch) {
              const uint4 xa = *reinterpret_cast<const uint4*>(xs + (size_t)r * xs_stride + cc * 512 +
                                                               ((lane ^ (r & 15)) << 3));
              const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
              const uint32_t dw[4] = {d[cc].x, d[cc].y, d[cc].z, d[cc].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v = fmaf(lo_bf(dw[e]), lo_bf(xw[e]), v);
                v = fmaf(hi_bf(dw[e]), hi_bf(xw[e]), v);
              }
            }
          }
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
          const int q = q0 + hq + wave;
          if (lane == 0 && q < rank) Tp[((size_t)kq * M + r) * pv.max_rank + q] = v;
        }
      }
    }
  } else if (shrink) {
    for (int r = cb; r < M; r += ncb) {
      const bool first = r == cb;
      int key, rank;
      if (first) {
        key = key0;
        rank = rank0;
      } else if (IDS) {
        const KeyRank kr = key_rank_from_ids(ids, pv, r);
        key = kr.key;
        rank = kr.rank;
      } else {
        key = __builtin_amdgcn_readfirstlane(row_key[r]);
      }
      if (kq == 0) write_row_desc(pv, proj, key, r, row_desc(Tp, M, pv.max_rank));
      if (key < 0) continue;
      if (!first && !IDS) rank = __builtin_amdgcn_readfirstlane(pv.rank[key]);
      const int32_t* dpage = pv.down_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank;
      uint4 d[2][2];
      // Down chunks of ranks q0 + wave and q0 + wave + 8 (the first group of
      // the first row came in with the W0 loads)
      auto fetch = [&](int q0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          int pg = dpage[min(q0 + wave + 8 * i, pv.max_rank - 1)];
          pg = pg < 0 ? dpage[0] : pg;
          const uint16_t* dr = pv.down + (size_t)pg * pv.din + k0;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
            d[i][cc] = *reinterpret_cast<const uint4*>(dr + min(lane + 64 * cc, nch - 1) * 8);
        }
      };
      if (first) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) d[i][cc] = dn[i][cc];
      } else {
        fetch(0);
      }
      for (int q0 = 0; q0 < rank; q0 += 16) {
        float v[2] = {0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int c = lane + 64 * cc;  // logical chunk of row r's slice
          if (c < nch) {
            const uint4 xa = *reinterpret_cast<const uint4*>(xs + (size_t)r * xs_stride + cc * 512 +
                                                             ((lane ^ (r & 15)) << 3));
            const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t dw[4] = {d[i][cc].x, d[i][cc].y, d[i][cc].z, d[i][cc].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v[i] = fmaf(lo_bf(dw[e]), lo_bf(xw[e]), v[i]);
                v[i] = fmaf(hi_bf(dw[e]), hi_bf(xw[e]), v[i]);
              }
            }
          }
        }
        if (q0 + 16 < rank) fetch(q0 + 16);
        // lanes 0-31 finish rank q0 + wave, lanes 32-63 rank q0 + wave + 8
        const bool up = (lane & 32) != 0;
        float t = (up ? v[1] : v[0]) + __shfl_xor(up ? v[0] : v[1], 32, 64);
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 8, 64);
        t += __shfl_xor(t, 4, 64);
        t += __shfl_xor(t, 2, 64);
        t += __shfl_xor(t, 1, 64);
        const int q = q0 + wave + (up ? 8 : 0);
        if ((lane & 31) == 0 && q < rank) Tp[((size_t)kq * M + r) * pv.max_rank + q] = t;
      }
    }
  }

  if (kh == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[(cg * MB + mb) * 64 + lane] = acc[mb];
  }
  __syncthreads();
  if (kh == 0) {
    // the slice's partial: both halves
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const floatx4 o = red[(cg * MB + mb) * 64 + lane];
      const int c = n0 + 16 * cg + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = mb * 16 + (lane >> 4) * 4 + v;
        if (r < M && c < N) part[((size_t)kq * M + r) * N + c] = acc[mb][v] + o[v];
      }
    }
  }
}

// Sums the S split-K partials of a tile in split order, adds the row's
// low-rank term when LORA (sum_q T[r][q] Up_a[c][q], Up streamed here), and
// writes Y (bf16 RNE); 8 columns per thread, so each Up page row is read as
// coalesced 16-byte pieces.  TPARTS: T holds S partial slices of t (the
// split-K slices of the decode form's shrink), summed and scaled here.
constexpr int kFinishThreads = 64;  // one wave per workgroup: the decode grid spreads over every CU

// sum[0..8) = the S slices (stride apart) of 8 fp32 at p, added in slice
// order; the loads of B slices go out together.
template <int B>
__device__ __forceinline__ void sum_parts(const float* __restrict__ p, size_t stride, int S, float (&sum)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.f;
  for (int q0 = 0; q0 < S; q0 += B) {
    float4 v[B][2];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float* pp = p + min(q0 + u, S - 1) * stride;
      v[u][0] = *reinterpret_cast<const float4*>(pp);
      v[u][1] = *reinterpret_cast<const float4*>(pp + 4);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (q0 + u < S) {
        sum[0] += v[u][0].x; sum[1] += v[u][0].y; sum[2] += v[u][0].z; sum[3] += v[u][0].w;
        sum[4] += v[u][1].x; sum[5] += v[u][1].y; sum[6] += v[u][1].z; sum[7] += v[u][1].w;
      }
    }
  }
}

template <bool LORA, bool TPARTS, int QG = 8>
__global__ __launch_bounds__(kFinishThreads) void finish_part(const float* __restrict__ part, int S,
                                                              uint16_t* __restrict__ Y, int M, int N, PoolView pv,
                                                              int proj, const int32_t* __restrict__ row_key,
                                                              const float* __restrict__ T) {
  const int t = blockIdx.x * kFinishThreads + threadIdx.x;
  const int per_row = N / 8;
  if (t >= M * per_row) return;
  const int r = t / per_row, c0 = (t % per_row) * 8;
  // the partials' loads go out before the low-rank term's dependent chain,
  // 4 or 8 slices' loads at once (summed in slice order)
  float sum[8];
  const float* pr = part + (size_t)r * N + c0;
  if (S <= 4)
    sum_parts<4>(pr, (size_t)M * N, S, sum);
  else
    sum_parts<8>(pr, (size_t)M * N, S, sum);
  float y[8];
  if (LORA) {
    lora_delta8_desc<true, TPARTS, QG>(pv, row_desc(const_cast<float*>(T), M, pv.max_rank), T, r, M, c0, N, y, S);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.f;
  }
  uint4 w;
  w.x = pack_bf2(sum[0] + y[0], sum[1] + y[1]);
  w.y = pack_bf2(sum[2] + y[2], sum[3] + y[3]);
  w.z = pack_bf2(sum[4] + y[4], sum[5] + y[5]);
  w.w = pack_bf2(sum[6] + y[6], sum[7] + y[7]);
  *reinterpret_cast<uint4*>(Y + (size_t)r * N + c0) = w;
}

size_t decode_lds_bytes(int M, int xs_stride, int MB) {
  return (size_t)M * xs_stride * 2 + (size_t)4 * MB * 64 * 16;
}

// shrink: the workgroups also compute T as K-slice partials (S slices of
// [M][max_rank] in T), which the finish pass sums and scales; otherwise T
// holds the finished t (scale folded).
template <int MB>
hipError_t launch_decode(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, const PoolView& pv,
                         int proj, const int32_t* row_key, float* T, float* part, bool shrink, hipStream_t st,
                         bool lora = true, const int32_t* ids = nullptr, int32_t* seg_ws = nullptr) {
  const int S = dec_slices(K), xs_stride = dec_xs_stride(K, S);
  if (S > rows_t_slices(M)) return hipErrorNotSupported;
  const size_t lds = decode_lds_bytes(M, xs_stride, MB);
  static LdsLimit limit;
  const hipError_t le = limit.ensure({(const void*)gemm_decode<MB, false>, (const void*)gemm_decode<MB, true>}, lds);
  if (le != hipSuccess) return le;
  const int ncb = (N + kDecCols - 1) / kDecCols;
  if (seg_ws)
    MLORA_LAUNCH("gemm_decode+seg+shrink_rows", (gemm_decode<MB, true>), dim3(ncb * S + 1), dim3(64 * kDecWaves),
                 lds, st, X, W, M, K, N, S, xs_stride, pv, proj, row_key, T, part, shrink ? 1 : 0, ids, seg_ws);
  else
    MLORA_LAUNCH(shrink ? "gemm_decode+shrink_rows" : "gemm_decode", (gemm_decode<MB, false>), dim3(ncb * S),
                 dim3(64 * kDecWaves), lds, st, X, W, M, K, N, S, xs_stride, pv, proj, row_key, T, part,
                 shrink ? 1 : 0, (const int32_t*)nullptr, (int32_t*)nullptr);
  hipError_t e = launched();
  if (e != hipSuccess) return e;
  const int threads = M * (N / 8);
  // a decode batch's finish has few waves per SIMD: ranks in rounds of 16
  if (!lora)
    MLORA_LAUNCH("finish_base", (finish_part<false, false>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
  else if (shrink)
    MLORA_LAUNCH("finish_part", (finish_part<true, true, 16>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
  else
    MLORA_LAUNCH("finish_part", (finish_part<true, false, 16>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
  return launched();
}

// medium batches: 128x128 tiles with split-K over S workgroups, then the
// finish pass (partials + low-rank term)
int mid_split(int M, int N, int K) {
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (S < kMidMaxSplit && tiles * S < 256 && K % (kRingKAlign * S * 2) == 0) S *= 2;
  return S;
}

bool mid_ring_ok(int M, int K) { return K % kRingKAlign == 0 && (long)M * K * 2 < (1L << 31); }

// rows from which a medium product without the low-rank term (the base GEMM
// of the split and fused plans) takes the 4-stage split-K tiles (the product
// alone: 18.5 us either way at 256 rows, 24.1 against 32.4 us at 512)
constexpr int kMidS4Rows = 384;

// shrink: the per-row shrink (T, one slice) runs in workgroups of its own
// ahead of the tiles, on the same CUs (co-resident form)
hipError_t launch_mid_lora(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, const PoolView& pv,
                           int proj, const int32_t* row_key, float* T, float* part, bool shrink, hipStream_t st,
                           bool lora = true, const int32_t* ids = nullptr, int32_t* seg_ws = nullptr) {
  const int S = mid_split(M, N, K);
  const int tiles_n = (N + 127) / 128, n_tiles = ((M + 127) / 128) * tiles_n;
  const int per_xcd = (n_tiles + 7) / 8;
  if (!lora && !shrink && ids == nullptr && M >= kMidS4Rows) {
    MLORA_LAUNCH("gemm_mid", gemm_ring_split4, dim3(per_xcd * 8 * S), dim3(kRingThreads), 0, st, X, W, part, M, K, N,
                 tiles_n, n_tiles, per_xcd, K / GBK64 / S);
    const hipError_t e = launched();
    if (e != hipSuccess) return e;
    const int threads = M * (N / 8);
    MLORA_LAUNCH("finish_base", (finish_part<false, false>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
    return launched();
  }
  if (ids != nullptr) {
    // the segment build takes the first of the co-resident form's shrink
    // workgroups (at least 72 of them above 64 rows)
    if (!(shrink && lora && M > 64 && M <= 1024)) return hipErrorNotSupported;
    // Up to 256 rows: one workgroup per row (a multiple of 8, at most 256),
    // the segment build's taking a row too, so that all 256 tile workgroups
    // find a free slot beside one (257-264 of them, one more for the build,
    // held tiles back: 256 rows, 25.9-26.3 against 22.0-22.9 us).  Above:
    // one more than the rows, up to 264 (at 512 rows every row workgroup then
    // takes two rows; 256 of them, the build's with rows or without, took
    // 35.7-37.2 us against 34.1-34.9).
    const int seg_rows = M <= 256 ? 1 : 0;
    const int nsw = seg_rows ? min((M + 7) / 8 * 8, 256) : min((M + 1 + 7) / 8 * 8, 264);
    const int passes = M <= kRingThreads ? 0 : ((pv.max_adapters + 1 < 256) ? 1 : 2);
    MLORA_LAUNCH("gemm_mid+seg+shrink_rows", gemm_ring_co_ids, dim3(nsw + per_xcd * 8 * S), dim3(kRingThreads), 0,
                 st, X, W, Y, part, M, K, N, tiles_n, n_tiles, per_xcd, K / GBK64 / S, pv, proj, T, nsw, ids, seg_ws,
                 passes, seg_rows);
  } else {
    // shrink workgroups ahead of the tiles: one per row up to one per CU
    // (each then loops over rows, so the tiles still find a free slot on
    // every CU), a multiple of 8 so the tile workgroups keep their XCD mapping
    const int nsw = shrink ? min((M + 7) / 8 * 8, 256) : 0;
    MLORA_LAUNCH(shrink ? "gemm_mid+shrink_rows" : "gemm_mid", gemm_ring_co, dim3(nsw + per_xcd * 8 * S),
                 dim3(kRingThreads), 0, st, X, W, Y, part, M, K, N, tiles_n, n_tiles, per_xcd, K / GBK64 / S, pv,
                 row_key, proj, T, nsw);
  }
  hipError_t e = launched();
  if (e != hipSuccess) return e;
  const int threads = M * (N / 8);
  if (!lora)
    MLORA_LAUNCH("finish_base", (finish_part<false, false>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
  else
    MLORA_LAUNCH("finish_part", (finish_part<true, false>), dim3((threads + kFinishThreads - 1) / kFinishThreads),
                 dim3(kFinishThreads), 0, st, part, S, Y, M, N, pv, proj, row_key, T);
  return launched();
}

template <bool VEC>
hipError_t launch_lora(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, const PoolView& pv,
                       int proj, const int32_t* row_key, const float* T, hipStream_t st) {
  if (M > 64) {
    const dim3 g((N + 31) / 32, (M + 32 * KS_MB - 1) / (32 * KS_MB)), b(64 * (kKsWaves + kKsLoraWaves));
    MLORA_LAUNCH("gemm_ksplit_lora", (gemm_ksplit<VEC, true>), g, b, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
    return launched();
  }
  const dim3 grid((N + 15) / 16), block(64 * (kSkinnyWaves + kLoraWaves));
  if (M <= 16)
    MLORA_LAUNCH("gemm_skinny_lora", (gemm_skinny_lora<1, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else if (M <= 32)
    MLORA_LAUNCH("gemm_skinny_lora", (gemm_skinny_lora<2, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else if (M <= 48)
    MLORA_LAUNCH("gemm_skinny_lora", (gemm_skinny_lora<3, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else
    MLORA_LAUNCH("gemm_skinny_lora", (gemm_skinny_lora<4, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  return launched();
}

}  // namespace

bool decode_splitk_ok(int M, int K, int N, bool vec) {
  // whole 128-wide units, at least one per slice, every slice at most 1024
  // deep (each wave's half in <= 8 segments, 16 loads)
  return vec && M <= 64 && K % kDecUnit == 0 && K >= kDecMinSlices * kDecUnit &&
         K <= kDecMaxSlices * kDecMaxDepth && (long)M * K * 2 < (1L << 31);
}

hipError_t launch_gemm_lora(const PoolView& pv, int proj, const uint16_t* X, const uint16_t* W, const int32_t* ws,
                            float* T, float* part, uint16_t* Y, int M, bool shrink, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int K = pv.din, N = pv.dout;
  const int32_t* row_key = ws + MLORA_SEG_ROWKEY(M);
  const uintptr_t al = reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W) |
                       reinterpret_cast<uintptr_t>(pv.up) | reinterpret_cast<uintptr_t>(Y);
  const bool vec = (K % 8 == 0) && (N % 8 == 0) && (al % 16 == 0);
  const bool down_vec = reinterpret_cast<uintptr_t>(pv.down) % 16 == 0;  // the in-launch shrink's loads
  if (decode_splitk_ok(M, K, N, vec) && (down_vec || !shrink)) {
    // the per-row shrink shares the GEMM launch
    if (M <= 16) return launch_decode<1>(X, W, Y, M, K, N, pv, proj, row_key, T, part, shrink, stream);
    if (M <= 32) return launch_decode<2>(X, W, Y, M, K, N, pv, proj, row_key, T, part, shrink, stream);
    if (M <= 48) return launch_decode<3>(X, W, Y, M, K, N, pv, proj, row_key, T, part, shrink, stream);
    return launch_decode<4>(X, W, Y, M, K, N, pv, proj, row_key, T, part, shrink, stream);
  }
  if (M > 64 && vec && down_vec && mid_ring_ok(M, K) && (long)N * K * 2 < (1L << 31))
    return launch_mid_lora(X, W, Y, M, K, N, pv, proj, row_key, T, part, shrink, stream);
  if (shrink) {
    hipError_t e = launch_shrink_rows(pv, proj, X, ws, M, T, stream);
    if (e != hipSuccess) return e;
  }
  return vec ? launch_lora<true>(X, W, Y, M, K, N, pv, proj, row_key, T, stream)
             : launch_lora<false>(X, W, Y, M, K, N, pv, proj, row_key, T, stream);
}

hipError_t launch_forward_rows(const PoolView& pv, int proj, const uint16_t* X, const uint16_t* W,
                               const int32_t* ids, int32_t* ws, float* T, float* part, uint16_t* Y, int M,
                               hipStream_t stream) {
  if (M <= 0 || M > 1024) return hipErrorNotSupported;
  const int K = pv.din, N = pv.dout;
  const uintptr_t al = reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W) |
                       reinterpret_cast<uintptr_t>(pv.up) | reinterpret_cast<uintptr_t>(Y) |
                       reinterpret_cast<uintptr_t>(pv.down);
  const bool vec = (K % 8 == 0) && (N % 8 == 0) && (al % 16 == 0);
  const int32_t* row_key = ws + MLORA_SEG_ROWKEY(M);
  if (M > 64) {
    if (vec && mid_ring_ok(M, K) && (long)N * K * 2 < (1L << 31))
      return launch_mid_lora(X, W, Y, M, K, N, pv, proj, row_key, T, part, true, stream, true, ids, ws);
    return hipErrorNotSupported;
  }
  if (!decode_splitk_ok(M, K, N, vec)) return hipErrorNotSupported;
  if (M <= 16) return launch_decode<1>(X, W, Y, M, K, N, pv, proj, row_key, T, part, true, stream, true, ids, ws);
  if (M <= 32) return launch_decode<2>(X, W, Y, M, K, N, pv, proj, row_key, T, part, true, stream, true, ids, ws);
  if (M <= 48) return launch_decode<3>(X, W, Y, M, K, N, pv, proj, row_key, T, part, true, stream, true, ids, ws);
  return launch_decode<4>(X, W, Y, M, K, N, pv, proj, row_key, T, part, true, stream, true, ids, ws);
}

size_t gemm_lora_part_floats(int M, int N, int K) {
  return (size_t)(M > 64 ? mid_split(M, N, K) : dec_slices(K)) * M * N;
}

hipError_t launch_base_split(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, float* part,
                             hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(Y);
  const bool vec = (K % 8 == 0) && (N % 8 == 0) && (al % 16 == 0);
  const PoolView none{};
  if (decode_splitk_ok(M, K, N, vec)) {
    if (M <= 16) return launch_decode<1>(X, W, Y, M, K, N, none, 0, nullptr, nullptr, part, false, stream, false);
    if (M <= 32) return launch_decode<2>(X, W, Y, M, K, N, none, 0, nullptr, nullptr, part, false, stream, false);
    if (M <= 48) return launch_decode<3>(X, W, Y, M, K, N, none, 0, nullptr, nullptr, part, false, stream, false);
    return launch_decode<4>(X, W, Y, M, K, N, none, 0, nullptr, nullptr, part, false, stream, false);
  }
  if (M > 64 && vec && mid_ring_ok(M, K) && (long)N * K * 2 < (1L << 31))
    return launch_mid_lora(X, W, Y, M, K, N, none, 0, nullptr, nullptr, part, false, stream, false);
  return hipErrorNotSupported;
}


bool big_lora_ok(const PoolView& pv, const uint16_t* X, const uint16_t* W, int M) {
  const int K = pv.din, N = pv.dout;
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) % 16 == 0);
  return vec && K % kRingKAlign == 0 && (long)M * N >= 2048L * 2048L && (long)M * K * 2 < (1L << 31) &&
         (long)N * K * 2 < (1L << 31);
}

hipError_t launch_big_lora(const PoolView& pv, const uint16_t* X, const uint16_t* W, const int32_t* ws,
                           const LoraOperands& lo, uint16_t* Y, int M, hipStream_t st) {
  const int K = pv.din, N = pv.dout;
  if (big_prefers_co(M, N)) {
    const int tiles_n = (N + 127) / 128, n_tiles = ((M + 127) / 128) * tiles_n;
    const int per_xcd = (n_tiles + 7) / 8;
    MLORA_LAUNCH("gemm_big_lora", gemm_ring_co_lora, dim3(per_xcd * 8), dim3(kRingThreads), 0, st, X, W, Y, M, K,
                 N, tiles_n, n_tiles, per_xcd, pv, ws + MLORA_SEG_ROWKEY(M), lo);
    return launched();
  }
  const int tiles_n = (N + 255) / 256, n_tiles = ((M + 255) / 256) * tiles_n;
  const int per_xcd = (n_tiles + 7) / 8;
  MLORA_LAUNCH("gemm_big_lora", (gemm_ring<256, 256, true>), dim3(per_xcd * 8), dim3(kRingThreads), 0, st, X, W, Y, M,
               K, N, tiles_n, n_tiles, per_xcd, pv, ws + MLORA_SEG_ROWKEY(M), lo);
  return launched();
}

hipError_t launch_base_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N,
                            hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) % 16 == 0);
  return vec ? launch_gemm<true>(X, W, Y, M, K, N, stream) : launch_gemm<false>(X, W, Y, M, K, N, stream);
}

}  // namespace mlora
