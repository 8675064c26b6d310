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
//    eight consecutive lanes hit eight different chunk positions (no bank
//    conflicts).
#include <stdlib.h>

#include "internal.h"

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
constexpr int kSkinnyUnroll = 4;

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

  const int nfull = VEC ? K / 32 : 0;  // steps whose 32 K values all exist
  int s = wave;
  if (VEC) {
    // groups of kSkinnyUnroll steps, two groups in flight: the loads of group
    // g+1 are issued before the MFMAs of group g, so W0 keeps streaming
    constexpr int kGroup = kSkinnyWaves * kSkinnyUnroll;  // steps spanned by one group
    uint4 b0[kSkinnyUnroll], a0[kSkinnyUnroll][MB], b1[kSkinnyUnroll], a1[kSkinnyUnroll][MB];
    auto load_group = [&](int s_, uint4 (&b)[kSkinnyUnroll], uint4 (&a)[kSkinnyUnroll][MB]) {
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u) {
        const int k = (s_ + u * kSkinnyWaves) * 32;
        b[u] = *reinterpret_cast<const uint4*>(wrow + k);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[u][mb] = *reinterpret_cast<const uint4*>(xrow[mb] + k);
      }
    };
    auto mma_group = [&](const uint4 (&b)[kSkinnyUnroll], const uint4 (&a)[kSkinnyUnroll][MB]) {
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][mb]), as_bf16x8(b[u]), acc[mb], 0, 0, 0);
    };
    // number of whole groups this wave owns
    const int ngroups = (nfull - wave + kGroup - kSkinnyWaves * (kSkinnyUnroll - 1) - 1) / kGroup;
    if (ngroups > 0) {
      load_group(s, b0, a0);
      int g = 0;
      for (; g + 2 <= ngroups; g += 2) {
        load_group(s + kGroup, b1, a1);
        mma_group(b0, a0);
        if (g + 2 < ngroups) load_group(s + 2 * kGroup, b0, a0);
        mma_group(b1, a1);
        s += 2 * kGroup;
      }
      if (g < ngroups) {
        mma_group(b0, a0);
        s += kGroup;
      }
    }
    for (; s < nfull; s += kSkinnyWaves) skinny_step<MB>(wrow, xrow, s * 32, acc);
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
      const int c0 = n0 + 8 * h;
      float acc8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
      const int key = (r < M && c0 < N) ? row_key[r] : -1;
      if (key >= 0) {
        const int rank = pv.rank[key];
        const int32_t* upage = pv.up_page + ((size_t)key * pv.n_proj + proj) * pv.max_rank;
        const float* tr = T + (size_t)r * pv.max_rank;
        for (int q0 = 0; q0 < rank; q0 += 8) {
          // ranks past the adapter's rank read its last column with weight 0
          float u8[8][8], tq[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int qq = min(q0 + q, rank - 1);
            load8<VEC>(pv.up + (size_t)upage[qq] * pv.dout, c0, N, u8[q]);
            const float tv = tr[qq];
            tq[q] = (q0 + q < rank) ? tv : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc8[e] = fmaf(tq[q], u8[q][e], acc8[e]);
        }
      } else if (key == -2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = __uint_as_float(0x7fc00000u);
      }
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
// tiled: 128 x 128 x 64 tiles, 4 waves, MFMA 32x32x16
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kTiledThreads = 256;
constexpr int kChunksPerRow = BK / 8;                          // 16-byte chunks per LDS row
constexpr int kLoadsA = BM * kChunksPerRow / kTiledThreads;    // 4
constexpr int kLoadsB = BN * kChunksPerRow / kTiledThreads;    // 4

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <bool VEC>
__global__ __launch_bounds__(kTiledThreads) void gemm_tiled(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ W,
                                                            uint16_t* __restrict__ Y, int M, int K, int N) {
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

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 31;        // fragment row (A) / column (B) inside a 32-wide tile
  const int fk = lane >> 5;        // which 8-wide half of a 16-wide k step
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
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
        if (r < M) Y[(size_t)r * N + c] = (uint16_t)f2bf(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// big: 256 x 256 x 64 tiles for large batches (prefill), 4 waves of 128x128
// (4 x 4 MFMA 32x32x16 tiles, 256 fp32 accumulators per lane).  Tiles are
// moved global -> LDS by the gfx950 LDS DMA (global_load_lds_dwordx4: each
// lane's 16 bytes land at a fixed LDS slot, so the XOR swizzle is applied by
// choosing which global chunk each lane fetches), double-buffered, so no
// registers are spent on staging.  Workgroups are mapped to tiles so that
// the tiles dispatched to one XCD (block ids congruent mod 8) are contiguous
// along N within one or two 256-row bands of X: they share X rows in that
// XCD's L2.  Needs K % 64 == 0 and 16-byte aligned rows.
// ---------------------------------------------------------------------------
constexpr int GB = 256, GBK = 64;
constexpr int kBigThreads = 256;
constexpr int kTileElems = GB * GBK;

// Four separate LDS arrays (A and B, two stages): with the stage fixed at
// compile time in each half of the unrolled K loop, the compiler can tell
// the DMA target from the buffer being read and does not wait for the DMA
// before every LDS read.
__shared__ __attribute__((aligned(16))) uint16_t big_a0[kTileElems];
__shared__ __attribute__((aligned(16))) uint16_t big_a1[kTileElems];
__shared__ __attribute__((aligned(16))) uint16_t big_b0[kTileElems];
__shared__ __attribute__((aligned(16))) uint16_t big_b1[kTileElems];

// DMA of one K tile (byte offset kb) into (as, bs): instruction j of this
// wave covers rows 8i..8i+7 of the tile, i = wave + 4j, 16 bytes per lane.
#define BIG_ISSUE(kb, as, bs)                                                                  \
  do {                                                                                         \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                            \
      const int i_ = wave + 4 * j;                                                             \
      const int so_ = i_ * 8 * row_bytes + (kb);                                               \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (as) + i_ * 8 * GBK, 16, voff, so_, 0, 0); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (bs) + i_ * 8 * GBK, 16, voff, so_, 0, 0); \
    }                                                                                          \
  } while (0)

// fragments of 16-wide K step kk from (as, bs)
#define BIG_FRAGS(as, bs, kk, fa, fb)                                                           \
  do {                                                                                          \
    const int kc_ = (kk) * 2 + fk;                                                              \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) fa[i] =                                       \
        *reinterpret_cast<const uint4*>((as) + swz(wm * 128 + i * 32 + fr, kc_));               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) fb[j] =                                       \
        *reinterpret_cast<const uint4*>((bs) + swz(wn * 128 + j * 32 + fr, kc_));               \
  } while (0)

// One 64-deep K tile: all 32 fragments of the tile are read from LDS first,
// then the DMA of the next tile is issued (NEXT), then the 64 MFMAs run.  No
// LDS read ever follows an outstanding DMA, so the compiler's conservative
// wait for DMA completion before LDS reads never stalls the pipeline.
#define BIG_STAGE(as, bs, NEXT)                                                                 \
  do {                                                                                          \
    uint4 fa0[4], fb0[4], fa1[4], fb1[4], fa2[4], fb2[4], fa3[4], fb3[4];                       \
    BIG_FRAGS(as, bs, 0, fa0, fb0);                                                             \
    BIG_FRAGS(as, bs, 1, fa1, fb1);                                                             \
    BIG_FRAGS(as, bs, 2, fa2, fb2);                                                             \
    BIG_FRAGS(as, bs, 3, fa3, fb3);                                                             \
    NEXT;                                                                                       \
    __builtin_amdgcn_sched_barrier(0); /* keep reads + DMA issue ahead of the MFMAs */          \
    BIG_MMA(fa0, fb0);                                                                          \
    BIG_MMA(fa1, fb1);                                                                          \
    BIG_MMA(fa2, fb2);                                                                          \
    BIG_MMA(fa3, fb3);                                                                          \
    __builtin_amdgcn_sched_barrier(0); /* the MFMAs stay ahead of the stage's closing wait */   \
  } while (0)

#define BIG_MMA(fa, fb)                                                                                         \
  do {                                                                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] =     \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j], 0, 0, 0);        \
  } while (0)

__global__ __launch_bounds__(kBigThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_big(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        uint16_t* __restrict__ Y, int M, int K, int N, int tiles_n,
                                                        int n_tiles, int per_xcd) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: DMA offsets stay scalar
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= n_tiles) return;
  const int m0 = (t / tiles_n) * GB, n0 = (t % tiles_n) * GB;
  const int fr = lane & 31, fk = lane >> 5, wm = wave >> 1, wn = wave & 1;
  const int row_bytes = K * 2;
  // X rows m0.. and W rows n0..; loads past the end of either return zeros
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (size_t)m0 * K), (short)0, (M - m0) * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + (size_t)n0 * K), (short)0, (N - n0) * row_bytes, 0x00020000);
  // lane L fills LDS chunk slot (row L/8 of its 8-row group, physical chunk
  // L%8), which holds logical chunk (L%8) ^ (L/8) of that row
  const int voff = (lane >> 3) * row_bytes + (((lane & 7) ^ (lane >> 3)) << 4);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / GBK;
  BIG_ISSUE(0, big_a0, big_b0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    // stage 0 holds tile kt; fetch tile kt+1 into stage 1
    BIG_STAGE(big_a0, big_b0, BIG_ISSUE((kt + 1) * GBK * 2, big_a1, big_b1));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // stage 1 holds tile kt+1; fetch tile kt+2 (if any) into stage 0
    BIG_STAGE(big_a1, big_b1, if (kt + 2 < nk) BIG_ISSUE((kt + 2) * GBK * 2, big_a0, big_b0));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (kt < nk) BIG_STAGE(big_a0, big_b0, (void)0);  // odd tile count: the last tile sits in stage 0

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < M) Y[(size_t)r * N + col] = (uint16_t)f2bf(acc[i][j][v]);
      }
    }
}

// MLORA_GEMM_BIG=0 keeps large products on the 128x128 kernel (for A/B timing)
bool big_gemm_enabled() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("MLORA_GEMM_BIG");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

hipError_t launch_big(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, hipStream_t st) {
  const int tiles_m = (M + GB - 1) / GB, tiles_n = (N + GB - 1) / GB;
  const int n_tiles = tiles_m * tiles_n;
  const int per_xcd = (n_tiles + 7) / 8;
  hipLaunchKernelGGL(gemm_big, dim3(per_xcd * 8), dim3(kBigThreads), 0, st, X, W, Y, M, K, N, tiles_n, n_tiles,
                     per_xcd);
  return hipGetLastError();
}

template <bool VEC>
hipError_t launch_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, hipStream_t st) {
  if (M <= 64) {
    const dim3 grid((N + 15) / 16), block(64 * kSkinnyWaves);
    if (M <= 16) hipLaunchKernelGGL((gemm_skinny<1, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 32) hipLaunchKernelGGL((gemm_skinny<2, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 48) hipLaunchKernelGGL((gemm_skinny<3, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else hipLaunchKernelGGL((gemm_skinny<4, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
  } else if (VEC && K % GBK == 0 && (long)M * N >= 2048L * 2048L && (long)M * K * 2 < (1L << 31) &&
             (long)N * K * 2 < (1L << 31) && big_gemm_enabled()) {
    return launch_big(X, W, Y, M, K, N, st);
  } else {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(kTiledThreads);
    hipLaunchKernelGGL((gemm_tiled<VEC>), grid, block, 0, st, X, W, Y, M, K, N);
  }
  return hipGetLastError();
}

template <bool VEC>
hipError_t launch_lora(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, const PoolView& pv,
                       int proj, const int32_t* row_key, const float* T, hipStream_t st) {
  const dim3 grid((N + 15) / 16), block(64 * (kSkinnyWaves + kLoraWaves));
  if (M <= 16)
    hipLaunchKernelGGL((gemm_skinny_lora<1, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else if (M <= 32)
    hipLaunchKernelGGL((gemm_skinny_lora<2, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else if (M <= 48)
    hipLaunchKernelGGL((gemm_skinny_lora<3, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  else
    hipLaunchKernelGGL((gemm_skinny_lora<4, VEC>), grid, block, 0, st, X, W, Y, M, K, N, pv, proj, row_key, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_lora(const PoolView& pv, int proj, const uint16_t* X, const uint16_t* W, const int32_t* ws,
                            const float* T, uint16_t* Y, int M, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int K = pv.din, N = pv.dout;
  const int32_t* row_key = ws + MLORA_SEG_ROWKEY(M);
  const uintptr_t al = reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W) |
                       reinterpret_cast<uintptr_t>(pv.up);
  const bool vec = (K % 8 == 0) && (N % 8 == 0) && (al % 16 == 0);
  return vec ? launch_lora<true>(X, W, Y, M, K, N, pv, proj, row_key, T, stream)
             : launch_lora<false>(X, W, Y, M, K, N, pv, proj, row_key, T, stream);
}

hipError_t launch_base_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N,
                            hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) % 16 == 0);
  return vec ? launch_gemm<true>(X, W, Y, M, K, N, stream) : launch_gemm<false>(X, W, Y, M, K, N, stream);
}

}  // namespace mlora
