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
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 4;

template <int MB, bool VEC>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ W,
                                                                  uint16_t* __restrict__ Y, int M, int K, int N) {
  __shared__ floatx4 red[kSkinnyWaves][MB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int col = n0 + (lane & 15);
  const int kl = (lane >> 4) * 8;  // this lane's K offset inside a 32-wide step
  const bool col_ok = col < N;
  const uint16_t* wrow = W + (size_t)(col_ok ? col : 0) * K;
  const uint16_t* xrow[MB];
  bool row_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * 16 + (lane & 15);
    row_ok[mb] = r < M;
    xrow[mb] = X + (size_t)(row_ok[mb] ? r : 0) * K;
  }
  floatx4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (K + 31) / 32;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  for (int s0 = wave; s0 < nsteps; s0 += kSkinnyWaves * kSkinnyUnroll) {
    uint4 b[kSkinnyUnroll];
    uint4 a[kSkinnyUnroll][MB];
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      const int s = s0 + u * kSkinnyWaves;
      const int k = s * 32 + kl;
      const bool in = s < nsteps;
      b[u] = (in && col_ok) ? load_chunk<VEC>(wrow, k, K) : zero;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a[u][mb] = (in && row_ok[mb]) ? load_chunk<VEC>(xrow[mb], k, K) : zero;
    }
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][mb]), as_bf16x8(b[u]), acc[mb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  // output tile element (row (lane/16)*4 + v, column lane%16) of row block mb;
  // thread t sums the waves' partials in wave order
  for (int t = threadIdx.x; t < MB * 64; t += 64 * kSkinnyWaves) {
    const int mb = t >> 6, l = t & 63;
    floatx4 s = red[0][mb][l];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) s += red[w][mb][l];
    const int c = n0 + (l & 15);
    if (c < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = mb * 16 + (l >> 4) * 4 + v;
        if (r < M) Y[(size_t)r * N + c] = (uint16_t)f2bf(s[v]);
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
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

  // global chunk assignment: chunk c = tid + i*256 -> (row c/8, kchunk c%8)
  uint4 ra[kLoadsA], rb[kLoadsB];
  auto gload = [&](int kt) {
    const int kbase = kt * BK;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int c = tid + i * kTiledThreads, r = c >> 3, kc = c & 7;
      const int gr = m0 + r;
      ra[i] = (gr < M) ? load_chunk<VEC>(X + (size_t)gr * K, kbase + kc * 8, K) : zero;
    }
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
      const int c = tid + i * kTiledThreads, r = c >> 3, kc = c & 7;
      const int gr = n0 + r;
      rb[i] = (gr < N) ? load_chunk<VEC>(W + (size_t)gr * K, kbase + kc * 8, K) : zero;
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

template <bool VEC>
hipError_t launch_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, hipStream_t st) {
  if (M <= 64) {
    const dim3 grid((N + 15) / 16), block(64 * kSkinnyWaves);
    if (M <= 16) hipLaunchKernelGGL((gemm_skinny<1, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 32) hipLaunchKernelGGL((gemm_skinny<2, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else if (M <= 48) hipLaunchKernelGGL((gemm_skinny<3, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
    else hipLaunchKernelGGL((gemm_skinny<4, VEC>), grid, block, 0, st, X, W, Y, M, K, N);
  } else {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(kTiledThreads);
    hipLaunchKernelGGL((gemm_tiled<VEC>), grid, block, 0, st, X, W, Y, M, K, N);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_base_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N,
                            hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) % 16 == 0);
  return vec ? launch_gemm<true>(X, W, Y, M, K, N, stream) : launch_gemm<false>(X, W, Y, M, K, N, stream);
}

}  // namespace mlora
