// Internal declarations shared by the library's translation units: device
// helpers for bf16 data and the host-side launchers of every kernel.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "../../include/mlora.h"

namespace mlora {

// ----------------------------------------------------------------------------
// device helpers
// ----------------------------------------------------------------------------

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// two bf16 packed in a 32-bit word -> two floats
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

// the same rounding (RNE) by the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32), branch-free: for MFMA operands built in registers
__device__ __forceinline__ uint32_t pack_bf2_hw(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight consecutive bf16 of row `p` starting at element `i`, as floats.
// VEC: the row base and i are 16-byte aligned and i + 8 <= limit, so one
// 16-byte load serves; otherwise element loads, zero past `limit`.
template <bool VEC>
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, int i, int limit, float (&v)[8]) {
  if (VEC) {
    uint4 w = *reinterpret_cast<const uint4*>(p + i);
    v[0] = lo_bf(w.x); v[1] = hi_bf(w.x); v[2] = lo_bf(w.y); v[3] = hi_bf(w.y);
    v[4] = lo_bf(w.z); v[5] = hi_bf(w.z); v[6] = lo_bf(w.w); v[7] = hi_bf(w.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (i + e < limit) ? bf2f(p[i + e]) : 0.f;
  }
}

// ----------------------------------------------------------------------------
// host launchers (return hipSuccess or the launch error)
// ----------------------------------------------------------------------------

// The largest dynamic LDS size a group of kernels has been allowed so far.
// ensure() raises the limit of every kernel of the group to `bytes` when a
// launch needs more than before; the check and the raise happen under the
// mutex, so host threads launching different sizes never leave a kernel's
// limit below what one of them then requests.
struct LdsLimit {
  std::mutex mu;
  size_t bytes = 0;
  hipError_t ensure(std::initializer_list<const void*> fns, size_t need) {
    std::lock_guard<std::mutex> g(mu);
    if (need <= bytes) return hipSuccess;
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)need);
      if (e != hipSuccess) return e;
    }
    bytes = need;
    return hipSuccess;
  }
};

// pool metadata view on the device
struct PoolView {
  const int32_t* rank;       // [max_adapters]
  const float* scale;        // [max_adapters]
  const int32_t* down_page;  // [max_adapters][n_proj][max_rank]
  const int32_t* up_page;    // [max_adapters][n_proj][max_rank]
  const uint16_t* down;      // [n_down_pages][din]
  const uint16_t* up;        // [n_up_pages][dout]
  int32_t din, dout, n_proj, max_adapters, max_rank;
};

hipError_t launch_seg_build(const int32_t* row_adapter, int n, const int32_t* pool_rank, int max_adapters,
                            int32_t* ws, hipStream_t stream);

hipError_t launch_base_gemm(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N,
                            hipStream_t stream);

// Y = X W^T plus the per-row expand of T (scaled t per original row).  The
// decode (M <= 64) and medium (M <= 1024) forms split K over workgroups and
// need gemm_lora_part_floats() of fp32 scratch for the partials.  shrink:
// compute T first (the per-row shrink), in the GEMM's own launch where the
// decode form applies.
hipError_t launch_gemm_lora(const PoolView& pv, int proj, const uint16_t* X, const uint16_t* W, const int32_t* ws,
                            float* T, float* part, uint16_t* Y, int M, bool shrink, hipStream_t stream);
// The per-row plan of a decode (M <= 64) or medium (M <= 1024) batch with
// its segment build in the same GEMM launch: row keys come from the adapter
// ids `ids` and the resident table, and one workgroup of the launch writes
// the segment workspace `ws`.  hipErrorNotSupported (nothing launched) where
// neither the split-K decode form nor the co-resident medium form applies.
hipError_t launch_forward_rows(const PoolView& pv, int proj, const uint16_t* X, const uint16_t* W,
                               const int32_t* ids, int32_t* ws, float* T, float* part, uint16_t* Y, int M,
                               hipStream_t stream);
// T's region in the per-row work holds rows_t_slices(M) [M][max_rank]
// slices: a batch of at most 64 rows may take the decode form, which computes
// T as partials over its K slices (at most kDecMaxSlices) inside its GEMM
// launch; larger batches keep one slice (the finished T).
constexpr int kDecMaxSlices = 16;
__host__ __device__ constexpr int rows_t_slices(int M) { return M <= 64 ? kDecMaxSlices : 1; }
// Per-row descriptor of the per-row path, written by whichever kernel runs a
// row's shrink and read by the pass that adds the low-rank term (one
// dependent load less there: the adapter's pages come with the row instead
// of through the row's key): word 0 the row key (adapter id, -1 base-only,
// -2 invalid id), 1 the rank, 2 the scale (fp32 bits), 3 unused, 4.. the
// adapter's Up page ids for the projection (entries past the rank repeat the
// first page).  The descriptors follow the rows_t_slices(M) slices of T in T's
// region of the work buffer.
__host__ __device__ constexpr int row_desc_words(int max_rank) { return 4 + max_rank; }
__host__ __device__ inline int32_t* row_desc(float* T, int M, int max_rank) {
  return reinterpret_cast<int32_t*>(T + (size_t)rows_t_slices(M) * M * max_rank);
}
size_t gemm_lora_part_floats(int M, int N, int K);
// Y = X W^T alone on the split-K decode / medium forms, with fp32 scratch
// `part` of gemm_lora_part_floats(M, N, K) floats (a finish pass sums the
// partials); hipErrorNotSupported where those forms do not apply.
hipError_t launch_base_split(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int K, int N, float* part,
                             hipStream_t stream);

hipError_t launch_shrink_rows(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, int n, float* T,
                              hipStream_t stream);

// Operands of the large-batch GEMM's low-rank term, prepared per batch
// and projection by launch_lora_prep from the shrink's slices and the pool:
//   tb   bf16 [M][wt]: s_a * t per original row (ranks past the adapter's
//        are zero; rows not on a resident adapter are not written),
//   koff int32 [max_adapters]: for each adapter of the batch, the first
//        rank row of its block in upt (other entries are not written),
//   upt  bf16: per adapter a block [dout][r_pad(a)] at element koff[a] * dout
//        (Up with ranks contiguous, r_pad = rank rounded up to 16, zeros
//        past the rank), room for upt_units rank rows in all,
//   over int32 (when not null): written by lora_prep, nonzero when the
//        batch's blocks need more than upt_units rank rows; then upt is
//        incomplete, the GEMM leaves the low-rank term out and
//        launch_expand_over adds it.
// The rank-concatenated form, for batches whose adapters' r_pad sum to at
// most txw ranks (txw a multiple of 64, 0 = never): the low-rank term is
// then the product of two more K stages, [X | Tx] [W0 | Ux]^T, in the
// GEMM's own pipeline instead of its epilogue.
//   kx   int32 (when not null): written by lora_prep, the extra depth Kx
//        (the batch's r_pad sum rounded up to 64) or 0 when the batch does
//        not take this form; then tb and upt above are written instead,
//   tx   bf16 [M][txw]: row r holds s_a * t of its adapter a at columns
//        koff[a] .. koff[a] + rank - 1, zeros elsewhere below Kx; NaN below
//        Kx for a row with an invalid id,
//   Ux   bf16 [dout][txw] in the upt region: Up_a[c][q] at column
//        koff[a] + q, zeros elsewhere below Kx.
struct LoraOperands {
  const uint16_t* tb;
  const int32_t* koff;
  const uint16_t* upt;
  int wt;
  const int32_t* over = nullptr;
  const uint16_t* tx = nullptr;
  int txw = 0;
  const int32_t* kx = nullptr;
};
// the largest extra depth of the rank-concatenated form
constexpr int kMaxConcatRanks = 256;
inline int t_rows_width(int max_rank) { return (max_rank + 15) / 16 * 16; }
// Rank rows of upt for a batch of n rows at most: every adapter of the
// batch padded to the largest rank.
inline size_t lora_upt_units(int n, int max_adapters, int max_rank) {
  return (size_t)(n < max_adapters ? n : max_adapters) * t_rows_width(max_rank);
}

// Large batches: Y = X W^T plus every row's low-rank term, added inside the
// large GEMM (extra K tiles over the rank-concatenated operands, or its
// epilogue; no read-modify-write of Y); invalid rows become NaN.  big_lora_ok: the shapes and pointers this kernel takes.
bool big_lora_ok(const PoolView& pv, const uint16_t* X, const uint16_t* W, int M);
hipError_t launch_big_lora(const PoolView& pv, const uint16_t* X, const uint16_t* W, const int32_t* ws,
                           const LoraOperands& lo, uint16_t* Y, int M, hipStream_t stream);
// Writes tb, koff, upt and *over (see LoraOperands) from the shrink's slices
// Ts [n_chunks][n][max_rank] (sorted positions; t = sum over slices in
// order); upt has room for upt_units rank rows.
hipError_t launch_lora_prep(const PoolView& pv, int proj, const int32_t* ws, int n, const float* Ts, int n_chunks,
                            uint16_t* tb, int wt, int32_t* koff, uint16_t* upt, long upt_units, int32_t* over,
                            uint16_t* tx, int txw, int32_t* kx, hipStream_t stream);

hipError_t launch_shrink(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, int n,
                         float* T, int n_chunks, int chunk_elems, hipStream_t stream);
// Batches of at least this many rows run the shrink on the matrix cores per
// 64-row segment tile (when din allows); shrink_tile_cap bounds the tiles.
constexpr int kShrinkTilesMinRows = 256;
bool shrink_uses_tiles(const PoolView& pv, int n, const void* X);
int shrink_tile_cap(const PoolView& pv, int n);

hipError_t launch_expand(const PoolView& pv, int proj, const float* T, int n_chunks, const int32_t* ws,
                         uint16_t* Y, int n, hipStream_t stream);
// launch_expand whose workgroups return at once unless *over is nonzero (the
// large-batch GEMM then left the low-rank term out)
hipError_t launch_expand_over(const PoolView& pv, int proj, const float* T, int n_chunks, const int32_t* ws,
                              uint16_t* Y, int n, const int32_t* over, hipStream_t stream);

hipError_t launch_fused(const PoolView& pv, int proj, const uint16_t* X, const int32_t* ws, uint16_t* Y,
                        int n, hipStream_t stream);

hipError_t launch_hbm_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* out, hipStream_t stream);
hipError_t launch_hbm_read_lds(const void* src, size_t bytes, uint32_t* out, hipStream_t stream);
// W (bf16 [dout][din], in place) += f * Up_a Down_a for adapter a's rank-r
// factors of projection proj (f = +-scale), fp32 sum, bf16 RNE store
hipError_t launch_merge(const PoolView& pv, int adapter, int proj, int rank, float f, uint16_t* W,
                        hipStream_t stream);

// Launch timing: while armed, each kernel launch of the library takes the
// next pair of events, which the runtime stamps with the kernel's own start
// and end (hipExtLaunchKernel); `on` is false when nothing is armed.
struct TimingSlot {
  hipEvent_t start = nullptr, stop = nullptr;
  bool on = false;
};
TimingSlot timing_next(const char* kernel);

// Every kernel launch goes through this: a plain launch, or one that stamps
// the armed timing events.
#define MLORA_LAUNCH(name, kernel, grid, block, lds, stream, ...)                                       \
  do {                                                                                                  \
    const ::mlora::TimingSlot ts_ = ::mlora::timing_next(name);                                         \
    if (ts_.on)                                                                                         \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ts_.start, ts_.stop, 0u, __VA_ARGS__);    \
    else                                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                                \
  } while (0)

// the error of the launch just made
inline hipError_t launched() { return hipGetLastError(); }

}  // namespace mlora
