/*
 * mlora.h - C ABI of the MI355X (gfx950) heterogeneous multi-LoRA linear.
 *
 * The layer computes, for every row k of a mixed batch,
 *
 *     Y[k] = W0 x_k + s_a * Up_a (Down_a x_k),      a = row_adapter[k]
 *
 * with one base weight W0 shared by the whole batch and a low-rank term of
 * each row's own adapter (rank and scale per adapter; a row with id -1 has
 * no adapter and keeps the base output).  This is the shared-base /
 * per-row-delta form of the M031 card (xuujii.github.io/ai-infra-kb/details/
 * M031.html, section 02) and the per-query formula of the airsota card
 * (airsota.com/?p=1825, section three, derivation 1; its A is Down^T and its
 * B is Up^T).  Rows are grouped by adapter and each group's result is
 * written back to the rows it came from (M031 card sections 02-03; wiblog
 * article "vLLM LoRA adapter batch scheduling", Punica section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns an mlora_status; nothing throws, aborts or
 *    synchronises the device unless its comment says so.  On failure the
 *    thread-local string of mlora_last_error() says why.
 *  - "device" pointers are caller-owned device memory, only borrowed for the
 *    call.  "host" pointers are caller-owned host memory, not retained after
 *    the call returns.  The library never allocates device memory; it
 *    allocates host memory (pinned staging for pool loads) only inside
 *    mlora_pool_create.
 *  - bf16 tensors are passed as their uint16_t bit patterns (IEEE binary32
 *    with the low 16 bits dropped), row-major and densely packed.
 *  - All device work is enqueued on the caller's stream (`stream` is a
 *    hipStream_t; NULL means the default stream) and is asynchronous.
 *    Calls on one pool must be ordered by the caller: issue them on one
 *    stream, or synchronise between streams.
 *  - Data-dependent errors (a row id that is not -1 and not a resident
 *    adapter) cannot be returned without a device sync: they set bits in
 *    the segment status word and the affected output rows become NaN.
 *  - Full speed needs din and dout multiples of 8 and 16-byte aligned
 *    pointers; any din, dout >= 1 is computed correctly.
 */
#ifndef MLORA_H
#define MLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlora_status {
  MLORA_OK = 0,
  MLORA_EINVAL = 1, /* bad argument: null pointer, shape, rank, projection, size */
  MLORA_ENOSPC = 2, /* not enough free pages in the pool; nothing was changed   */
  MLORA_EEXIST = 3, /* load of an adapter id that is already resident          */
  MLORA_ENOENT = 4, /* unload of an adapter id that is not resident            */
  MLORA_EHIP = 5    /* a HIP runtime call or kernel launch failed              */
} mlora_status;

/* Apply variants.  AUTO lets the library choose; the others force one
 * implementation of the low-rank branch (all give the same result within
 * the bf16 tolerance, each is bitwise deterministic). */
typedef enum mlora_variant {
  MLORA_VARIANT_AUTO = 0,  /* ROWS up to 1024 rows, SPLIT above                  */
  MLORA_VARIANT_SPLIT = 1, /* base GEMM, then shrink kernel -> fp32 t in `work`
                              -> expand kernel (large batches: the expand inside
                              the GEMM instead, as extra K stages over the
                              ranks concatenated when the batch's ranks, each
                              rounded up to 16, sum to at most 256, else in its
                              epilogue, unless the batch's Up blocks overrun
                              the epilogue's 256 MiB operand budget; then an
                              expand follows the GEMM)                           */
  MLORA_VARIANT_FUSED = 2, /* base GEMM, then one kernel per work item of up to
                              MLORA_ITEM_ROWS rows: t stays on chip              */
  MLORA_VARIANT_ROWS = 3   /* n_rows <= 1024: the per-row shrink inside the
                              split-K base GEMM's launch, then a pass that sums
                              the K partials and adds each row's expand          */
} mlora_variant;
/* SPLIT and FUSED split the base GEMM's K over workgroups too (partials in
 * `work`) when n_rows <= 1024 and `work` holds mlora_work_bytes(); with a
 * smaller or absent buffer (FUSED needs none) they take the one-pass GEMM. */

/* Limits. */
#define MLORA_MAX_ROWS 16384        /* rows per batch (segment builder works in one workgroup) */
#define MLORA_MAX_RANK 128          /* largest adapter rank a pool may hold                   */
#define MLORA_MAX_ADAPTERS 65533    /* adapter ids are 0 .. max_adapters-1                    */
#define MLORA_ITEM_ROWS 4           /* rows per low-rank work item                            */
#define MLORA_TILE_ROWS 64          /* rows per segment tile (matrix-core shrink of big groups) */

/* Segment status bits (header word MLORA_SEG_STATUS). */
#define MLORA_SEG_BAD_ID 1          /* an id < -1 or >= max_adapters appeared                 */
#define MLORA_SEG_NOT_RESIDENT 2    /* an id named an adapter with no weights loaded          */

/* ---------------------------------------------------------------------------
 * Library information
 * ------------------------------------------------------------------------- */
const char* mlora_version(void);
const char* mlora_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* mlora_last_error(void);

/* ---------------------------------------------------------------------------
 * Rank-stacked paged adapter pool
 *
 * One page holds one rank row of one adapter for one projection: the Down
 * arena has pages of din bf16 (a row of Down), the Up arena pages of dout
 * bf16 (a column of Up, i.e. a row of Up^T).  An adapter of rank r takes
 * n_proj * r pages in each arena, wherever they are free: no padding to the
 * largest rank, and adapters of different ranks share one pool.  This is
 * the adapter half of the unified paging the M031 card (section 06) and the
 * wiblog article (memory-cost section) point to, sized by the card's
 * section 06 arithmetic (rank 16 over a 4096 x 4096 projection is 0.25 MiB).
 *
 * Device metadata (the `meta` buffer, mlora_pool_meta_bytes() long, 256-byte
 * aligned regions in this order):
 *   int32 rank[max_adapters]                        0 = not resident
 *   float scale[max_adapters]
 *   int32 down_page[max_adapters][n_proj][max_rank] page index, -1 past rank
 *   int32 up_page  [max_adapters][n_proj][max_rank]
 * ------------------------------------------------------------------------- */
typedef struct mlora_pool mlora_pool; /* opaque host handle */

typedef struct mlora_pool_desc {
  int32_t din;          /* input features of the projection(s), >= 1          */
  int32_t dout;         /* output features, >= 1                               */
  int32_t n_proj;       /* projections (layers x modules) per adapter, >= 1    */
  int32_t max_adapters; /* adapter ids are 0 .. max_adapters-1                 */
  int32_t max_rank;     /* 1 .. MLORA_MAX_RANK                                 */
  int32_t reserved;     /* must be 0                                           */
  int64_t n_down_pages; /* pages in the Down arena                             */
  int64_t n_up_pages;   /* pages in the Up arena                               */
  void* down_pages;     /* device bf16 [n_down_pages][din]                     */
  void* up_pages;       /* device bf16 [n_up_pages][dout]                      */
  void* meta;           /* device, mlora_pool_meta_bytes() bytes, 256-aligned  */
} mlora_pool_desc;

size_t mlora_pool_meta_bytes(int32_t max_adapters, int32_t n_proj, int32_t max_rank);

/* Creates the host handle of an adapter pool in HBM (M031 card, section
 * 06: adapters kept in GPU memory as pages, the pool sized by max_adapters
 * and max_rank; wiblog article, memory cost: one paged pool for every
 * adapter), binds it to the current device and clears the device metadata
 * on `stream` (no adapter resident).  The three device buffers stay owned
 * by the caller and must outlive the pool.  Errors: MLORA_EINVAL for a
 * descriptor outside the documented ranges or misaligned buffers,
 * MLORA_EHIP. */
mlora_status mlora_pool_create(const mlora_pool_desc* desc, void* stream, mlora_pool** out);
/* Releases the host handle after waiting for the pool's own pending copies
 * (M031 card, section 07: an adapter's storage goes only after its last
 * reader); the caller frees the device buffers afterwards.  Errors:
 * MLORA_EINVAL for NULL, MLORA_EHIP if a pending copy failed. */
mlora_status mlora_pool_destroy(mlora_pool* pool);

/* Loads adapter `adapter_id` with the given rank and scale:
 *   down: host bf16 [n_proj][rank][din]   (Down, the "lora A" layout)
 *   up:   host bf16 [n_proj][dout][rank]  (Up,   the "lora B" layout)
 * Pages are taken from the free lists, Up is transposed to rank-major rows
 * on the host, and the pages plus metadata are copied on `stream` from
 * pinned staging.  The caller's buffers may be reused when this returns.
 * The weights are ready for any later call on the same stream (the card's
 * lifecycle: weights must be resident before the branch runs); a call on
 * another stream first makes that stream wait with mlora_pool_ready, so a
 * load on a copy stream can overlap the layer running on a compute stream.
 * Pages an unload parked (below) are reused only after `stream` waits, on
 * the device, for their last readers; the host does not block on readers.
 * Errors: EINVAL (id, rank, pointers), EEXIST (already resident: no silent
 * overwrite of a live id), ENOSPC (not enough free pages; nothing changed). */
mlora_status mlora_pool_load(mlora_pool* pool, int32_t adapter_id, int32_t rank, float scale,
                             const uint16_t* down, const uint16_t* up, void* stream);

/* Marks the adapter not resident (rank 0, on `stream`) and parks its pages
 * behind an event recorded on `stream`: every reader enqueued on `stream`
 * before the unload finishes before a later load, on ANY stream, writes
 * those pages (the M031 card, sections 06-07: evict only after the last
 * reader).  Readers on other streams must be ordered before the unload by
 * the caller (an event, as for any buffer).  Parked pages count as free in
 * mlora_pool_free_pages.  Errors: EINVAL (id range), ENOENT (not resident). */
mlora_status mlora_pool_unload(mlora_pool* pool, int32_t adapter_id, void* stream);

/* Makes `stream` wait, on the device, until the copies of the adapter's
 * latest load (possibly issued on another stream) have completed: the
 * adapter's weights and metadata are then visible to work enqueued on
 * `stream` afterwards.  The host does not block.
 * Errors: EINVAL (id range), ENOENT (not resident). */
mlora_status mlora_pool_ready(mlora_pool* pool, int32_t adapter_id, void* stream);

/* Testing aid for the load's error path: the next mlora_pool_load on this
 * pool fails with MLORA_EHIP at `step` once its copies are staged (1:
 * before its last staging flush, whose copies carry the metadata; 2: after
 * the metadata copies, before the ready event is recorded); 0 turns it off.
 * A load that fails there, as after any failure once its copies may have
 * been issued, leaves the adapter not resident on the host and on the
 * device (its rank is set back to 0 on the stream) and parks its pages
 * behind an event on the stream, as an unload does.  Errors: EINVAL. */
mlora_status mlora_pool_fail_next_load(mlora_pool* pool, int32_t step);

/* Host-side view of the pool (no device access). */
mlora_status mlora_pool_query(const mlora_pool* pool, int32_t adapter_id, int32_t* rank, float* scale);
mlora_status mlora_pool_free_pages(const mlora_pool* pool, int64_t* free_down, int64_t* free_up,
                                   int32_t* n_resident);

/* ---------------------------------------------------------------------------
 * Segment builder: groups the batch's rows by adapter (M031 card sections
 * 02-03: group order ascending by adapter, original order inside a group,
 * results written back to the original rows; the map is rebuilt for every
 * batch as requests join and leave).  It is a stable sort of rows by key,
 * key = adapter id for a row on a resident adapter, then all base-only rows
 * (id -1), then all rows with an invalid id.  Bit-exact and deterministic.
 *
 * seg_ws layout (int32 words; n = n_rows; mlora_segments_bytes(n) bytes):
 *   [0..16)            header, indices MLORA_SEG_*
 *   perm[n]            at MLORA_SEG_PERM(n):  sorted position -> original row
 *   inv[n]             at MLORA_SEG_INV(n):   original row -> sorted position
 *   seg_adapter[n]     at MLORA_SEG_ADAPTER(n): adapter of segment s (nseg used)
 *   seg_off[n+1]       at MLORA_SEG_OFF(n):   first sorted position of s;
 *                                             seg_off[nseg] = n_act
 *   items[2*max_items] at MLORA_SEG_ITEMS(n): work items (segment, first
 *                      sorted position), each covering up to MLORA_ITEM_ROWS
 *                      rows of one segment, in segment order.
 *   row_key[n]         at MLORA_SEG_ROWKEY(n): per original row, the
 *                      adapter id if resident, -1 for a base-only row, -2
 *                      for an invalid id (what the per-row kernels read).
 *   tiles[2*n]         at MLORA_SEG_TILES(n): (segment, first sorted
 *                      position) of every MLORA_TILE_ROWS-row tile of every
 *                      segment, in segment order: tile t of segment s
 *                      starts at seg_off[s] + t * MLORA_TILE_ROWS; header
 *                      word MLORA_SEG_NTILES holds the count.
 * ------------------------------------------------------------------------- */
#define MLORA_SEG_NSEG 0
#define MLORA_SEG_NACT 1
#define MLORA_SEG_NNONE 2
#define MLORA_SEG_NBAD 3
#define MLORA_SEG_STATUS 4
#define MLORA_SEG_NITEMS 5
#define MLORA_SEG_NROWS 6
#define MLORA_SEG_MAXAD 7
#define MLORA_SEG_NTILES 8
#define MLORA_SEG_HEADER 16
#define MLORA_SEG_PERM(n) (MLORA_SEG_HEADER)
#define MLORA_SEG_INV(n) (MLORA_SEG_HEADER + (n))
#define MLORA_SEG_ADAPTER(n) (MLORA_SEG_HEADER + 2 * (n))
#define MLORA_SEG_OFF(n) (MLORA_SEG_HEADER + 3 * (n))
#define MLORA_SEG_ITEMS(n) ((MLORA_SEG_HEADER + 4 * (n) + 2) & ~1)
#define MLORA_SEG_MAX_ITEMS(n) ((n) + ((n) + MLORA_ITEM_ROWS - 1) / MLORA_ITEM_ROWS + 1)
#define MLORA_SEG_ROWKEY(n) (MLORA_SEG_ITEMS(n) + 2 * MLORA_SEG_MAX_ITEMS(n))
#define MLORA_SEG_TILES(n) (MLORA_SEG_ROWKEY(n) + (n))

size_t mlora_segments_bytes(int32_t n_rows);

/* row_adapter: device int32 [n_rows]; seg_ws: device, mlora_segments_bytes().
 * Reads the pool's device rank table to tell resident ids from others. */
mlora_status mlora_build_segments(const mlora_pool* pool, const int32_t* row_adapter, int32_t n_rows,
                                  void* seg_ws, void* stream);

/* Copies the 16-word header of seg_ws to host `header` and SYNCHRONISES the
 * stream (for tests and for callers that want to check the status word). */
mlora_status mlora_segments_header(const void* seg_ws, int32_t* header, void* stream);

/* The batch's status word alone (MLORA_SEG_BAD_ID | MLORA_SEG_NOT_RESIDENT,
 * 0 when every id was -1 or a resident adapter) copied to host `status`;
 * SYNCHRONISES the stream.  The rows behind a nonzero status are NaN rows in
 * Y: a request bound to an id that is not loaded is reported, never served
 * by another adapter (M031 card, section 03: a wrong write-back is wrong
 * semantics even without a shape error; section 07: weights resident
 * before use).  Errors: MLORA_EINVAL for a NULL pointer, MLORA_EHIP. */
mlora_status mlora_segments_status(const void* seg_ws, int32_t* status, void* stream);

/* ---------------------------------------------------------------------------
 * The steps of the layer, each usable on its own
 * ------------------------------------------------------------------------- */

/* Base GEMM over the whole batch, Y = X W0^T (the card's shared-base step):
 *   X: device bf16 [n_rows][din], W0: device bf16 [dout][din],
 *   Y: device bf16 [n_rows][dout] (overwritten).
 * bf16 inputs, fp32 accumulation on the matrix cores, bf16 output (RNE). */
mlora_status mlora_base_gemm(const uint16_t* X, const uint16_t* W0, uint16_t* Y, int32_t n_rows,
                             int32_t din, int32_t dout, void* stream);

/* Shrink, t = Down_a x_k for every row on a resident adapter, rows gathered
 * through perm (each group computes its own Down product):
 *   T: device fp32 [n_chunks][n_rows][max_rank]; row j is sorted position j,
 *   column q < rank of its segment; chunk c holds the partial sum over the
 *   c-th of n_chunks equal slices of din (slices are multiples of 512
 *   elements; a slice past din contributes zeros), so t = sum over c.
 *   Entries of rows past n_act and columns past the rank are not written.
 *   1 <= n_chunks <= mlora_shrink_max_chunks(din). */
int32_t mlora_shrink_max_chunks(int32_t din);
mlora_status mlora_shrink(const mlora_pool* pool, int32_t proj, const uint16_t* X, const void* seg_ws,
                          int32_t n_rows, float* T, int32_t n_chunks, void* stream);

/* Expand, Y[perm[j]] += s_a * Up_a t_j (read-modify-write in fp32, stored as
 * bf16 RNE; no atomics: one thread owns each output element), with t_j the
 * sum over the n_chunks partials of T (layout as mlora_shrink; 1 <= n_chunks
 * <= 1024, summed in slice order).  Rows with
 * an invalid id are set to NaN; base-only rows are untouched. */
mlora_status mlora_expand(const mlora_pool* pool, int32_t proj, const float* T, int32_t n_chunks,
                          const void* seg_ws, uint16_t* Y, int32_t n_rows, void* stream);

/* Fused shrink + expand: Y[perm[j]] += s_a * Up_a (Down_a x_perm[j]) with t
 * kept on chip, one workgroup per work item (for decode steps, where most
 * groups hold one or a few tokens).  Invalid rows become NaN. */
mlora_status mlora_fused(const mlora_pool* pool, int32_t proj, const uint16_t* X, const void* seg_ws,
                         uint16_t* Y, int32_t n_rows, void* stream);

/* Per-row path (decode-sized batches, n_rows <= 1024), in two calls that
 * share the caller's `work` buffer (mlora_work_bytes() long, 256-byte
 * aligned).  Its first n_rows * max_rank floats hold T: T[k][q] = s_a *
 * (Down_a x_k)[q] for every row k on a resident adapter a, q < rank(a), in
 * ORIGINAL row order (rows read directly by index, as the M031 card's
 * section 02 allows instead of regrouping); other entries are not written.
 * After the T slices, T's region holds a descriptor per row (its adapter,
 * rank, scale and Up pages) that mlora_shrink_rows writes and
 * mlora_gemm_lora reads.  The rest of `work` is the GEMM's scratch (split-K
 * partials), so the two calls go in this order on one stream, and calls
 * that share a `work` buffer must not overlap.  mlora_apply with ROWS computes the same T and Y; for
 * decode shapes it runs the per-row shrink as extra workgroups of the GEMM
 * launch (two kernels in all: GEMM + shrink, then partial sums + expand). */
mlora_status mlora_shrink_rows(const mlora_pool* pool, int32_t proj, const uint16_t* X, const void* seg_ws,
                               int32_t n_rows, void* work, size_t work_bytes, void* stream);

/* Base GEMM with the expand of the low-rank branch in the same kernel:
 * Y = X W0^T, plus for every row k on a resident adapter sum_q T[k][q]
 * Up_a[:, q] with T from mlora_shrink_rows in `work`; rows with an invalid
 * id become NaN; base-only rows get the plain product.  Y is written once. */
mlora_status mlora_gemm_lora(const mlora_pool* pool, int32_t proj, const uint16_t* X, const uint16_t* W0,
                             const void* seg_ws, void* work, size_t work_bytes, uint16_t* Y, int32_t n_rows,
                             void* stream);

/* ---------------------------------------------------------------------------
 * The whole layer for one projection of one batch (M031 card, section 02:
 * one base product shared by all rows, each row's low-rank term from its
 * own adapter written back at its original row; section 03 worked example):
 *   Y = X W0^T, then every row's low-rank term added at its original row.
 *   X: device bf16 [n_rows][din]; W0: device bf16 [dout][din] (projection
 *   `proj`'s base weight); Y: device bf16 [n_rows][dout] (overwritten);
 *   seg_ws from mlora_build_segments on the same rows (reusable for every
 *   projection of the batch); work: device scratch of at least
 *   mlora_work_bytes(pool, n_rows) bytes, 256-byte aligned.
 * n_rows = 0 is a no-op.
 * ------------------------------------------------------------------------- */
/* mlora_work_bytes: the scratch any variant of mlora_apply needs for a batch
 * of n_rows on this pool (t per row and rank, split-K partials, the
 * large GEMM's low-rank operands); 0 for a NULL pool or n_rows < 0.  Host
 * only. */
size_t mlora_work_bytes(const mlora_pool* pool, int32_t n_rows);

/* The launch plan mlora_apply follows for `variant` (AUTO resolved) on a
 * batch of n_rows: the variant it runs and, for SPLIT, the number of din
 * slices of its shrink (the n_chunks of mlora_shrink/mlora_expand).  ROWS
 * is only valid for n_rows <= 1024.
 * Host only; lets a caller run the same steps one by one. */
mlora_status mlora_plan(const mlora_pool* pool, int32_t n_rows, int32_t variant, int32_t* out_variant,
                        int32_t* out_chunks);

mlora_status mlora_apply(const mlora_pool* pool, int32_t proj, const uint16_t* X, const uint16_t* W0,
                         const void* seg_ws, uint16_t* Y, int32_t n_rows, void* work, size_t work_bytes,
                         int32_t variant, void* stream);

/* Segment build and the layer for one projection in a single call: what
 * mlora_build_segments(pool, row_adapter, n_rows, seg_ws) followed by
 * mlora_apply(pool, proj, X, W0, seg_ws, Y, n_rows, work, work_bytes,
 * variant) computes (M031 card, sections 02-03: group the batch's rows by
 * adapter, one shared base product, each row's low-rank term back at its
 * original row), with the same results in Y, seg_ws and work.
 *   row_adapter: device int32 [n_rows], as for mlora_build_segments;
 *   seg_ws: device, mlora_segments_bytes(n_rows) bytes, 8-byte aligned;
 *   the other arguments as for mlora_apply.
 * For the per-row plan (16-byte aligned operands) at decode sizes
 * (n_rows <= 64, din a multiple of 128 from 512 to 16384) and medium ones (65 ..
 * 1024 rows, din a multiple of 128) the segment build runs in a workgroup
 * of the base GEMM's launch, whose
 * other workgroups take each row's key from row_adapter and the resident
 * table directly: one launch fewer on the stream.  Otherwise the two calls
 * run one after the other.
 * seg_ws stays valid for mlora_apply on further projections of the batch.
 * Errors: those of the two calls; nothing is launched on an argument error. */
mlora_status mlora_forward(const mlora_pool* pool, int32_t proj, const uint16_t* X, const uint16_t* W0,
                           const int32_t* row_adapter, void* seg_ws, uint16_t* Y, int32_t n_rows, void* work,
                           size_t work_bytes, int32_t variant, void* stream);

/* mlora_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results as mlora_forward, with the `work` buffer
 * replaced by scratch the library owns, a static device array of
 * MLORA_STATIC_SCRATCH_BYTES on each GPU it runs on (held until the process
 * ends).  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); the caller still passes X, W0, row_adapter, seg_ws and
 * Y as for mlora_forward.  Every call on a GPU uses that GPU's one scratch
 * array, whose contents stay from the last call: calls that overlap on one
 * GPU (concurrent streams or host threads) race and must be ordered by the
 * caller.  Errors: those of mlora_forward, and MLORA_EINVAL for a batch
 * whose launch plan needs more scratch than MLORA_STATIC_SCRATCH_BYTES
 * (nothing is launched then).  The per-row plan of 256 rows at dout = 4096
 * needs 16.1 MiB (512 rows, which split K in two, about the same); the
 * split plan of 4096 rows over six adapters of rank <= 64 at dout = 11008
 * needs 17 MB; pools with many adapter slots of large rank need more (the
 * split plan's per-adapter Up blocks) and take mlora_forward. */
#define MLORA_STATIC_SCRATCH_BYTES (20u << 20)
mlora_status mlora_forward_static(const mlora_pool* pool, int32_t proj, const uint16_t* X, const uint16_t* W0,
                                  const int32_t* row_adapter, void* seg_ws, uint16_t* Y, int32_t n_rows,
                                  int32_t variant, void* stream);

/* ---------------------------------------------------------------------------
 * The merged alternative (M031 card, section 04: W_merged = W_base + scale *
 * Up Down serves that one adapter with a plain GEMM; airsota card, section
 * three, derivation 2): adds, or with sign = -1 takes out, one resident
 * adapter's low-rank term into a base weight IN PLACE:
 *   W0[c][i] <- bf16_rne( W0[c][i] + sign * s_a * sum_q Up_a[c][q] Down_a[q][i] )
 * with the sum over q < rank(a) in fp32, in rank order.
 *   W0: device bf16 [dout][din] of projection `proj` (read and written);
 *   sign: +1 merges, -1 unmerges (any finite factor is accepted; an unmerge
 *   restores W0 only up to the bf16 rounding of the two stores).
 * Returns MLORA_ENOENT if the adapter is not resident, MLORA_EINVAL for a bad
 * id, projection, NULL W0 or non-finite sign.  Rows of a merged weight give
 * the adapter's output through mlora_base_gemm (or mlora_apply with id -1);
 * rows of other adapters must not be served from it.
 * ------------------------------------------------------------------------- */
mlora_status mlora_merge(const mlora_pool* pool, int32_t adapter_id, int32_t proj, uint16_t* W0, float sign,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers: a plain streaming copy (dst = src, `bytes` a multiple
 * of 16, both 16-byte aligned), used to calibrate achievable HBM bandwidth
 * and hardware byte counters against a kernel of known traffic.
 * ------------------------------------------------------------------------- */
mlora_status mlora_hbm_copy(void* dst, const void* src, size_t bytes, void* stream);

/* The read half of the same measurement: streams `bytes` from src (a
 * multiple of 16, 16-byte aligned) and XORs every 32-bit word read into
 * *out (device uint32, caller-owned; the caller clears it first), so the
 * achievable streaming read rate can be measured.  Errors: EINVAL, EHIP. */
mlora_status mlora_hbm_read(const void* src, size_t bytes, uint32_t* out, void* stream);

/* The same read through LDS DMA (buffer loads into LDS, the path by which
 * the ring GEMMs fetch X, W0 and the rank-concatenated operands), so that a
 * byte counter's reading for that path can be calibrated as well: streams
 * `bytes` from src (a multiple of 1024 up to 2^31 - 1, 16-byte aligned) in
 * 1 KiB pieces and XORs a few of the words received into *out (device
 * uint32, caller-owned).  Errors: EINVAL, EHIP. */
mlora_status mlora_hbm_read_lds(const void* src, size_t bytes, uint32_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Launch timing, a measurement aid that changes no result.
 * mlora_timing_arm(n) arms the library's next n kernel launches (1..2048),
 * from any entry point: each is made with a pair of HIP events that the
 * runtime stamps when that kernel starts and ends on the GPU.
 * mlora_timing_read disarms, sets *out_n to the number of launches marked,
 * and, if `capacity` holds them, waits for their events and writes ms[i],
 * launch i's kernel duration in milliseconds; otherwise it fails with
 * MLORA_EINVAL.  mlora_timing_name(i) is the kernel of launch i (a static
 * string; NULL past the marked launches).  Not for use while a stream is
 * captured into a graph; one armed sequence per process at a time.
 * ------------------------------------------------------------------------- */
mlora_status mlora_timing_arm(int32_t n_launches);
mlora_status mlora_timing_read(float* ms, int32_t capacity, int32_t* out_n);
const char* mlora_timing_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* MLORA_H */
