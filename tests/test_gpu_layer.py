"""GPU parity of every step of the layer against the CPU oracle, called
through the C ABI: base GEMM, shrink, expand, fused shrink+expand and the
whole apply (both variants) on the named workloads and on ragged and edge
shapes.  Bar: max |Y - ref| <= 2e-2 (1 + |ref|) element-wise (bf16 inputs,
fp32 accumulation), ref in fp64 from the oracle on the same bf16 inputs."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import (TOL, assert_close, dev_to_f64, ids_dev, make_pool, oracle_adapters, say, to_dev_bf16,
                         torch_cuda)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


# ------------------------------------------------------------------ base GEMM

GEMM_SHAPES = [(1, 4, 4), (4, 4, 4), (3, 5, 7), (16, 64, 16), (17, 72, 33), (32, 4096, 4096), (33, 1000, 520),
               (48, 40, 1000), (64, 520, 1000), (65, 4096, 300), (200, 136, 136), (300, 1000, 777),
               (256, 4096, 4096), (513, 264, 392),
               # medium batches on the K-split kernel, incl. K tails and unaligned K
               (65, 4096, 4096), (129, 520, 4104), (700, 1000, 2000), (100, 20, 4096), (512, 4096, 4096),
               # large products: 128x128 co-resident tiles where 256x256 tiles would underfill the chip
               (2048, 1024, 2048), (2100, 640, 2200), (1030, 4096, 4104),
               # 256x256 tiles: full tiles, ragged M and N, the shortest K (two stages)
               (4096, 256, 4096), (4000, 384, 4000), (4096, 128, 4096),
               # ring tiles with N % 4 != 0: element stores instead of 4-column stores
               (100, 512, 777), (2100, 512, 2203)]


@pytest.mark.parametrize("m,k,n", GEMM_SHAPES)
def test_base_gemm(M, m, k, n):
    w = synth.custom("gemm", 3000 + m + k + n, k, n, np.full(m, -1, np.int32), {0: 1})
    X, W0 = w.x_bits(), w.w0_bits()
    say(f"base_gemm M={m} K={k} N={n}")
    Y = M.base_gemm(to_dev_bf16(X), to_dev_bf16(W0))
    ref = O.widen_bf16(X) @ O.widen_bf16(W0).T
    assert_close(dev_to_f64(Y), ref, f"gemm {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", [(100, 512, 776), (2100, 512, 2200)])
def test_base_gemm_unaligned_output(M, m, k, n):
    """Y two bytes past an 8-byte boundary: the ring tiles' 4-column stores
    need 8-byte alignment and fall back to element stores."""
    import torch
    w = synth.custom("gemm", 3100 + m + n, k, n, np.full(m, -1, np.int32), {0: 1})
    X, W0 = w.x_bits(), w.w0_bits()
    say(f"base_gemm unaligned Y M={m} K={k} N={n}")
    buf = torch.full((m * n + 4,), float("nan"), dtype=torch.bfloat16, device="cuda")
    Y = buf[1:1 + m * n].view(m, n)
    M.base_gemm(to_dev_bf16(X), to_dev_bf16(W0), Y)
    ref = O.widen_bf16(X) @ O.widen_bf16(W0).T
    assert_close(dev_to_f64(Y), ref, f"gemm unaligned {m}x{k}x{n}")
    edges = buf[[0, m * n + 1, m * n + 2, m * n + 3]].float()
    assert torch.isnan(edges).all(), "a store left the output"


def test_hbm_read_kernels(M):
    """The calibration reads run to completion on a buffer of known size:
    the plain read's XOR of all words is the host's, and the LDS-DMA read
    (1 KiB pieces) accepts whole KiB only."""
    import torch
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")  # 4 MiB
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.hbm_read(src, out)
    want = np.bitwise_xor.reduce(np.arange(1 << 20, dtype=np.int64)).astype(np.int32)
    assert int(out.item()) == int(want)
    out.zero_()
    M.hbm_read_lds(src, out)
    torch.cuda.synchronize()
    with pytest.raises(M.MloraError):
        M.hbm_read_lds(src, out, nbytes=1000)


def test_base_gemm_prefill_full_size(M):
    """The prefill workload's base product (4096 x 4096 -> 11008) at full
    size, every element against the fp64 product."""
    w = synth.prefill_hetero()
    X, W0 = w.x_bits(), w.w0_bits()
    say("base_gemm 4096x4096x11008")
    Y = dev_to_f64(M.base_gemm(to_dev_bf16(X), to_dev_bf16(W0)))
    ref = O.widen_bf16(X) @ O.widen_bf16(W0).T
    assert_close(Y, ref, "gemm prefill")


# ------------------------------------------------------------------ workloads for the branch

def small_workload(seed, din, dout, n, ranks, p_none=0.15, n_proj=1, max_rank=None):
    ids = synth.random_ids(seed, n, sorted(ranks), p_none)
    return synth.custom(f"small{seed}", seed, din, dout, ids, ranks, n_proj=n_proj,
                        max_adapters=max(ranks) + 1, max_rank=max_rank or max(ranks.values()))


SMALL = [
    # (seed, din, dout, n, ranks)
    (1, 64, 64, 9, {0: 1, 1: 2, 2: 3}),
    (2, 512, 520, 37, {0: 16, 3: 8, 5: 64}),
    (3, 1000, 1544, 130, {0: 16, 1: 1, 2: 17, 4: 33}),
    (4, 12, 20, 23, {0: 4, 1: 7}),                    # din, dout not multiples of 8: element-wise path
    (5, 4104, 136, 70, {i: 16 for i in range(20)}),   # many one/two-row groups
    (6, 256, 11008, 40, {0: 64, 1: 128}),              # rank up to the limit, wide dout
    # >= 256 rows: the matrix-core shrink over 64-row segment tiles
    (7, 4128, 264, 300, {0: 1, 1: 8, 2: 17, 3: 64, 4: 128}),   # din = 32 * 129: K tail, empty slices
    (8, 512, 1000, 700, {i: (16 if i % 3 else 64) for i in range(40)}),
    (9, 1000, 520, 260, {0: 16, 1: 3, 2: 64}),        # din not a multiple of 32: vector-ALU shrink
    (10, 520, 1000, 13, {0: 16, 1: 5, 2: 9}),          # ranks <= 16, din and dout <= 4096: fused fast form
    (12, 640, 1000, 200, {0: 16, 1: 5, 2: 9}),         # medium rows, K one ring split deep, ranks <= 16
]
LARGE = [
    # large batch on the 256x256 GEMM with the low-rank epilogue, ragged rows and columns
    (11, 512, 4000, 4000, {0: 8, 1: 16, 2: 64, 3: 1, 4: 33}),
]


def _prepare(M, w, proj=0):
    pool = make_pool(M, w)
    X = w.x_bits()
    seg = O.segments(w.row_adapter, w.max_adapters, w.adapter_ids())
    seg_ws = M.build_segments(pool, ids_dev(w.row_adapter))
    return pool, X, seg, seg_ws


@pytest.mark.parametrize("case", SMALL + [(None, "decode_3"), (None, "decode_frag"), (None, "prefill")],
                         ids=lambda c: str(c[0] if c[0] is not None else c[1]))
def test_shrink(M, case):
    if case[0] is None:
        w = synth.NAMED[case[1]]()
    else:
        w = small_workload(*case)
    pool, X, seg, seg_ws = _prepare(M, w)
    ad = oracle_adapters(w)
    ref = O.shrink_rows(O.widen_bf16(X), w.row_adapter, ad, w.max_adapters)
    Xd = to_dev_bf16(X)
    for chunks in sorted({1, M.shrink_max_chunks(w.din), min(3, M.shrink_max_chunks(w.din))}):
        say(f"shrink {w.name} chunks={chunks}")
        T = M.shrink(pool, 0, Xd, seg_ws, n_chunks=chunks).cpu().numpy().astype(np.float64).sum(axis=0)
        inv = seg["inv"]
        for k, t in ref.items():
            got = T[inv[k], : len(t)]
            assert_close(got, t, f"shrink {w.name} row {k}")


@pytest.mark.parametrize("case", SMALL + [(None, "decode_3"), (None, "decode_frag"), (None, "layer_stack")],
                         ids=lambda c: str(c[0] if c[0] is not None else c[1]))
def test_shrink_rows(M, case):
    """Per-row shrink: T[k] = s * Down_a x_k in original row order."""
    w = synth.NAMED[case[1]]() if case[0] is None else small_workload(*case)
    if w.n_proj > 1:
        w = synth.custom(w.name, w.seed, w.din, w.dout, w.row_adapter, w.ranks, scales=w.scales,
                         max_adapters=w.max_adapters, max_rank=w.max_rank, down_std=1 / 64)
    pool, X, seg, seg_ws = _prepare(M, w)
    ad = oracle_adapters(w)
    ref = O.shrink_rows(O.widen_bf16(X), w.row_adapter, ad, w.max_adapters)
    say(f"shrink_rows {w.name}")
    work = M.shrink_rows(pool, 0, to_dev_bf16(X), seg_ws)
    T = M.rows_t(pool, work, w.n).cpu().numpy().astype(np.float64)
    for k, t in ref.items():
        a = int(w.row_adapter[k])
        assert_close(T[k, : len(t)], w.scales[a] * t, f"shrink_rows {w.name} row {k}")


@pytest.mark.parametrize("case", SMALL + [(None, "decode_3"), (None, "decode_frag")],
                         ids=lambda c: str(c[0] if c[0] is not None else c[1]))
def test_expand(M, case):
    torch = torch_cuda()
    w = synth.NAMED[case[1]]() if case[0] is None else small_workload(*case)
    pool, X, seg, seg_ws = _prepare(M, w)
    ad = oracle_adapters(w)
    for chunks in (1, 2):
        Tn = synth.draw_t(w.seed, w.n, w.max_rank, chunks)
        Yin = synth.draw_bf16(w.seed + chunks, (w.n, w.dout))
        say(f"expand {w.name} chunks={chunks}")
        Y = to_dev_bf16(Yin)
        M.expand(pool, 0, torch.from_numpy(Tn).cuda(), seg_ws, Y)
        tsum = Tn.astype(np.float64).sum(axis=0)
        t_rows = {k: tsum[seg["inv"][k], : w.ranks[int(a)]] for k, a in enumerate(w.row_adapter) if a >= 0}
        ref = O.expand_rows(O.widen_bf16(Yin), t_rows, w.row_adapter, ad, w.max_adapters)
        assert_close(dev_to_f64(Y), ref, f"expand {w.name}")


@pytest.mark.parametrize("case", SMALL + [(None, "decode_3"), (None, "decode_frag")],
                         ids=lambda c: str(c[0] if c[0] is not None else c[1]))
def test_fused(M, case):
    w = synth.NAMED[case[1]]() if case[0] is None else small_workload(*case)
    pool, X, seg, seg_ws = _prepare(M, w)
    ad = oracle_adapters(w)
    Yin = synth.draw_bf16(w.seed + 11, (w.n, w.dout))
    say(f"fused {w.name}")
    Y = to_dev_bf16(Yin)
    M.fused(pool, 0, to_dev_bf16(X), seg_ws, Y)
    t = O.shrink_rows(O.widen_bf16(X), w.row_adapter, ad, w.max_adapters)
    ref = O.expand_rows(O.widen_bf16(Yin), t, w.row_adapter, ad, w.max_adapters)
    assert_close(dev_to_f64(Y), ref, f"fused {w.name}")


# ------------------------------------------------------------------ whole layer

def check_apply(M, w, projs=(0,), rows=None, variants=None, pool=None, w0_zero=False):
    if variants is None:
        variants = ("split", "fused", "rows") if w.n <= 1024 else ("split", "fused")
    pool = pool or make_pool(M, w)
    X = w.x_bits()
    Xd = to_dev_bf16(X)
    seg_ws = M.build_segments(pool, ids_dev(w.row_adapter))
    seg = O.segments(w.row_adapter, w.max_adapters, w.adapter_ids())
    sel = rows(seg) if callable(rows) else rows
    errs = {}
    for p in projs:
        W0 = np.zeros((w.dout, w.din), np.uint16) if w0_zero else w.w0_bits(p)
        W0d = to_dev_bf16(W0)
        ad = oracle_adapters(w, p)
        ref = O.linear(O.widen_bf16(X), O.widen_bf16(W0), w.row_adapter, ad, w.max_adapters, rows=sel,
                       base_batched=True)
        for v in variants:
            say(f"apply {w.name} proj={p} variant={v}")
            Y = dev_to_f64(M.apply(pool, p, Xd, W0d, seg_ws, variant=v))
            errs[(p, v)] = assert_close(Y if sel is None else Y[sel], ref, f"apply {w.name} p{p} {v}")
    return errs


def test_apply_worked_example(M):
    check_apply(M, synth.worked_example())


def test_apply_decode_3(M):
    check_apply(M, synth.decode_3_adapters())


def test_apply_decode_fragmented(M):
    check_apply(M, synth.decode_fragmented())


def test_apply_prefill(M):
    """4096 rows, 4096 -> 11008, ranks 8/16/64, 410 base-only rows: every
    element of Y in both variants against the oracle."""
    check_apply(M, synth.prefill_hetero())


def test_apply_layer_stack(M):
    """100 resident adapters over 64 projections (1600 MiB of pages), 512
    rows; all rows of projections 0, 37 and 63 against the oracle."""
    check_apply(M, synth.layer_stack(), projs=(0, 37, 63))


@pytest.mark.parametrize("case", SMALL + LARGE, ids=lambda c: str(c[0]))
def test_apply_small(M, case):
    check_apply(M, small_workload(*case))


def test_apply_multi_projection_pool(M):
    w = small_workload(21, 264, 200, 50, {0: 5, 1: 12, 3: 2}, n_proj=4)
    check_apply(M, w, projs=(0, 1, 3))


@pytest.mark.parametrize("name", ["decode_3", "decode_frag"])
def test_delta_only(M, name):
    """W0 = 0, so the output is the low-rank term alone and the tolerance
    scales with it: a missing or misrouted delta cannot hide under the base."""
    check_apply(M, synth.NAMED[name](), w0_zero=True)


@pytest.mark.parametrize("n,din,dout", [(40, 520, 264), (300, 520, 4104), (1024, 520, 1000),
                                        # split-K decode form: up to 64 rows, K a multiple of 128 from
                                        # 512 to 16384 (4 slices up to 4096, then one per 1024; slices of
                                        # unequal depth where the 128-wide units do not divide evenly)
                                        (1, 4096, 4096), (17, 2048, 1000), (32, 4096, 136), (48, 2048, 4096),
                                        (64, 4096, 4104), (1, 640, 1000), (13, 2560, 264), (32, 11008, 4096),
                                        (48, 8192, 520), (64, 16384, 1000),
                                        # medium batches on the split-K tiled kernel + finish pass
                                        (130, 512, 1000), (700, 1024, 2000), (256, 4096, 4096)])
def test_gemm_lora_with_synthetic_t(M, n, din, dout):
    """The GEMM-with-expand kernel alone (skinny, split-K decode and K-split
    forms), fed a synthetic per-row T."""
    torch = torch_cuda()
    w = small_workload(61 + n, din, dout, n, {0: 16, 1: 3, 2: 64}, p_none=0.2)
    pool, X, seg, seg_ws = _prepare(M, w)
    Tn = synth.draw_t(w.seed, w.n, w.max_rank, 1)[0]
    W0 = w.w0_bits()
    say(f"gemm_lora synthetic T n={n} dout={dout}")
    # the per-row shrink fills T and the rows' descriptors; T is then
    # replaced by the synthetic values (the descriptors stay)
    work = M.shrink_rows(pool, 0, to_dev_bf16(X), seg_ws)
    M.rows_t(pool, work, w.n).copy_(torch.from_numpy(Tn))
    Y = M.gemm_lora(pool, 0, to_dev_bf16(X), to_dev_bf16(W0), seg_ws, work)
    base = O.widen_bf16(X) @ O.widen_bf16(W0).T
    ad = oracle_adapters(w)
    # T already carries the scale: expand with unit scale
    unit = {a: (1.0, d, u) for a, (s_, d, u) in ad.items()}
    t_rows = {k: Tn[k, : w.ranks[int(a)]].astype(np.float64) for k, a in enumerate(w.row_adapter) if a >= 0}
    ref = O.expand_rows(base, t_rows, w.row_adapter, unit, w.max_adapters)
    assert_close(dev_to_f64(Y), ref, "gemm_lora")


@pytest.mark.parametrize("n,din,dout", [(1, 2048, 1000), (17, 2048, 1000), (33, 4096, 136), (48, 4096, 4104),
                                        (64, 4096, 4096), (65, 4096, 4096),
                                        # wider K: 8 to 16 slices, and depths that leave a ragged 1 KiB block
                                        (13, 640, 264), (1, 8192, 1000), (32, 11008, 4096), (17, 2560, 1000),
                                        (48, 14336, 136), (64, 16384, 4104)])
def test_apply_rows_decode_forms(M, n, din, dout):
    """The per-row variant end to end where the per-row shrink shares the
    split-K GEMM launch (K a multiple of 128 from 512 to 16384, up to 64
    rows; 65 rows takes the separate shrink), mixed ranks up to 64 and
    base-only rows."""
    w = small_workload(71 + n, din, dout, n, {0: 16, 1: 3, 2: 64}, p_none=0.2)
    check_apply(M, w, variants=("rows",))


@pytest.mark.parametrize("din", [8192, 11008])
def test_apply_decode_wide_din(M, din):
    """A down projection's decode step (din 8192 or 11008 -> 4096, 32 rows
    split 20/8/4 over three rank-16 adapters): every variant against the
    oracle; the split and fused variants take the same split-K base GEMM
    without the low-rank term."""
    ids = np.array([0] * 20 + [1] * 8 + [2] * 4, dtype=np.int32)
    w = synth.custom(f"decode_din{din}", 81, din, 4096, ids, {0: 16, 1: 16, 2: 16})
    check_apply(M, w)


def test_launch_timing_marks_every_launch(M):
    """The timing hook names and times each kernel launch of an apply call
    (two for the decode form: GEMM with the shrink, then the finish pass)."""
    torch = torch_cuda()
    w = synth.decode_3_adapters()
    pool = make_pool(M, w)
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    seg = M.build_segments(pool, ids_dev(w.row_adapter))
    work = M.new_work(pool, w.n)
    Y = torch.empty((w.n, w.dout), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    say("launch timing")
    M.timing_arm(8)
    M.build_segments(pool, ids_dev(w.row_adapter), seg)
    M.apply(pool, 0, Xd, W0d, seg, Y=Y, work=work, variant="rows")
    marks = M.timing_read()
    assert [m[0] for m in marks] == ["seg_build", "gemm_decode+shrink_rows", "finish_part"], marks
    assert all(0.0 < ms < 100.0 for _, ms in marks), marks
    # disarmed after the read: further launches are not marked
    M.apply(pool, 0, Xd, W0d, seg, Y=Y, work=work, variant="rows")
    torch.cuda.synchronize()
    assert [m[0] for m in M.timing_read()] == [m[0] for m in marks]
    # a down projection's din (11008 = 86 units of 128) takes the same form
    w2 = synth.custom("timing_din11008", 82, 11008, 1024, np.array([0, 1, -1, 0] * 4, dtype=np.int32),
                      {0: 16, 1: 8})
    pool2 = make_pool(M, w2)
    seg2 = M.build_segments(pool2, ids_dev(w2.row_adapter))
    torch.cuda.synchronize()
    M.timing_arm(8)
    M.apply(pool2, 0, to_dev_bf16(w2.x_bits()), to_dev_bf16(w2.w0_bits()), seg2, variant="rows")
    assert [m[0] for m in M.timing_read()] == ["gemm_decode+shrink_rows", "finish_part"]


@pytest.mark.parametrize("variant", ["split", "fused", "rows"])
def test_base_only_rows_bitwise_and_deterministic(M, variant):
    torch = torch_cuda()
    w = synth.decode_3_adapters()
    ids = w.row_adapter.copy()
    ids[::5] = -1
    w = synth.custom("mixed", w.seed, w.din, w.dout, ids, w.ranks, scales=w.scales, max_adapters=3, max_rank=16,
                     x_std=1.0, w0_std=0.02, down_std=1 / 64, up_std=0.02)
    pool = make_pool(M, w)
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    say(f"bitwise {variant}")
    seg = M.build_segments(pool, ids_dev(ids))
    Y1 = M.apply(pool, 0, Xd, W0d, seg, variant=variant)
    Y2 = M.apply(pool, 0, Xd, W0d, seg, variant=variant)
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16)), "two runs differ"
    none = M.build_segments(pool, ids_dev(np.full_like(ids, -1)))
    Yb = M.apply(pool, 0, Xd, W0d, none, variant=variant)
    rows = torch.from_numpy(np.nonzero(ids < 0)[0]).cuda()
    assert torch.equal(Y1[rows].view(torch.int16), Yb[rows].view(torch.int16))
    # and the all-none run is the base GEMM (the layer sums K in split
    # partials through its work buffer, the plain entry point in one pass:
    # the same products in another order, so within rounding)
    assert_close(dev_to_f64(Yb), dev_to_f64(M.base_gemm(Xd, W0d)), f"{variant} all-none", tol=1e-2)


# ranks padded to 16 sum to 272 (> 256: the epilogue form), 144 (the
# rank-concatenated form, 192 deep with 48 zero columns) and exactly 256
LARGE_RANKS = {"epilogue": {0: 1, 1: 8, 2: 17, 3: 64, 4: 128, 6: 16},
               "concat": {0: 1, 1: 8, 2: 17, 3: 64, 6: 16},
               "concat256": {0: 64, 1: 48, 2: 64, 3: 64, 6: 16}}


@pytest.mark.parametrize("form", list(LARGE_RANKS))
@pytest.mark.parametrize("n,dout", [(2100, 2200),   # few 256x256 tiles: 128x128 tiles, two per CU
                                    (4090, 4090)])  # 16 x 16 tiles of 256x256
def test_apply_large_batch_epilogue(M, n, dout, form):
    """Batches large enough for the large GEMM take the split variant with
    the low-rank term added inside the GEMM: in its epilogue, or as extra K
    stages over the rank-concatenated operands when the batch's ranks
    (padded to 16) sum to at most 256.  Ragged M and N, ranks 1 to 128,
    base-only rows and invalid ids (NaN), all rows checked, on both tile
    shapes of the large GEMM."""
    w = small_workload(91, 640, dout, n, LARGE_RANKS[form], p_none=0.1)
    ids = w.row_adapter.copy()
    ids[[5, 700, n - 1]] = [5, 99, -3]      # 5 not resident, 99 out of range, -3 invalid
    w = synth.custom("large_epi", w.seed, w.din, w.dout, ids, w.ranks, scales=w.scales, max_adapters=7,
                     max_rank=128)
    check_apply(M, w, variants=("split",))


@pytest.mark.parametrize("n,dout", [(2100, 2200), (4090, 4090)])
def test_apply_large_batch_concat_narrow(M, n, dout):
    """A pool of two adapters of rank at most 32 gives the low-rank
    operands room for 2 x 32 = 64 rank rows only: the rank-concatenated
    operands are then 64 wide, and ranks 16 + 32 fill 48 of them.  Base-only
    rows and invalid ids (NaN), all rows checked, both tile shapes."""
    w = small_workload(94, 512, dout, n, {0: 16, 1: 32}, p_none=0.1)
    ids = w.row_adapter.copy()
    ids[[3, n // 2]] = [2, -5]  # out of range, invalid
    w = synth.custom("concat_narrow", w.seed, w.din, w.dout, ids, w.ranks, scales=w.scales, max_adapters=2,
                     max_rank=32)
    check_apply(M, w, variants=("split",))


def _apply_launches(M, w, pool):
    """Kernel names of one split-variant apply call."""
    torch = torch_cuda()
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    seg = M.build_segments(pool, ids_dev(w.row_adapter))
    torch.cuda.synchronize()
    M.timing_arm(16)
    M.apply(pool, 0, Xd, W0d, seg, variant="split")
    return [m[0] for m in M.timing_read()]


def test_apply_large_batch_many_adapters(M):
    """A large batch spread over 300 adapters: more segments than the
    operand preparation has threads per block (256), all within the
    epilogue's operand budget, so the GEMM epilogue adds every row's term."""
    ranks = {i: (8 if i % 3 else 16) for i in range(300)}
    ids = synth.random_ids(92, 2048, list(range(300)), 0.05)
    ids[[3, 999]] = [300, -3]  # an id of the table that is not resident, and an invalid one
    w = synth.custom("large_300ad", 92, 512, 4096, ids, ranks, max_adapters=301)
    pool = make_pool(M, w)
    say("many adapters: launches")
    names = _apply_launches(M, w, pool)
    assert "gemm_big_lora" in names and "expand" not in names and "expand_over" not in names, names
    check_apply(M, w, variants=("split",), pool=pool)


def test_apply_large_batch_epilogue_overrun(M):
    """200 rank-64 adapters at dout 11008: one batch touching all of them
    needs 200 * 64 = 12800 rank rows of packed Up (22016 bytes each), more
    than the 256 MiB operand budget holds (12176), so the GEMM leaves the
    low-rank term out and the expand that follows adds it; a batch of the
    same pool over 40 of them fits, the epilogue adds the term and that
    expand does nothing.  Every row against the oracle in both."""
    ranks = {i: 64 for i in range(200)}
    ids = (np.arange(1024) % 200).astype(np.int32)
    ids[[7, 500]] = [-1, -3]  # a base-only row and an invalid id
    w = synth.custom("overrun_200ad", 93, 512, 11008, ids, ranks)
    pool = make_pool(M, w)
    say("overrun: launches")
    names = _apply_launches(M, w, pool)
    assert names[-2:] == ["gemm_big_lora", "expand_over"], names
    check_apply(M, w, variants=("split",), pool=pool)
    ids40 = (np.arange(1024) % 40).astype(np.int32)
    w40 = synth.custom("overrun_200ad", 93, 512, 11008, ids40, ranks)
    say("overrun pool, 40 adapters in the batch")
    check_apply(M, w40, variants=("split",), pool=pool)


def test_invalid_ids_give_nan_rows(M):
    w = small_workload(31, 136, 72, 40, {0: 4, 2: 8}, p_none=0.1)
    ids = w.row_adapter.copy()
    ids[[3, 7, 11]] = [1, 99, -2]           # 1 not resident, 99 and -2 out of range
    w = synth.custom("bad", w.seed, w.din, w.dout, ids, w.ranks, scales=w.scales, max_adapters=3, max_rank=8)
    pool = make_pool(M, w)
    seg_ws = M.build_segments(pool, ids_dev(ids))
    h = M.segments_header(seg_ws)
    assert h["status"] == O.STATUS_BAD_ID | O.STATUS_NOT_RESIDENT and h["n_bad"] == 3
    assert M.segments_status(seg_ws) == h["status"]
    check_apply(M, w, pool=pool)
    # a batch of resident and base-only rows reports no problem
    ok = ids.copy()
    ok[[3, 7, 11]] = [0, -1, 2]
    assert M.segments_status(M.build_segments(pool, ids_dev(ok))) == 0


def test_zero_rows_is_a_noop(M):
    torch = torch_cuda()
    w = small_workload(41, 64, 64, 5, {0: 2})
    pool = make_pool(M, w)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    seg = M.build_segments(pool, torch.empty(0, dtype=torch.int32, device="cuda"))
    Y = M.apply(pool, 0, X, to_dev_bf16(w.w0_bits()), seg)
    assert Y.shape == (0, 64)
    # the one-call form: the workspace header of an empty batch, no layer work
    Y, seg = M.forward(pool, 0, X, to_dev_bf16(w.w0_bits()), torch.empty(0, dtype=torch.int32, device="cuda"))
    h = M.segments_header(seg)
    assert Y.shape == (0, 64) and h["n_rows"] == 0 and h["nseg"] == 0 and h["n_act"] == 0


def test_one_row(M):
    check_apply(M, synth.custom("one", 51, 4096, 4096, [0], {0: 16}, max_rank=16))
    check_apply(M, synth.custom("one_none", 52, 4096, 4096, [-1], {0: 16}, max_rank=16))


def test_apply_max_rows(M):
    """A batch at the row limit (MLORA_MAX_ROWS = 16384) through both grouped
    variants: the segment builder's largest form, tile and item lists of
    every length, the large-batch GEMM with the low-rank epilogue (split)
    and the fused branch; mixed ranks, base-only rows; every row checked."""
    n = 16384
    w = small_workload(97, 136, 264, n, {0: 1, 1: 8, 2: 17, 3: 64, 4: 16}, p_none=0.1)
    assert w.n == n
    check_apply(M, w)
