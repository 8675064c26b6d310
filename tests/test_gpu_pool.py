"""The paged adapter pool on the GPU: load/unload lifecycle, error codes,
page accounting and reuse of freed (possibly scattered) pages."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import (assert_close, dev_to_f64, ids_dev, oracle_adapters, say, to_dev_bf16, torch_cuda)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


def _w(ranks, n=60, seed=61, din=136, dout=200, n_proj=2, max_adapters=8, max_rank=16):
    ids = synth.random_ids(seed, n, sorted(ranks), 0.1)
    return synth.custom("pool", seed, din, dout, ids, ranks, n_proj=n_proj, max_adapters=max_adapters,
                        max_rank=max_rank)


def _apply_matches(M, pool, w, resident):
    ids = w.row_adapter
    X = w.x_bits()
    seg_ws = M.build_segments(pool, ids_dev(ids))
    for p in range(w.n_proj):
        W0 = w.w0_bits(p)
        ref = O.linear(O.widen_bf16(X), O.widen_bf16(W0), ids, oracle_adapters(w, p, resident), w.max_adapters)
        for v in ("split", "fused"):
            Y = M.apply(pool, p, to_dev_bf16(X), to_dev_bf16(W0), seg_ws, variant=v)
            assert_close(dev_to_f64(Y), ref, f"pool apply p{p} {v}")


def test_error_codes(M):
    w = _w({0: 4, 1: 8})
    pool = M.Pool(w.din, w.dout, w.n_proj, w.max_adapters, w.max_rank, 30)
    d, u = w.down_all_bits(0), w.up_all_bits(0)
    say("pool errors")
    pool.load(0, 4, 2.0, d, u)
    assert pool.query(0) == (4, 2.0)
    with pytest.raises(M.MloraError) as e:
        pool.load(0, 4, 2.0, d, u)
    assert e.value.status == M.EEXIST
    with pytest.raises(M.MloraError) as e:
        pool.unload(3)
    assert e.value.status == M.ENOENT
    for bad_id in (-1, w.max_adapters):
        with pytest.raises(M.MloraError) as e:
            pool.load(bad_id, 4, 2.0, d, u)
        assert e.value.status == M.EINVAL
    big = np.zeros((w.n_proj, 17, w.din), np.uint16)
    with pytest.raises(M.MloraError) as e:
        pool.load(2, 17, 1.0, big, np.zeros((w.n_proj, w.dout, 17), np.uint16))
    assert e.value.status == M.EINVAL
    # 30 pages per arena, 8 used: a rank-16 adapter over 2 projections needs 32
    before = pool.free_pages()
    assert before == (30 - 8, 30 - 8, 1)
    with pytest.raises(M.MloraError) as e:
        pool.load(1, 16, 1.0, np.zeros((2, 16, w.din), np.uint16), np.zeros((2, w.dout, 16), np.uint16))
    assert e.value.status == M.ENOSPC
    assert pool.free_pages() == before
    assert pool.query(1) is None
    # bad projection index
    seg = M.build_segments(pool, ids_dev(np.zeros(4, np.int32)))
    X = to_dev_bf16(np.zeros((4, w.din), np.uint16))
    with pytest.raises(M.MloraError) as e:
        M.apply(pool, w.n_proj, X, to_dev_bf16(w.w0_bits(0)), seg)
    assert e.value.status == M.EINVAL
    pool.unload(0)
    assert pool.free_pages() == (30, 30, 0)
    assert pool.query(0) is None


def test_reuse_of_scattered_pages(M):
    """Load, unload in the middle, then load a bigger adapter that has to
    take the freed hole plus the tail: results still match the oracle."""
    ranks = {0: 4, 1: 8, 2: 4, 3: 12}
    w = _w(ranks)
    pool = M.Pool(w.din, w.dout, w.n_proj, w.max_adapters, w.max_rank, 2 * (4 + 8 + 4) + 10)
    say("pool scattered reuse")
    for a in (0, 1, 2):
        pool.load(a, ranks[a], w.scales[a], w.down_all_bits(a), w.up_all_bits(a))
    pool.unload(1)                      # 16 free pages in the middle, 10 at the end
    pool.load(3, 12, w.scales[3], w.down_all_bits(3), w.up_all_bits(3))   # needs 24: 16 + 8 of the tail
    assert pool.free_pages() == (2, 2, 3)
    ids = w.row_adapter.copy()
    ids[ids == 1] = 3
    w2 = synth.custom("pool", w.seed, w.din, w.dout, ids, ranks, scales=w.scales, n_proj=w.n_proj,
                      max_adapters=w.max_adapters, max_rank=w.max_rank)
    _apply_matches(M, pool, w2, [0, 2, 3])
    # unloaded adapter id now counts as invalid: its rows become NaN
    ids[:3] = 1
    w3 = synth.custom("pool", w.seed, w.din, w.dout, ids, ranks, scales=w.scales, n_proj=w.n_proj,
                      max_adapters=w.max_adapters, max_rank=w.max_rank)
    _apply_matches(M, pool, w3, [0, 2, 3])


def test_reload_after_unload_uses_new_weights(M):
    """An id unloaded and loaded again with other weights: later applies see
    only the new weights (no stale pages, no silent overwrite of a live id)."""
    ranks = {0: 8}
    w = _w(ranks, n=20, seed=71, n_proj=1, max_adapters=2, max_rank=8)
    pool = M.Pool(w.din, w.dout, 1, 2, 8, 8)
    say("pool reload")
    pool.load(0, 8, 2.0, w.down_all_bits(0), w.up_all_bits(0))
    _apply_matches(M, pool, w, [0])
    pool.unload(0)
    w_new = synth.custom("pool", 72, w.din, w.dout, w.row_adapter, {0: 8}, scales={0: 0.5}, n_proj=1,
                         max_adapters=2, max_rank=8)
    pool.load(0, 8, 0.5, w_new.down_all_bits(0), w_new.up_all_bits(0))
    X, W0 = w.x_bits(), w.w0_bits(0)
    seg = M.build_segments(pool, ids_dev(w.row_adapter))
    Y = dev_to_f64(M.apply(pool, 0, to_dev_bf16(X), to_dev_bf16(W0), seg))
    ad = {0: (0.5, O.widen_bf16(w_new.down_bits(0, 0)), O.widen_bf16(w_new.up_bits(0, 0)))}
    assert_close(Y, O.linear(O.widen_bf16(X), O.widen_bf16(W0), w.row_adapter, ad, 2), "reload")


def test_layer_stack_pool_is_1600_mib_and_full(M):
    """The layer-stack pool: 100 rank-16 adapters over 64 projections of
    4096 x 4096 fill exactly 1600 MiB of pages (0.25 MiB per adapter and
    projection)."""
    torch = torch_cuda()
    pages = 100 * 16 * 64
    pool = M.Pool(4096, 4096, 64, 100, 16, pages)
    nbytes = pool.down_pages.numel() * 2 + pool.up_pages.numel() * 2
    assert nbytes == 1600 * 2 ** 20
    d = np.zeros((64, 16, 4096), np.uint16)
    u = np.zeros((64, 4096, 16), np.uint16)
    say("pool 1600 MiB fill")
    for a in range(100):
        pool.load(a, 16, 2.0, d, u)
    assert pool.free_pages() == (0, 0, 100)
    with pytest.raises(M.MloraError) as e:
        pool.load(0, 16, 2.0, d, u)
    assert e.value.status == M.EEXIST
    torch.cuda.synchronize()


def _spin_cycles(torch, ms):
    """Cycles of torch's spin kernel that take about `ms` milliseconds."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(1_000_000)
    b.record()
    torch.cuda.synchronize()
    return int(ms / max(a.elapsed_time(b), 1e-3) * 1_000_000)


def test_cross_stream_reuse_waits_for_last_reader(M):
    """Evict only after the last reader, across streams: the layer runs on
    stream A behind a ~50 ms spin, adapter 0 is unloaded on A, and a new
    adapter is loaded on stream B into the only free pages (adapter 0's).
    B's copies must wait on the device for A's layer: the layer still sees
    the old weights.  Then A waits for the new adapter (pool.ready) and
    serves a batch with it."""
    torch = torch_cuda()
    ranks = {0: 16, 1: 16, 2: 16}
    w = _w(ranks, n=24, seed=81, din=512, dout=520, n_proj=1, max_adapters=4, max_rank=16)
    ids_a = np.where(w.row_adapter == 2, 0, w.row_adapter).astype(np.int32)  # batch on adapters 0 and 1
    ids_b = np.where(ids_a == 0, 2, ids_a).astype(np.int32)                 # adapter 0's rows on adapter 2
    pool = M.Pool(w.din, w.dout, 1, 4, 16, 32)  # room for two rank-16 adapters
    for a in (0, 1):
        pool.load(a, 16, w.scales[a], w.down_all_bits(a), w.up_all_bits(a))
    X, W0 = w.x_bits(), w.w0_bits(0)
    Xd, W0d = to_dev_bf16(X), to_dev_bf16(W0)
    seg_a = M.build_segments(pool, ids_dev(ids_a))
    spin = _spin_cycles(torch, 50.0)
    torch.cuda.synchronize()
    say("pool cross-stream reuse")
    s_b = torch.cuda.Stream()
    torch.cuda._sleep(spin)                       # stream A: the layer starts ~50 ms from now
    Y_a = M.apply(pool, 0, Xd, W0d, seg_a, variant="split")
    pool.unload(0)                                # parked behind the layer
    assert pool.free_pages()[0] == 16
    with torch.cuda.stream(s_b):
        pool.load(2, 16, w.scales[2], w.down_all_bits(2), w.up_all_bits(2))   # reuses adapter 0's pages
    assert pool.free_pages()[0] == 0
    torch.cuda.synchronize()
    ref_a = O.linear(O.widen_bf16(X), O.widen_bf16(W0), ids_a, oracle_adapters(w, 0, [0, 1]), w.max_adapters)
    assert_close(dev_to_f64(Y_a), ref_a, "layer read its adapter after the unload, before the reload on B")

    # a load on B, used on A after A waits for it
    with torch.cuda.stream(s_b):
        pool.unload(2)
        pool.load(2, 16, w.scales[2], w.down_all_bits(2), w.up_all_bits(2))
    pool.ready(2)
    seg_b = M.build_segments(pool, ids_dev(ids_b))
    Y_b = M.apply(pool, 0, Xd, W0d, seg_b, variant="split")
    torch.cuda.synchronize()
    ref_b = O.linear(O.widen_bf16(X), O.widen_bf16(W0), ids_b, oracle_adapters(w, 0, [1, 2]), w.max_adapters)
    assert_close(dev_to_f64(Y_b), ref_b, "layer on the adapter loaded on another stream")
    with pytest.raises(M.MloraError):
        pool.ready(0)                             # not resident


@pytest.mark.parametrize("step", [1, 2])
def test_failed_load_leaves_no_resident_adapter_and_parks_its_pages(M, step):
    """A load that fails once its copies may have been issued (an injected
    failure before its last staging flush, or after its metadata copies)
    leaves the id not resident on the host AND on the device (rank 0 in the
    device table, so an apply treats its rows as invalid, not as reading
    pages a later load overwrites), and its pages come back for the next
    load; the retried load then serves the oracle's result."""
    torch = torch_cuda()
    w = _w({0: 4, 1: 8}, seed=67)
    pool = M.Pool(w.din, w.dout, w.n_proj, w.max_adapters, w.max_rank, 40)
    say(f"pool failed load step {step}")
    pool.load(0, 4, float(w.scales[0]), w.down_all_bits(0), w.up_all_bits(0))
    before = pool.free_pages()
    pool.fail_next_load(step)
    with pytest.raises(M.MloraError) as e:
        pool.load(1, 8, float(w.scales[1]), w.down_all_bits(1), w.up_all_bits(1))
    assert e.value.status == M.EHIP
    assert pool.query(1) is None
    torch.cuda.synchronize()
    dev_rank = pool.meta[: 4 * w.max_adapters].view(torch.int32).cpu().tolist()
    assert dev_rank[1] == 0 and dev_rank[0] == 4
    assert pool.free_pages() == before          # the failed load's pages are free again (parked)
    # rows on the id that failed to load are invalid: NaN, status bit set
    seg_ws = M.build_segments(pool, ids_dev(w.row_adapter))
    assert M.segments_header(seg_ws)["status"] & M.SEG_NOT_RESIDENT
    # the retry takes the parked pages and serves the oracle's result
    pool.load(1, 8, float(w.scales[1]), w.down_all_bits(1), w.up_all_bits(1))
    assert pool.free_pages() == (before[0] - 8 * w.n_proj, before[1] - 8 * w.n_proj, before[2] + 1)
    _apply_matches(M, pool, w, [0, 1])
