"""Segment builder on the GPU: bit-exact against the oracle's stable sort."""
import itertools

import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import ids_dev, say, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


_pools = {}


def tiny_pool(M, max_adapters, resident):
    """A din = dout = 8 pool where `resident` ids hold rank-1 adapters (the
    builder only reads which ids are resident)."""
    key = (max_adapters, tuple(resident))
    if key not in _pools:
        pool = M.Pool(8, 8, 1, max_adapters, 1, max(len(resident), 1))
        one = np.zeros((1, 1, 8), dtype=np.uint16)
        for a in resident:
            pool.load(int(a), 1, 1.0, one, one.reshape(1, 8, 1))
        _pools[key] = pool
    return _pools[key]


def check(M, pool, ids, max_adapters, resident, what):
    ids = np.asarray(ids, dtype=np.int32)
    n = len(ids)
    say(f"segments {what} n={n} A={max_adapters}")
    seg_ws = M.build_segments(pool, ids_dev(ids) if n else ids_dev(np.zeros(1, np.int32))[:0])
    got = M.read_segments(seg_ws, n)
    ref = O.segments(ids, max_adapters, resident)
    for k in ("nseg", "n_act", "n_none", "n_bad", "status"):
        assert got[k] == ref[k], (what, k, got[k], ref[k])
    assert got["n_rows"] == n and got["max_adapters"] == max_adapters
    for k in ("perm", "inv", "seg_adapter", "seg_off"):
        assert np.array_equal(got[k], ref[k]), (what, k)
    res = set(int(a) for a in resident)
    want_key = [int(a) if int(a) in res else (-1 if a == -1 else -2) for a in ids]
    assert got["row_key"].tolist() == want_key, what
    # work items: every active sorted position exactly once, inside its own
    # segment, at most ITEM_ROWS rows, in segment order
    cover = np.zeros(ref["n_act"], dtype=np.int64)
    last = -1
    for s, j0 in got["items"]:
        lo, hi = ref["seg_off"][s], ref["seg_off"][s + 1]
        assert lo <= j0 < hi, (what, s, j0)
        assert j0 > last
        last = j0
        cover[j0:min(j0 + M.ITEM_ROWS, hi)] += 1
    assert np.all(cover == 1), what
    # tiles: fixed by the segments, (s, seg_off[s] + t * TILE_ROWS) in order
    want = [(s, int(ref["seg_off"][s]) + t)
            for s in range(ref["nseg"])
            for t in range(0, int(ref["seg_off"][s + 1] - ref["seg_off"][s]), M.TILE_ROWS)]
    assert got["n_tiles"] == len(want), (what, got["n_tiles"], len(want))
    assert [tuple(int(v) for v in t) for t in got["tiles"]] == want, what
    return got


def test_worked_example(M):
    w = synth.worked_example()
    got = check(M, tiny_pool(M, 2, [0, 1]), w.row_adapter, 2, [0, 1], "worked example")
    assert got["perm"].tolist() == [0, 2, 1, 3]


@pytest.mark.parametrize("name", ["decode_3", "decode_frag", "prefill", "layer_stack"])
def test_named_workloads(M, name):
    w = synth.NAMED[name]()
    res = w.adapter_ids()
    check(M, tiny_pool(M, w.max_adapters, res), w.row_adapter, w.max_adapters, res, name)


def test_all_assignments_of_five_rows(M):
    pool = tiny_pool(M, 3, [0, 1, 2])
    for ids in itertools.product([-1, 0, 1, 2], repeat=5):
        check(M, pool, ids, 3, [0, 1, 2], f"ids={ids}")


@pytest.mark.parametrize("n,A,seed", [(0, 4, 1), (1, 4, 2), (63, 7, 3), (64, 254, 4), (65, 255, 5),
                                      (1000, 256, 6), (4097, 300, 7), (16384, 5000, 8), (16384, 3, 9),
                                      (777, 1, 10),
                                      # resident-table edges: read into LDS up to 64 ids (one wave) and up
                                      # to one id per thread within the free buffer, else per row
                                      (40, 64, 11), (40, 65, 12), (200, 256, 13), (200, 257, 14),
                                      (70, 200, 15), (1025, 1024, 16), (1025, 1025, 17)])
def test_random_batches(M, n, A, seed):
    g = np.random.default_rng(seed)
    resident = sorted(g.choice(A, size=max(1, (2 * A) // 3), replace=False).tolist())
    ids = g.integers(-1, A, size=n).astype(np.int32)
    check(M, tiny_pool(M, A, resident), ids, A, resident, f"random seed {seed}")


def test_invalid_ids_sort_last_and_set_status(M):
    g = np.random.default_rng(77)
    A = 40
    resident = list(range(0, 40, 2))
    ids = g.integers(-3, A + 5, size=3000).astype(np.int32)
    got = check(M, tiny_pool(M, A, resident), ids, A, resident, "invalid ids")
    assert got["status"] == O.STATUS_BAD_ID | O.STATUS_NOT_RESIDENT
    assert got["n_bad"] > 0


def test_one_adapter_all_rows_and_all_none(M):
    pool = tiny_pool(M, 4, [0, 1, 2, 3])
    check(M, pool, np.full(5000, 2, np.int32), 4, [0, 1, 2, 3], "all on one adapter")
    check(M, pool, np.full(5000, -1, np.int32), 4, [0, 1, 2, 3], "all base-only")


def test_header_and_determinism(M):
    w = synth.prefill_hetero()
    pool = tiny_pool(M, w.max_adapters, w.adapter_ids())
    ids = ids_dev(w.row_adapter)
    say("segments determinism")
    a = M.read_segments(M.build_segments(pool, ids), w.n)
    b = M.read_segments(M.build_segments(pool, ids), w.n)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    h = M.segments_header(M.build_segments(pool, ids))
    ref = O.segments(w.row_adapter, w.max_adapters, w.adapter_ids())
    assert (h["nseg"], h["n_act"], h["n_none"], h["n_bad"], h["status"]) == \
        (ref["nseg"], ref["n_act"], ref["n_none"], ref["n_bad"], 0)


def test_too_many_rows_is_rejected(M):
    import ctypes
    torch = torch_cuda()
    pool = tiny_pool(M, 2, [0])
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = M.lib().mlora_build_segments(pool.handle, ctypes.c_void_p(buf.data_ptr()), M.MAX_ROWS + 1,
                                      ctypes.c_void_p(buf.data_ptr()), None)
    assert st == M.EINVAL
    assert b"n_rows" in M.lib().mlora_last_error()
