"""GPU parity of the two naive baselines the benchmark times beside the
grouped layer (wiblog article, baseline methods; M031 card section 03):
serving each adapter group through its own launches, and a pool where every
adapter is zero-padded to the largest rank.  Both must give the oracle's
output: grouping and padding change the work, not the result."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import assert_close, dev_to_f64, ids_dev, make_pool, oracle_adapters, say, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


def _workload():
    ranks = {0: 8, 1: 16, 2: 64}
    ids = synth.random_ids(41, 300, sorted(ranks), p_none=0.1)
    return synth.custom("baselines", 41, 1024, 768, ids, ranks)


def test_per_group_launches_match_oracle(M):
    torch = torch_cuda()
    w = _workload()
    pool = make_pool(M, w)
    X = O.widen_bf16(w.x_bits())
    W0 = O.widen_bf16(w.w0_bits())
    ref = O.linear(X, W0, w.row_adapter, oracle_adapters(w), w.max_adapters, base_batched=True)
    Wd = to_dev_bf16(w.w0_bits())
    for a in list(w.adapter_ids()) + [-1]:
        rows = np.flatnonzero(w.row_adapter == a)
        xa = to_dev_bf16(w.x_bits()[rows])
        say(f"per-group launches adapter={a} rows={len(rows)}")
        if a < 0:
            Y = M.base_gemm(xa, Wd)
        else:
            ia = ids_dev(np.full(len(rows), a, dtype=np.int32))
            Y = M.apply(pool, 0, xa, Wd, M.build_segments(pool, ia))
        torch.cuda.synchronize()
        assert_close(dev_to_f64(Y), ref[rows], f"group {a}")


def test_padded_pool_matches_oracle(M):
    torch = torch_cuda()
    w = _workload()
    rmax = max(w.ranks.values())
    pool = M.Pool(w.din, w.dout, 1, w.max_adapters, rmax, len(w.ranks) * rmax)
    for a in w.adapter_ids():
        r = w.ranks[a]
        d = np.zeros((1, rmax, w.din), dtype=np.uint16)
        u = np.zeros((1, w.dout, rmax), dtype=np.uint16)
        d[0, :r] = w.down_bits(a)
        u[0, :, :r] = w.up_bits(a)
        pool.load(a, rmax, w.scales[a], d, u)
    X = O.widen_bf16(w.x_bits())
    ref = O.linear(X, O.widen_bf16(w.w0_bits()), w.row_adapter, oracle_adapters(w), w.max_adapters,
                   base_batched=True)
    Xd, Wd = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    seg = M.build_segments(pool, ids_dev(w.row_adapter))
    for variant in ("split", "rows", "fused"):
        say(f"padded pool variant={variant}")
        Y = M.apply(pool, 0, Xd, Wd, seg, variant=variant)
        torch.cuda.synchronize()
        assert_close(dev_to_f64(Y), ref, f"padded {variant}")


@pytest.mark.parametrize("name,n_rows", [("decode_3", None), ("prefill", 1200)])
def test_per_request_serial_matches_oracle(M, name, n_rows):
    """The per-request serial baseline (wiblog article, baseline methods):
    every request through its own layer call on its own rows.  Each
    request's output equals the oracle's rows of that request.  (The
    prefill case keeps its first requests up to about n_rows rows, so the
    fp64 oracle stays quick.)"""
    torch = torch_cuda()
    w = synth.NAMED[name]()
    reqs = synth.request_rows(w)
    if n_rows is not None:
        keep, total = [], 0
        for rows in reqs:
            if total >= n_rows:
                break
            keep.append(rows)
            total += len(rows)
        reqs = keep
    pool = make_pool(M, w)
    X, W0 = w.x_bits(), w.w0_bits()
    Wd = to_dev_bf16(W0)
    sel = np.concatenate(reqs)
    ref = O.linear(O.widen_bf16(X), O.widen_bf16(W0), w.row_adapter, oracle_adapters(w), w.max_adapters,
                   rows=sel.tolist(), base_batched=True)
    at = {int(k): i for i, k in enumerate(sel)}
    for r, rows in enumerate(reqs):
        say(f"per-request {name} request={r} rows={len(rows)}")
        Y, _ = M.forward(pool, 0, to_dev_bf16(X[rows]), Wd, ids_dev(w.row_adapter[rows]))
        torch.cuda.synchronize()
        assert_close(dev_to_f64(Y), ref[[at[int(k)] for k in rows]], f"request {r}")
