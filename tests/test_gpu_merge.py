"""GPU parity of the merged alternative (mlora_merge) against the CPU oracle.

The merge writes bf16(W0 + sign * s Up Down) in place; the oracle's merge is
the same sum in fp64.  The kernel sums the r products in fp32 (error at most
E = (r + 2) 2^-24 (s sum_q |Up Down| + |W0|) per element) and rounds once to
bf16 (at most one unit in the last place, 2^-7 of the magnitude), so each
element must satisfy |got - ref| <= 2^-7 (|ref| + E) + E.  The merged weight
must then serve its adapter's rows through the plain base GEMM within the
layer's tolerance (M031 card section 04), and an unmerge must restore W0 up
to the two roundings."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import assert_close, dev_to_f64, make_pool, oracle_adapters, say, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu

ULP = 2.0 ** -7   # bf16: 8 significant bits


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


def _sum_error(W0, adapter):
    """Bound on the fp32 error of W0 + s sum_q Up Down summed in rank order."""
    s, d, u = adapter
    return (d.shape[0] + 2) * 2.0 ** -24 * (abs(s) * (np.abs(u) @ np.abs(d)) + np.abs(W0))


def _within(got, ref, E, what, ulps=1.0, mag=None):
    mag = np.abs(ref) if mag is None else mag
    bound = ulps * ULP * (mag + E) + E + 2.0 ** -126
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound, worst {float((err / bound).max()):.2f}x"


MERGE_CASES = [
    # (seed, din, dout, ranks, n_proj, proj)
    (1, 4, 4, {0: 1, 1: 2}, 1, 0),             # the worked example's shape
    (2, 64, 40, {0: 16, 3: 8}, 2, 1),          # second projection of a two-projection pool
    (3, 1000, 520, {0: 7, 1: 33}, 1, 0),       # din not a multiple of 8: element-wise path
    (4, 4096, 512, {0: 16, 1: 64}, 1, 0),      # several column blocks, 16-row tail-free
    (5, 2056, 1000, {0: 128, 2: 1}, 1, 0),     # largest rank; dout not a multiple of 16
    (6, 4096, 4096, {0: 16, 1: 16, 2: 16}, 1, 0),  # the decode workload's shape
    # rank <= 16 on 16-byte rows (Down held in registers over 16 rows): a
    # partial column block (din 2056) and a ragged last row block (dout 1000)
    (7, 2056, 1000, {0: 5, 1: 9}, 2, 1),
    (8, 512, 24, {0: 17}, 1, 0),               # rank 17: the general form on 16-byte rows
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=lambda c: str(c[0]))
def test_merge_matches_oracle(M, case):
    seed, din, dout, ranks, n_proj, proj = case
    torch = torch_cuda()
    ids = np.array([a for a in ranks] * 3 + [-1], dtype=np.int32)
    w = synth.custom(f"merge{seed}", seed, din, dout, ids, ranks, n_proj=n_proj,
                     scales={a: 1.0 + 0.5 * i for i, a in enumerate(ranks)})
    pool = make_pool(M, w)
    ad = oracle_adapters(w, proj=proj)
    W0 = O.widen_bf16(w.w0_bits(proj))
    a = next(iter(ranks))
    Wd = to_dev_bf16(w.w0_bits(proj))
    say(f"merge case={seed} din={din} dout={dout} rank={ranks[a]} proj={proj}")
    M.merge(pool, a, proj, Wd, 1.0)
    torch.cuda.synchronize()
    Wm = dev_to_f64(Wd)
    ref = O.merge(W0, ad[a])
    E = _sum_error(W0, ad[a])
    _within(Wm, ref, E, f"merge case {seed}")

    # the merged weight serves adapter a's rows through the plain GEMM
    rows = np.flatnonzero(ids == a)
    X = O.widen_bf16(w.x_bits())[rows]
    Xd = to_dev_bf16(w.x_bits()[rows])
    Y = torch.empty((len(rows), dout), dtype=torch.bfloat16, device="cuda")
    say(f"merged gemm case={seed}")
    M.base_gemm(Xd, Wd, Y)
    torch.cuda.synchronize()
    want = O.linear(X, W0, ids[rows], ad, w.max_adapters)
    assert_close(dev_to_f64(Y), want, f"merged serving case {seed}")

    # and an unmerge restores W0 up to the two bf16 roundings
    say(f"unmerge case={seed}")
    M.merge(pool, a, proj, Wd, -1.0)
    torch.cuda.synchronize()
    _within(dev_to_f64(Wd), W0, 2 * E, f"unmerge case {seed}", mag=np.abs(W0) + np.abs(ref))


def test_merge_other_adapter_differs(M):
    """Negative control: the weight merged with adapter 0 must fail the
    tolerance for rows of adapter 1."""
    torch = torch_cuda()
    ranks = {0: 16, 1: 16}
    ids = np.array([1] * 8, dtype=np.int32)
    w = synth.custom("mergeneg", 9, 512, 256, ids, ranks)
    pool = make_pool(M, w)
    ad = oracle_adapters(w)
    Wd = to_dev_bf16(w.w0_bits())
    say("merge negative control")
    M.merge(pool, 0, 0, Wd)
    Y = torch.empty((8, 256), dtype=torch.bfloat16, device="cuda")
    M.base_gemm(to_dev_bf16(w.x_bits()), Wd, Y)
    torch.cuda.synchronize()
    want = O.linear(O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits()), ids, ad, w.max_adapters)
    assert not O.within_tolerance(dev_to_f64(Y), want)


def test_merge_errors(M):
    """Host-side argument checks: nothing is launched."""
    ranks = {0: 4}
    w = synth.custom("mergeerr", 10, 64, 32, np.array([0], dtype=np.int32), ranks, max_adapters=3)
    pool = make_pool(M, w)
    Wd = to_dev_bf16(w.w0_bits())
    with pytest.raises(M.MloraError, match="not resident"):
        M.merge(pool, 1, 0, Wd)
    with pytest.raises(M.MloraError, match="outside"):
        M.merge(pool, 3, 0, Wd)
    with pytest.raises(M.MloraError, match="projection"):
        M.merge(pool, 0, 1, Wd)
    with pytest.raises(M.MloraError, match="finite"):
        M.merge(pool, 0, 0, Wd, float("nan"))
