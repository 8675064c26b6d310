"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test ties an oracle function to a value the pages print, a closed form,
an exact rational brute force, an exhaustive search or an invariant, so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed factor, a wrong group order or write-back row) fails at least one.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _adapters_f64(w, proj=0, rounded=True):
    out = {}
    for a in w.adapter_ids():
        if rounded:
            d = O.widen_bf16(w.down_bits(a, proj))
            u = O.widen_bf16(w.up_bits(a, proj))
        else:
            d = w.down_f32(a, proj).astype(np.float64)
            u = w.up_f32(a, proj).astype(np.float64)
        out[a] = (float(w.scales[a]), d, u)
    return out


# ---------------------------------------------------------------- worked example

def test_worked_example_segments_match_page():
    g = _load("worked_example.json")
    seg = O.segments(g["row_adapter"], max_adapters=2, resident=[0, 1])
    assert seg["perm"].tolist() == g["perm"]
    assert seg["perm"][: g["n_act"]].tolist() == g["group_order_rows"]
    assert seg["seg_adapter"].tolist() == g["seg_adapter"]
    assert seg["seg_off"].tolist() == g["seg_off"]
    assert seg["n_act"] == g["n_act"] and seg["n_none"] == 1 and seg["n_bad"] == 0
    assert seg["status"] == 0
    # write-back rows: the rows of each segment, in original order
    for s, a in enumerate(seg["seg_adapter"].tolist()):
        rows = seg["perm"][seg["seg_off"][s]: seg["seg_off"][s + 1]].tolist()
        assert rows == g["writeback_rows"][str(a)]
    assert seg["perm"][seg["n_act"]:].tolist() == g["base_only_rows"]
    # inverse permutation
    assert all(seg["inv"][seg["perm"][j]] == j for j in range(4))


def test_worked_example_flops_match_page():
    g = _load("worked_example.json")
    rank = {int(k): v for k, v in g["rank"].items()}
    ids = g["row_adapter"]
    for a, want in g["flops_group"].items():
        rows = [r for r in ids if r == int(a)]
        assert O.branch_flops([rank[int(a)]] * len(rows), g["din"], g["dout"]) == want
    active = [rank[a] for a in ids if a >= 0]
    assert O.branch_flops(active, g["din"], g["dout"]) == g["flops_effective"]
    assert O.padded_flops(len(ids), max(rank.values()), g["din"], g["dout"]) == g["flops_padded_max_rank"]


@pytest.mark.parametrize("rounded", [False, True])
def test_worked_example_values_route_to_the_right_rows(rounded):
    """On the page's example: rows 0 and 2 equal the A-merged weight applied
    to them, row 1 the B-merged weight, row 3 the base alone; and no row
    matches another adapter's merged weight (the wrong-adapter counterexample
    of the card's section 08)."""
    w = synth.worked_example()
    if rounded:
        X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    else:
        X, W0 = w.x_f32().astype(np.float64), w.w0_f32().astype(np.float64)
    ad = _adapters_f64(w, rounded=rounded)
    Y = O.linear(X, W0, w.row_adapter, ad, w.max_adapters)
    merged = {a: W0 + s * (u @ d) for a, (s, d, u) in ad.items()}
    np.testing.assert_allclose(Y[0], merged[0] @ X[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Y[2], merged[0] @ X[2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Y[1], merged[1] @ X[1], rtol=1e-12, atol=1e-12)
    assert np.array_equal(Y[3], W0 @ X[3])
    assert not O.within_tolerance(Y[1], merged[0] @ X[1])
    assert not O.within_tolerance(Y[0], merged[1] @ X[0])
    assert not O.within_tolerance(Y[0], W0 @ X[0])


def test_pool_sizes_match_page():
    g = _load("pool_sizes.json")
    per_proj = O.adapter_bytes(g["din"], g["dout"], g["rank"], g["bytes_per_param"])
    assert per_proj == g["mib_per_projection"] * 2 ** 20
    per_adapter = per_proj * g["layers"] * g["proj_per_layer"]
    assert per_adapter == g["mib_per_adapter"] * 2 ** 20
    assert per_adapter * g["resident"] == g["mib_resident"] * 2 ** 20


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("seed,din,dout,ranks", [
    (11, 16, 16, {0: 1, 1: 4, 2: 8}),
    (12, 24, 40, {0: 3, 5: 7}),
    (13, 64, 8, {2: 16}),
])
def test_merge_identity(seed, din, dout, ranks):
    """(W0 + s Up Down) x = W0 x + s Up (Down x) for every active row (M031
    card section 04; airsota card section three, derivation 2)."""
    ids = synth.random_ids(seed, 37, sorted(ranks), p_none=0.2)
    w = synth.custom("merge", seed, din, dout, ids, ranks, max_adapters=max(ranks) + 1,
                     scales={a: 0.5 + a for a in ranks})
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    Y = O.linear(X, W0, ids, ad, w.max_adapters)
    for k, a in enumerate(ids):
        if a < 0:
            assert np.array_equal(Y[k], W0 @ X[k])
            continue
        s, d, u = ad[int(a)]
        ref = (W0 + s * (u @ d)) @ X[k]
        np.testing.assert_allclose(Y[k], ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


@pytest.mark.parametrize("seed,din,dout,rank", [(31, 16, 24, 3), (32, 40, 8, 8), (33, 8, 64, 16)])
def test_merge_serves_its_adapter(seed, din, dout, rank):
    """O.merge: the merged weight's plain product equals the layer's output
    for every row of that adapter (M031 card section 04), and differs for a
    row of another adapter; merging with -1 restores W0."""
    ranks = {0: rank, 1: rank + 1}
    ids = np.array([0, 1, 0, -1, 0, 1], dtype=np.int32)
    w = synth.custom("mrg", seed, din, dout, ids, ranks, scales={0: 1.5, 1: 0.75})
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    Y = O.linear(X, W0, ids, ad, w.max_adapters)
    Wm = O.merge(W0, ad[0])
    for k in (0, 2, 4):
        np.testing.assert_allclose(Wm @ X[k], Y[k], rtol=1e-10, atol=1e-12)
    assert not O.within_tolerance(Wm @ X[1], Y[1])
    np.testing.assert_allclose(O.merge(Wm, ad[0], sign=-1.0), W0, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(O.merge(W0, (0.0, ad[0][1], ad[0][2])), W0)  # scale 0: no change


@pytest.mark.parametrize("seed", range(4))
def test_merge_exact_rational(seed):
    """O.merge against an exact rational evaluation on tiny integer factors."""
    g = np.random.default_rng(700 + seed)
    din, dout, r = int(g.integers(1, 7)), int(g.integers(1, 7)), int(g.integers(1, 5))
    s = float(g.choice([1.0, 2.0, 0.5]))
    sign = float(g.choice([1.0, -1.0]))
    W0 = g.integers(-3, 4, size=(dout, din)).astype(np.float64)
    D = g.integers(-2, 3, size=(r, din)).astype(np.float64)
    U = g.integers(-2, 3, size=(dout, r)).astype(np.float64)
    got = O.merge(W0, (s, D, U), sign=sign)
    want = [[Fraction(int(W0[c][i])) + Fraction(sign) * Fraction(s) *
             sum(Fraction(int(U[c][q])) * int(D[q][i]) for q in range(r)) for i in range(din)] for c in range(dout)]
    assert [[Fraction(v) for v in row] for row in got.tolist()] == want


def test_all_rows_one_adapter_is_one_matmul():
    ranks = {0: 5}
    ids = np.zeros(29, dtype=np.int32)
    w = synth.custom("one", 21, 48, 33, ids, ranks, scales={0: 1.75})
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    s, d, u = ad[0]
    Y = O.linear(X, W0, ids, ad, w.max_adapters)
    np.testing.assert_allclose(Y, X @ (W0 + s * (u @ d)).T, rtol=1e-10, atol=1e-12)
    Yb = O.linear(X, W0, ids, ad, w.max_adapters, base_batched=True)
    np.testing.assert_allclose(Yb, Y, rtol=1e-12, atol=1e-12)


def test_all_rows_base_only_is_plain_gemm():
    ids = np.full(19, -1, dtype=np.int32)
    w = synth.custom("none", 22, 40, 24, ids, {0: 4})
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    Y = O.linear(X, W0, ids, _adapters_f64(w), w.max_adapters)
    np.testing.assert_allclose(Y, X @ W0.T, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- exact brute force

def _frac_eval(X, W0, ids, ad):
    """Exact rational evaluation through the merged weight of each row's
    adapter (a different association order from the oracle's)."""
    n, din = len(X), len(X[0])
    dout = len(W0)
    Y = []
    for k in range(n):
        a = ids[k]
        if a >= 0:
            s, D, U = ad[a]
            r = len(D)
            M = [[W0[c][i] + s * sum(U[c][q] * D[q][i] for q in range(r)) for i in range(din)]
                 for c in range(dout)]
        else:
            M = W0
        Y.append([sum(M[c][i] * X[k][i] for i in range(din)) for c in range(dout)])
    return Y


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_brute_force(seed):
    g = np.random.default_rng(500 + seed)
    din, dout = int(g.integers(1, 9)), int(g.integers(1, 9))
    n = int(g.integers(1, 7))
    n_ad = int(g.integers(1, 4))
    ranks = {a: int(g.integers(1, 5)) for a in range(n_ad)}
    scales = {a: float(g.choice([1.0, 2.0, 0.5])) for a in range(n_ad)}
    ids = [int(v) for v in g.integers(-1, n_ad, size=n)]
    iv = lambda *sh: g.integers(-2, 3, size=sh).astype(np.int64)
    X, W0 = iv(n, din), iv(dout, din)
    D = {a: iv(ranks[a], din) for a in range(n_ad)}
    U = {a: iv(dout, ranks[a]) for a in range(n_ad)}
    ad = {a: (scales[a], D[a].astype(np.float64), U[a].astype(np.float64)) for a in range(n_ad)}
    Y = O.linear(X.astype(np.float64), W0.astype(np.float64), ids, ad, n_ad)
    F = lambda m: [[Fraction(int(v)) for v in row] for row in m]
    adF = {a: (Fraction(scales[a]), F(D[a]), F(U[a])) for a in range(n_ad)}
    ref = _frac_eval(F(X), F(W0), ids, adF)
    assert [[Fraction(v) for v in row] for row in Y.tolist()] == ref
    # the two halves on their own
    t = O.shrink_rows(X.astype(np.float64), ids, ad, n_ad)
    for k, a in enumerate(ids):
        if a >= 0:
            want = [sum(Fraction(int(D[a][q][i])) * int(X[k][i]) for i in range(din))
                    for q in range(ranks[a])]
            assert [Fraction(v) for v in t[k].tolist()] == want
        else:
            assert k not in t
    Yb = O.linear(X.astype(np.float64), W0.astype(np.float64), [-1] * n, ad, n_ad)
    Ye = O.expand_rows(Yb, t, ids, ad, n_ad)
    assert [[Fraction(v) for v in row] for row in Ye.tolist()] == ref


# ---------------------------------------------------------------- segments

def _perm_by_search(keys):
    """The unique permutation whose (key, row) sequence is strictly
    increasing, found by trying every permutation."""
    n = len(keys)
    found = [p for p in itertools.permutations(range(n))
             if all((keys[p[j]], p[j]) < (keys[p[j + 1]], p[j + 1]) for j in range(n - 1))]
    assert len(found) == 1
    return list(found[0])


def test_segments_exhaustive_five_rows():
    """All 4^5 id assignments over {none, 0, 1, 2}: perm, inv, groups and
    offsets against exhaustive search and direct counting."""
    A = 3
    for ids in itertools.product([-1, 0, 1, 2], repeat=5):
        seg = O.segments(ids, A, resident=[0, 1, 2])
        keys = [a if a >= 0 else A for a in ids]
        perm = _perm_by_search(keys)
        assert seg["perm"].tolist() == perm
        assert [seg["inv"][p] for p in perm] == list(range(5))
        present = sorted(set(a for a in ids if a >= 0))
        assert seg["seg_adapter"].tolist() == present
        assert seg["seg_off"].tolist() == [sum(1 for b in ids if 0 <= b < a) for a in present] + \
            [sum(1 for b in ids if b >= 0)]
        assert seg["nseg"] == len(present) and seg["status"] == 0


def test_segments_invalid_ids_sort_last_and_flag():
    ids = [2, -3, 1, -1, 7, 1, 4, 2]          # resident {1, 2, 4}? 4 is not resident; 7 is out of range
    seg = O.segments(ids, max_adapters=5, resident=[1, 2])
    keys = [2, 6, 1, 5, 6, 1, 6, 2]
    assert seg["perm"].tolist() == _perm_by_search(keys)
    assert seg["seg_adapter"].tolist() == [1, 2]
    assert seg["seg_off"].tolist() == [0, 2, 4]
    assert (seg["n_act"], seg["n_none"], seg["n_bad"]) == (4, 1, 3)
    assert seg["status"] == O.STATUS_BAD_ID | O.STATUS_NOT_RESIDENT


def test_segments_of_named_workloads_are_counting_sorts():
    for name in ["decode_3", "decode_frag", "prefill", "layer_stack"]:
        w = synth.NAMED[name]()
        ids = w.row_adapter
        seg = O.segments(ids, w.max_adapters, w.adapter_ids())
        keys = np.where(ids >= 0, ids, w.max_adapters)
        assert np.array_equal(seg["perm"], np.argsort(keys, kind="stable"))
        assert sorted(seg["perm"].tolist()) == list(range(len(ids)))
        counts = np.bincount(ids[ids >= 0], minlength=w.max_adapters)
        assert seg["seg_adapter"].tolist() == np.nonzero(counts)[0].tolist()
        assert np.array_equal(np.diff(seg["seg_off"]), counts[counts > 0])


# ---------------------------------------------------------------- invariants

def test_row_permutation_equivariance():
    ranks = {0: 2, 1: 6, 3: 3}
    ids = synth.random_ids(31, 23, [0, 1, 3], p_none=0.25)
    w = synth.custom("eq", 31, 20, 12, ids, ranks, max_adapters=4)
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    Y = O.linear(X, W0, ids, ad, 4)
    p = np.random.default_rng(3).permutation(len(ids))
    Yp = O.linear(X[p], W0, ids[p], ad, 4)
    assert np.array_equal(Yp, Y[p])


def test_zero_padded_rank_changes_nothing():
    """Padding an adapter to a larger rank with zero Down rows and zero Up
    columns (the rank-padded baseline of the airsota card's trade-off (4) and
    the wiblog article's naive shared batch) leaves every output row as it
    was, in the one-call oracle and in its shrink/expand split; t of a padded
    adapter is the unpadded t followed by zeros."""
    ranks = {0: 3, 1: 7, 2: 1}
    ids = synth.random_ids(47, 19, [0, 1, 2], p_none=0.2)
    w = synth.custom("pad", 47, 24, 20, ids, ranks, max_adapters=3)
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    R = 16
    padded = {a: (s_, np.vstack([d, np.zeros((R - d.shape[0], d.shape[1]))]),
                  np.hstack([u, np.zeros((u.shape[0], R - u.shape[1]))])) for a, (s_, d, u) in ad.items()}
    Y = O.linear(X, W0, ids, ad, 3)
    np.testing.assert_allclose(O.linear(X, W0, ids, padded, 3), Y, rtol=1e-13, atol=1e-15)
    t, tp = O.shrink_rows(X, ids, ad, 3), O.shrink_rows(X, ids, padded, 3)
    assert sorted(t) == sorted(tp)
    for k in t:
        r = ranks[int(ids[k])]
        assert np.array_equal(tp[k][:r], t[k]) and not tp[k][r:].any()
    base = X @ W0.T
    np.testing.assert_allclose(O.expand_rows(base, tp, ids, padded, 3), Y, rtol=1e-13, atol=1e-15)


def test_linearity_in_scale():
    ranks = {0: 4, 1: 2}
    ids = synth.random_ids(41, 17, [0, 1], p_none=0.2)
    w = synth.custom("lin", 41, 16, 24, ids, ranks)
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    base = O.linear(X, W0, [-1] * len(ids), ad, 2)
    zero = {a: (0.0, d, u) for a, (s, d, u) in ad.items()}
    assert np.array_equal(O.linear(X, W0, ids, zero, 2), base)
    up0 = {a: (s, d, np.zeros_like(u)) for a, (s, d, u) in ad.items()}
    assert np.array_equal(O.linear(X, W0, ids, up0, 2), base)
    d1 = O.linear(X, W0, ids, ad, 2) - base
    dbl = {a: (2 * s, d, u) for a, (s, d, u) in ad.items()}
    d2 = O.linear(X, W0, ids, dbl, 2) - base
    np.testing.assert_allclose(d2, 2 * d1, rtol=1e-9, atol=1e-12)


def test_invalid_rows_are_nan_and_others_unaffected():
    ranks = {0: 3, 2: 5}
    ids = np.array([0, 2, 1, -1, 9, -4, 2], dtype=np.int32)   # 1 not resident, 9 and -4 out of range
    w = synth.custom("bad", 51, 12, 10, ids, ranks, max_adapters=4)
    X, W0 = O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits())
    ad = _adapters_f64(w)
    Y = O.linear(X, W0, ids, ad, 4)
    assert np.all(np.isnan(Y[[2, 4, 5]]))
    assert not np.any(np.isnan(Y[[0, 1, 3, 6]]))
    good = O.linear(X, W0, np.where(np.isin(ids, [0, 2, -1]), ids, -1), ad, 4)
    assert np.array_equal(Y[[0, 1, 3, 6]], good[[0, 1, 3, 6]])


# ---------------------------------------------------------------- planted mistakes

def _case(name, n_rows=None):
    w = synth.NAMED[name]()
    X = O.widen_bf16(w.x_bits())
    W0 = O.widen_bf16(w.w0_bits(0))
    ad = _adapters_f64(w)
    rows = list(range(w.n)) if n_rows is None else \
        sorted(np.random.default_rng(9).choice(w.n, size=n_rows, replace=False).tolist())
    return w, X, W0, ad, rows


@pytest.mark.parametrize("name,n_rows", [("worked_example", None), ("decode_3", None),
                                         ("decode_frag", 24), ("prefill", 24)])
def test_planted_mistakes_fail_the_parity_bar(name, n_rows):
    """Misrouting that raises no shape error must still fail the 2e-2 bar:
    swapped adapters, group results written contiguously into the first
    rows, and one shared adapter for every row (M031 card section 03 and
    section 08; wiblog article, naive mixed batch)."""
    w, X, W0, ad, rows = _case(name, n_rows)
    ids = w.row_adapter
    ref = O.linear(X, W0, ids, ad, w.max_adapters, rows=rows, base_batched=True)
    # 1. swap the first two adapters' weights (same id -> other weights)
    a0, a1 = w.adapter_ids()[:2]
    swapped = dict(ad)
    swapped[a0], swapped[a1] = ad[a1], ad[a0]
    bad = O.linear(X, W0, ids, swapped, w.max_adapters, rows=rows, base_batched=True)
    assert not O.within_tolerance(bad, ref)
    # 2. contiguous write-back: the delta of sorted position j lands on row j
    seg = O.segments(ids, w.max_adapters, w.adapter_ids())
    base = O.linear(X, W0, [-1] * w.n, ad, w.max_adapters, rows=rows, base_batched=True)
    src = [int(seg["perm"][k]) for k in rows if k < seg["n_act"]]
    delta = O.linear(X, W0, ids, ad, w.max_adapters, rows=src, base_batched=True) - \
        O.linear(X, W0, [-1] * w.n, ad, w.max_adapters, rows=src, base_batched=True)
    contig = base.copy()
    for i, k in enumerate(rows):
        if k < seg["n_act"]:
            contig[i] += delta[src.index(int(seg["perm"][k]))]
    assert not O.within_tolerance(contig, ref)
    # 3. one shared adapter for every active row
    shared = [a0 if a >= 0 else -1 for a in ids]
    bad = O.linear(X, W0, shared, ad, w.max_adapters, rows=rows, base_batched=True)
    assert not O.within_tolerance(bad, ref)
    # 4. the low-rank term dropped altogether
    assert not O.within_tolerance(base, ref)


def test_tolerance_is_nan_aware():
    a = np.array([1.0, np.nan])
    assert O.within_tolerance(a, a)
    assert not O.within_tolerance(np.array([1.0, 0.0]), a)
    assert not O.within_tolerance(np.array([np.nan, 1.0]), np.array([1.0, 1.0]))
    assert O.within_tolerance(np.array([1.03]), np.array([1.0]))
    assert not O.within_tolerance(np.array([1.05]), np.array([1.0]))
