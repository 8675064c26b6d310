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


# ---------------------------------------------------------------- bf16 widening

def _bf16_by_definition(bits):
    """Value of a bf16 pattern from the binary format's definition: sign bit,
    8 exponent bits (bias 127), 7 fraction bits; exponent 0 is subnormal
    (no implicit 1, exponent -126), 255 is inf (fraction 0) or NaN."""
    s = -1.0 if bits >> 15 else 1.0
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        return s * float("inf") if f == 0 else float("nan")
    if e == 0:
        return s * float(Fraction(f, 128) * Fraction(2) ** -126)
    return s * float((1 + Fraction(f, 128)) * Fraction(2) ** (e - 127))


def test_widen_bf16_fixed_patterns():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3F81: 1.0 + 2.0 ** -7,
             0x0001: 2.0 ** -133, 0x8001: -(2.0 ** -133), 0x007F: 127 * 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
             0x7F80: float("inf"), 0xFF80: float("-inf"), 0x4049: 3.140625}
    got = O.widen_bf16(np.array(list(cases), dtype=np.uint16))
    assert got.tolist() == list(cases.values())
    z = O.widen_bf16(np.array([0x8000], dtype=np.uint16))[0]
    assert z == 0.0 and np.signbit(z)
    assert np.isnan(O.widen_bf16(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))).all()


def test_widen_bf16_every_pattern_against_definition_and_torch():
    """All 65536 patterns: the exact value from the format's definition, and
    torch's own bfloat16 -> float64 conversion (a library routine), agree with
    the oracle's widening (NaN where they give NaN, sign of zero included)."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.widen_bf16(bits)
    ref = np.array([_bf16_by_definition(int(b)) for b in bits.tolist()])
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for want in (ref, lib):
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # float32 widening is the same exact value (every bf16 is a float32)
    got32 = O.widen_bf16(bits, dtype=np.float32)
    assert got32.dtype == np.float32
    assert np.array_equal(got32[~np.isnan(ref)].astype(np.float64), ref[~np.isnan(ref)])


def test_widen_bf16_inverts_the_input_rounding():
    """Widening the generator's RNE-rounded bits gives the float32 value
    nearest the sample, ties to even: |x - widen(b)| <= half a bf16 ulp."""
    g = np.random.default_rng(17)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-30, 30, 20000))).astype(np.float32)
    b = synth.round_to_bf16_bits(x)
    w = O.widen_bf16(b)
    ulp = np.ldexp(1.0, np.frexp(np.abs(x).astype(np.float64))[1] - 8)
    assert np.all(np.abs(x.astype(np.float64) - w) <= ulp / 2)


# ---------------------------------------------------------------- base FLOP count

def _count_matvec_ops(n, din, dout):
    """Multiplies and adds of the plain row-by-row product y_k = W0 x_k,
    counted by walking it: each output is a sum of din products, and the
    count follows the pages' convention of a multiply plus an add per weight
    (accumulation into zero)."""
    ops = 0
    for _k in range(n):
        for _c in range(dout):
            for _i in range(din):
                ops += 2      # acc = acc + w * x
    return ops


@pytest.mark.parametrize("n,din,dout", [(1, 1, 1), (4, 4, 4), (3, 5, 7), (6, 2, 9), (0, 3, 3)])
def test_base_flops_brute_force(n, din, dout):
    assert O.base_flops(n, din, dout) == _count_matvec_ops(n, din, dout)


def test_base_and_branch_flops_share_the_pages_convention():
    """On the worked example (din = dout = 4), the page counts 2*r*(din+dout)
    per active row for the branch; the same convention applied to a rank-r
    product through a dense din x dout matrix with r = din = dout is the base
    count of one row, and a merged rank-din adapter costs exactly one base
    product per row in each factor."""
    g = _load("worked_example.json")
    din, dout = g["din"], g["dout"]
    assert O.base_flops(1, din, dout) == 2 * din * dout
    assert O.branch_flops([din], din, dout) == O.base_flops(1, din, din) + O.base_flops(1, din, dout)
    assert O.base_flops(len(g["row_adapter"]), din, dout) == 4 * O.base_flops(1, din, dout)


# ---------------------------------------------------------------- mutation check

def _mutants():
    """Plausible slips planted in the oracle (a dropped term, a wrong sign,
    order or index, a transposed factor).  Each replaces one oracle function
    for the duration of one check; every one must make at least one pin
    above fail."""
    lin, seg, shr, exp_, mrg = O.linear, O.segments, O.shrink_rows, O.expand_rows, O.merge
    wid, bfl, brf, adb = O.widen_bf16, O.base_flops, O.branch_flops, O.adapter_bytes

    def unscaled(ad):
        return {a: (1.0, d, u) for a, (s, d, u) in ad.items()}

    def negated(ad):
        return {a: (-s, d, u) for a, (s, d, u) in ad.items()}

    def seg_reverse_ties(ids, max_adapters, resident):
        out = seg(ids, max_adapters, resident)
        perm = out["perm"].copy()
        off = out["seg_off"]
        for s in range(out["nseg"]):
            perm[off[s]:off[s + 1]] = perm[off[s]:off[s + 1]][::-1].copy()
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm), dtype=perm.dtype)
        return dict(out, perm=perm, inv=inv)

    def seg_inv_is_perm(ids, max_adapters, resident):
        out = seg(ids, max_adapters, resident)
        return dict(out, inv=out["perm"].copy())

    def seg_none_first(ids, max_adapters, resident):
        out = seg(ids, max_adapters, resident)
        n_act, n_none = out["n_act"], out["n_none"]
        p = out["perm"]
        perm = np.concatenate([p[n_act:n_act + n_none], p[:n_act], p[n_act + n_none:]])
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm), dtype=perm.dtype)
        return dict(out, perm=perm, inv=inv)

    def seg_descending(ids, max_adapters, resident):
        # groups in descending adapter order
        out = seg(ids, max_adapters, resident)
        blocks = [out["perm"][out["seg_off"][s]:out["seg_off"][s + 1]] for s in range(out["nseg"])][::-1]
        rest = out["perm"][out["n_act"]:]
        perm = np.concatenate(blocks + [rest]).astype(np.int32) if blocks else out["perm"]
        sa = out["seg_adapter"][::-1].copy()
        off = np.concatenate([[0], np.cumsum([len(b) for b in blocks])]).astype(np.int32)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm), dtype=perm.dtype)
        return dict(out, perm=perm, inv=inv, seg_adapter=sa, seg_off=off)

    def shrink_next_row(X, ids, ad, m, rows=None, dtype=np.float64):
        t = shr(X, ids, ad, m, rows, dtype)
        n = np.asarray(X).shape[0]
        return {k: (np.asarray(ad[int(ids[k])][1], dtype) @ np.asarray(X, dtype)[(k + 1) % n]) for k in t}

    return {
        "linear: scale dropped": ("linear", lambda X, W, i, ad, m, **kw: lin(X, W, i, unscaled(ad), m, **kw)),
        "linear: delta subtracted": ("linear", lambda X, W, i, ad, m, **kw: lin(X, W, i, negated(ad), m, **kw)),
        "linear: Up and Down swapped": ("linear", lambda X, W, i, ad, m, **kw: lin(
            X, W, i, {a: (s, u.T, d.T) for a, (s, d, u) in ad.items()}, m, **kw)),
        "linear: invalid ids treated as none": ("linear", lambda X, W, i, ad, m, **kw: lin(
            X, W, [a if (a == -1 or a in ad) else -1 for a in np.asarray(i).tolist()], ad, m, **kw)),
        "segments: ties in reverse row order": ("segments", seg_reverse_ties),
        "segments: inverse taken as perm": ("segments", seg_inv_is_perm),
        "segments: base-only rows first": ("segments", seg_none_first),
        "segments: groups in descending id order": ("segments", seg_descending),
        "shrink_rows: next row's x": ("shrink_rows", shrink_next_row),
        "expand_rows: scale dropped": ("expand_rows", lambda Y, t, i, ad, m, dtype=np.float64: exp_(
            Y, t, i, unscaled(ad), m, dtype)),
        "merge: sign ignored": ("merge", lambda W, a, sign=1.0, dtype=np.float64: mrg(W, a, 1.0, dtype)),
        "merge: factors transposed": ("merge", lambda W, a, sign=1.0, dtype=np.float64: np.asarray(W, dtype) +
                                      sign * a[0] * (np.asarray(a[1], dtype).T @ np.asarray(a[2], dtype).T)
                                      if np.asarray(a[1]).shape[1] == np.asarray(a[2]).shape[0]
                                      else mrg(W, a, sign, dtype)),
        "widen_bf16: fraction one bit short": ("widen_bf16", lambda b, dtype=np.float64: (
            (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) & np.uint32(0xFFFE)) << np.uint32(16)
        ).view(np.float32).astype(dtype)),
        "widen_bf16: read as float16": ("widen_bf16", lambda b, dtype=np.float64: np.ascontiguousarray(
            b, dtype=np.uint16).view(np.float16).astype(dtype)),
        "base_flops: multiply only": ("base_flops", lambda n, din, dout: bfl(n, din, dout) // 2),
        "branch_flops: Down only": ("branch_flops", lambda r, din, dout: brf(r, din, 0)),
        "adapter_bytes: one factor": ("adapter_bytes", lambda din, dout, rank, b=2: adb(din, 0, rank, b)),
    }


def _pin_calls():
    return [
        test_worked_example_segments_match_page, test_worked_example_flops_match_page,
        lambda: test_worked_example_values_route_to_the_right_rows(True),
        lambda: test_worked_example_values_route_to_the_right_rows(False),
        test_pool_sizes_match_page,
        lambda: test_merge_identity(11, 16, 16, {0: 1, 1: 4, 2: 8}),
        lambda: test_merge_serves_its_adapter(31, 16, 24, 3),
        *[lambda s=s: test_merge_exact_rational(s) for s in range(4)],
        test_all_rows_one_adapter_is_one_matmul, test_all_rows_base_only_is_plain_gemm,
        *[lambda s=s: test_exact_rational_brute_force(s) for s in range(6)],
        test_segments_exhaustive_five_rows, test_segments_invalid_ids_sort_last_and_flag,
        test_row_permutation_equivariance, test_zero_padded_rank_changes_nothing, test_linearity_in_scale,
        test_invalid_rows_are_nan_and_others_unaffected, test_widen_bf16_fixed_patterns,
        lambda: test_base_flops_brute_force(3, 5, 7), test_base_and_branch_flops_share_the_pages_convention,
    ]


@pytest.mark.parametrize("mutant", sorted(_mutants()))
def test_every_planted_oracle_slip_fails_a_pin(mutant, monkeypatch):
    name, fn = _mutants()[mutant]
    monkeypatch.setattr(O, name, fn)
    caught = []
    for i, pin in enumerate(_pin_calls()):
        try:
            pin()
        except (AssertionError, ValueError):   # a failed check, or a shape mismatch numpy refuses
            caught.append(i)
    assert caught, f"no pin catches the planted slip '{mutant}'"
