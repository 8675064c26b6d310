"""The seeded input generators: determinism, structure and distributions."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1.0, 300.0)])
    # values exactly halfway between two bf16 numbers exercise the ties-to-even rule
    halves = ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    a = np.concatenate([a, halves, -halves])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.round_to_bf16_bits(a), want)


@pytest.mark.parametrize("name", synth.ORDER)
def test_workloads_are_deterministic(name):
    w1, w2 = synth.NAMED[name](), synth.NAMED[name]()
    assert np.array_equal(w1.row_adapter, w2.row_adapter)
    a = w1.adapter_ids()[-1]
    if w1.din * w1.dout <= 4096 * 4096:
        assert np.array_equal(w1.w0_bits(0), w2.w0_bits(0))
    assert np.array_equal(w1.down_bits(a, 0), w2.down_bits(a, 0))
    assert np.array_equal(w1.up_bits(a, w1.n_proj - 1), w2.up_bits(a, w1.n_proj - 1))
    # different tensors come from different streams
    assert not np.array_equal(w1.down_bits(a, 0)[:1, :8], w1.up_bits(a, 0).T[:1, :8])


def test_decode_3_split():
    w = synth.decode_3_adapters()
    assert np.bincount(w.row_adapter).tolist() == [20, 8, 4]
    assert w.row_adapter.tolist() != sorted(w.row_adapter.tolist())


def test_decode_down_is_the_decode_split_on_the_down_projection():
    w = synth.decode_down_projection()
    assert (w.din, w.dout, w.n) == (11008, 4096, 32)
    assert np.bincount(w.row_adapter).tolist() == [20, 8, 4]
    assert w.down_std == pytest.approx(1.0 / np.sqrt(11008.0))


def test_decode_frag_is_a_permutation():
    w = synth.decode_fragmented()
    assert sorted(w.row_adapter.tolist()) == list(range(256))


def test_prefill_structure():
    w = synth.prefill_hetero()
    L = w.extra["lengths"]
    assert len(L) == 8 and sum(L) == 4096 and all(64 <= v <= 1024 for v in L)
    assert (w.row_adapter == -1).sum() == 410
    assert sorted(set(w.extra["request_adapter"][:6])) == list(range(6))
    assert sorted(set(w.row_adapter.tolist()) - {-1}) == list(range(6))
    assert [w.ranks[a] for a in range(6)] == [8, 8, 16, 16, 64, 64]
    # round-robin interleave: the first 8 rows come from 8 different requests
    assert w.dout == 11008


def test_layer_stack_structure():
    w = synth.layer_stack()
    ids = w.row_adapter
    assert ids.shape == (512,) and (ids == -1).sum() == 26 and w.n_proj == 64
    assert 30 <= len(set(ids.tolist()) - {-1}) <= 60
    # Zipf: id 0 is the most common
    counts = np.bincount(ids[ids >= 0], minlength=100)
    assert counts[0] == counts.max()


def test_value_distributions():
    w = synth.decode_3_adapters()
    x = w.x_f32()
    assert abs(x.std() - 1.0) < 0.01
    assert abs(w.w0_f32().std() - 0.02) < 1e-4
    assert abs(w.down_f32(0).std() - 1 / 64) < 5e-4
    assert abs(w.up_f32(1).std() - 0.02) < 5e-4


def test_request_rows_follow_the_workload_recipes():
    """Requests of the prefill batch: the recipe's lengths, each request's
    rows on its adapter or base-only, round-robin interleaving; the layer
    stack: 4 contiguous prefill requests of 96 rows, then one decode token
    each; decode batches: one token per request."""
    w = synth.prefill_hetero()
    rr = synth.request_rows(w)
    assert [len(r) for r in rr] == w.extra["lengths"]
    for r, rows in enumerate(rr):
        a = w.extra["request_adapter"][r]
        assert set(w.row_adapter[rows].tolist()) <= {a, -1}
    assert [int(np.flatnonzero([k in rows for rows in rr])[0]) for k in range(8)] == list(range(8))
    ls = synth.layer_stack()
    rr = synth.request_rows(ls)
    assert len(rr) == 132 and [len(r) for r in rr[:5]] == [96, 96, 96, 96, 1]
    assert rr[0].tolist() == list(range(96)) and rr[4].tolist() == [384]
    assert all(len(r) == 1 for r in synth.request_rows(synth.decode_fragmented()))
    assert sorted(np.concatenate(rr).tolist()) == list(range(ls.n))
