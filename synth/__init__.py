"""Seeded synthetic inputs for the heterogeneous multi-LoRA linear.

This module only *draws* inputs: row->adapter ids, activations X, base weight
W0 and each adapter's Down/Up factors, rank and scale.  It holds none of the
method's arithmetic (no products, no grouping, no accumulation), so both the
CPU oracle's tests and the GPU path's tests and benchmark can take their
inputs from here without sharing any of the computation.

Every tensor is drawn in float32 from its own counter-free PCG64 stream whose
SeedSequence is keyed by (workload seed, tensor tag, indices), so any slice of
a workload (one projection, one adapter) can be regenerated on its own and in
any order.  The GPU path consumes bfloat16, so each draw is rounded to bf16
with round-to-nearest-even on the bit pattern; the uint16 bit patterns are
what both sides receive.

The five named workloads reproduce the shapes, value distributions and id
structure of the multi-LoRA examples on the pages (the M031 card's worked
example in its section 02/03, the Punica fragmentation example of 32 decode
tokens split 20/8/4 on the wiblog vLLM scheduling article, the mixed
r = 8/16/64 ranks named on the airsota card's trade-off item 4, and the
32-layer x 2-projection, 100-adapter pool sizing of the M031 card's section
06).  The readings taken where those pages leave a detail open are listed
with each builder below.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

NONE = -1

# tensor tags used in SeedSequence spawn keys
_TAG_IDS, _TAG_X, _TAG_W0, _TAG_DOWN, _TAG_UP = 0, 1, 2, 3, 4


def _rng(seed: int, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even.

    Inputs are finite draws from normal distributions, so the NaN/overflow
    corner of the rounding rule never arises here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal(seed: int, key, shape, std: float) -> np.ndarray:
    g = _rng(seed, *key)
    return g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


@dataclass
class Workload:
    """One seeded multi-LoRA linear workload (all sizes in elements).

    row_adapter[k] is the adapter id of row k, or -1 for a row served by the
    base weight only.  ranks/scales map each resident adapter id to its rank
    and its fp32 scale.  Tensors are produced on demand by the *_f32 / *_bits
    methods so that large workloads can be sliced.
    """
    name: str
    seed: int
    din: int
    dout: int
    n_proj: int
    row_adapter: np.ndarray
    ranks: Dict[int, int]
    scales: Dict[int, float]
    x_std: float
    w0_std: float
    down_std: float
    up_std: float
    max_adapters: int
    max_rank: int
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.row_adapter.shape[0])

    # fp32 draws (before bf16 rounding)
    def x_f32(self) -> np.ndarray:
        return _normal(self.seed, (_TAG_X,), (self.n, self.din), self.x_std)

    def w0_f32(self, proj: int = 0) -> np.ndarray:
        return _normal(self.seed, (_TAG_W0, proj), (self.dout, self.din), self.w0_std)

    def down_f32(self, adapter: int, proj: int = 0) -> np.ndarray:
        r = self.ranks[adapter]
        return _normal(self.seed, (_TAG_DOWN, adapter, proj), (r, self.din), self.down_std)

    def up_f32(self, adapter: int, proj: int = 0) -> np.ndarray:
        r = self.ranks[adapter]
        return _normal(self.seed, (_TAG_UP, adapter, proj), (self.dout, r), self.up_std)

    # bf16 bit patterns (what the GPU path and the oracle both consume)
    def x_bits(self) -> np.ndarray:
        return round_to_bf16_bits(self.x_f32())

    def w0_bits(self, proj: int = 0) -> np.ndarray:
        return round_to_bf16_bits(self.w0_f32(proj))

    def down_bits(self, adapter: int, proj: int = 0) -> np.ndarray:
        return round_to_bf16_bits(self.down_f32(adapter, proj))

    def up_bits(self, adapter: int, proj: int = 0) -> np.ndarray:
        return round_to_bf16_bits(self.up_f32(adapter, proj))

    def adapter_ids(self) -> List[int]:
        return sorted(self.ranks)

    def down_all_bits(self, adapter: int) -> np.ndarray:
        """[n_proj][rank][din] bf16 bits: the layout a pool load takes."""
        return np.stack([self.down_bits(adapter, p) for p in range(self.n_proj)])

    def up_all_bits(self, adapter: int) -> np.ndarray:
        """[n_proj][dout][rank] bf16 bits: the layout a pool load takes."""
        return np.stack([self.up_bits(adapter, p) for p in range(self.n_proj)])


# ---------------------------------------------------------------------------
# named workloads
# ---------------------------------------------------------------------------

def worked_example() -> Workload:
    """M031 card section 02/03: one linear, din = dout = 4, rows P, Q, R, S on
    adapters A, B, A and none; A has rank 1, B rank 2.  Scale = alpha/r with
    alpha = r, i.e. 1.  Every tensor ~ N(0, 1).  Ids: A -> 0, B -> 1."""
    return Workload(
        name="worked_example_4x4", seed=1001, din=4, dout=4, n_proj=1,
        row_adapter=np.array([0, 1, 0, NONE], dtype=np.int32),
        ranks={0: 1, 1: 2}, scales={0: 1.0, 1: 1.0},
        x_std=1.0, w0_std=1.0, down_std=1.0, up_std=1.0,
        max_adapters=2, max_rank=2,
        notes="rows P,Q,R,S -> A,B,A,none")


_DECODE_STD = dict(x_std=1.0, w0_std=0.02, down_std=1.0 / 64.0, up_std=0.02)


def decode_3_adapters() -> Workload:
    """wiblog vLLM scheduling article, Punica section: one decode step of 32
    tokens (one per request) whose adapters split 20/8/4 over three adapters.
    Projection 4096 x 4096, rank 16, scale 2.0, rows shuffled.  W0 ~ N(0,
    0.02^2), Down ~ N(0, 1/din) (fan-in variance), Up ~ N(0, 0.02^2), X ~ N(0,1)."""
    seed = 1002
    g = _rng(seed, _TAG_IDS)
    ids = np.array([0] * 20 + [1] * 8 + [2] * 4, dtype=np.int32)
    ids = g.permutation(ids).astype(np.int32)
    return Workload(
        name="decode_32tok_3ad_20-8-4", seed=seed, din=4096, dout=4096, n_proj=1,
        row_adapter=ids, ranks={a: 16 for a in range(3)}, scales={a: 2.0 for a in range(3)},
        max_adapters=3, max_rank=16, **_DECODE_STD)


def decode_fragmented() -> Workload:
    """Fully fragmented decode: 256 tokens, each on a distinct adapter out of
    256 resident rank-16 adapters (the article's extreme case of one token per
    adapter, scaled to 256).  Row k -> adapter pi(k), a seeded permutation."""
    seed = 1003
    g = _rng(seed, _TAG_IDS)
    ids = g.permutation(256).astype(np.int32)
    return Workload(
        name="decode_256tok_256ad", seed=seed, din=4096, dout=4096, n_proj=1,
        row_adapter=ids, ranks={a: 16 for a in range(256)}, scales={a: 2.0 for a in range(256)},
        max_adapters=256, max_rank=16, **_DECODE_STD)


def decode_down_projection() -> Workload:
    """The 32-token decode step of decode_3_adapters (20/8/4 over three
    rank-16 adapters, rows shuffled) on the down projection of the prefill
    workload's MLP: din 11008 -> dout 4096, the transpose of its 4096 ->
    11008 shape.  The same distributions as decode_3_adapters (Down ~
    N(0, 1/din) with din = 11008)."""
    seed = 1006
    g = _rng(seed, _TAG_IDS)
    ids = np.array([0] * 20 + [1] * 8 + [2] * 4, dtype=np.int32)
    ids = g.permutation(ids).astype(np.int32)
    std = dict(_DECODE_STD, down_std=1.0 / np.sqrt(11008.0))
    return Workload(
        name="decode_32tok_3ad_down_11008x4096", seed=seed, din=11008, dout=4096, n_proj=1,
        row_adapter=ids, ranks={a: 16 for a in range(3)}, scales={a: 2.0 for a in range(3)},
        max_adapters=3, max_rank=16, **std)


def prefill_hetero() -> Workload:
    """Heterogeneous-rank prefill: din 4096, dout 11008, 4096 tokens in 8
    requests over 6 adapters of ranks {8, 16, 64}; 10% of rows base-only;
    rows interleaved by request.

    Readings: request lengths are 7 uniform integer draws in [64, 1024] with
    the 8th = 4096 - sum, redrawn until it also lies in [64, 1024]; ranks of
    ids 0..5 are [8, 8, 16, 16, 64, 64]; requests 0..5 take a seeded
    permutation of ids 0..5 and requests 6, 7 draw uniformly from them;
    interleaving is round-robin over requests that still have tokens; exactly
    round(0.1 n) = 410 rows, chosen uniformly without replacement, are set to
    -1; scale 2.0 as in the other decode/prefill workloads."""
    seed = 1004
    n = 4096
    g = _rng(seed, _TAG_IDS)
    while True:
        l7 = g.integers(64, 1025, size=7)
        l8 = n - int(l7.sum())
        if 64 <= l8 <= 1024:
            break
    lengths = [int(v) for v in l7] + [l8]
    req_ad = list(g.permutation(6)) + [int(g.integers(0, 6)), int(g.integers(0, 6))]
    left = list(lengths)
    order = []
    while any(left):
        for r in range(8):
            if left[r]:
                order.append(r)
                left[r] -= 1
    ids = np.array([req_ad[r] for r in order], dtype=np.int32)
    none_rows = g.choice(n, size=round(0.1 * n), replace=False)
    ids[none_rows] = NONE
    ranks = {0: 8, 1: 8, 2: 16, 3: 16, 4: 64, 5: 64}
    return Workload(
        name="prefill_4096tok_4096x11008_r8-16-64", seed=seed, din=4096, dout=11008, n_proj=1,
        row_adapter=ids, ranks=ranks, scales={a: 2.0 for a in ranks},
        max_adapters=6, max_rank=64,
        extra=dict(lengths=lengths, request_adapter=[int(a) for a in req_ad],
                   request=np.array(order, dtype=np.int32)),
        **_DECODE_STD)


def layer_stack() -> Workload:
    """Layer-stack serving batch: 32 layers x 2 projections of 4096 x 4096,
    100 resident rank-16 adapters (16 MiB each, 1600 MiB pool), 512 tokens:
    4 prefill requests of 96 tokens (contiguous rows) then 128 decode tokens.
    Each of the 132 requests draws its adapter from a truncated Zipf(1.1) over
    the 100 adapters (P(k) ~ k^-1.1, k = 1..100 -> id k-1); then exactly
    round(0.05 n) = 26 rows, uniform without replacement, are base-only.
    One X feeds every projection independently."""
    seed = 1005
    g = _rng(seed, _TAG_IDS)
    k = np.arange(1, 101, dtype=np.float64)
    pmf = k ** -1.1
    pmf /= pmf.sum()
    req_ad = g.choice(100, size=132, p=pmf)
    ids = np.concatenate([np.repeat(req_ad[:4], 96), req_ad[4:]]).astype(np.int32)
    n = ids.shape[0]
    none_rows = g.choice(n, size=round(0.05 * n), replace=False)
    ids[none_rows] = NONE
    request = np.concatenate([np.repeat(np.arange(4), 96), np.arange(4, 132)]).astype(np.int32)
    return Workload(
        name="layerstack_64proj_100ad_512tok", seed=seed, din=4096, dout=4096, n_proj=64,
        row_adapter=ids, ranks={a: 16 for a in range(100)}, scales={a: 2.0 for a in range(100)},
        max_adapters=100, max_rank=16, extra=dict(request=request), **_DECODE_STD)


NAMED: Dict[str, Callable[[], Workload]] = {
    "worked_example": worked_example,
    "decode_3": decode_3_adapters,
    "decode_frag": decode_fragmented,
    "prefill": prefill_hetero,
    "layer_stack": layer_stack,
    "decode_down": decode_down_projection,
}
ORDER = ["worked_example", "decode_3", "decode_frag", "prefill", "layer_stack", "decode_down"]


def request_rows(w: Workload) -> List[np.ndarray]:
    """The rows of each request of the batch, in request order (each request
    in its original row order).  Workloads that record no request map
    (decode steps, custom batches) have one token per request."""
    req = w.extra.get("request")
    if req is None:
        return [np.array([k]) for k in range(w.n)]
    return [np.flatnonzero(req == r) for r in range(int(req.max()) + 1)]


def custom(name: str, seed: int, din: int, dout: int, row_adapter, ranks: Dict[int, int],
           scales: Optional[Dict[int, float]] = None, n_proj: int = 1,
           max_adapters: Optional[int] = None, max_rank: Optional[int] = None,
           x_std: float = 1.0, w0_std: float = 0.02, down_std: Optional[float] = None,
           up_std: float = 0.02) -> Workload:
    """An arbitrary seeded workload for small parity and edge cases."""
    ra = np.asarray(row_adapter, dtype=np.int32)
    scales = scales if scales is not None else {a: 2.0 for a in ranks}
    return Workload(
        name=name, seed=seed, din=din, dout=dout, n_proj=n_proj, row_adapter=ra,
        ranks=dict(ranks), scales=dict(scales), x_std=x_std, w0_std=w0_std,
        down_std=(down_std if down_std is not None else 1.0 / np.sqrt(din)), up_std=up_std,
        max_adapters=(max_adapters if max_adapters is not None else (max(ranks) + 1 if ranks else 1)),
        max_rank=(max_rank if max_rank is not None else (max(ranks.values()) if ranks else 1)))


def random_ids(seed: int, n: int, adapters: List[int], p_none: float) -> np.ndarray:
    """Row ids drawn uniformly from `adapters`, each row base-only with
    probability p_none."""
    g = _rng(seed, _TAG_IDS, 7)
    ids = g.choice(np.asarray(adapters, dtype=np.int32), size=n)
    ids[g.random(n) < p_none] = NONE
    return ids.astype(np.int32)


def draw_t(seed: int, n: int, max_rank: int, n_chunks: int = 1) -> np.ndarray:
    """Partial low-rank activations fed to the expand step on its own:
    fp32 [n_chunks][n][max_rank] ~ N(0, 1/n_chunks), so each row's sum over
    chunks is ~ N(0, 1)."""
    g = _rng(seed, 5, n, max_rank, n_chunks)
    return (g.standard_normal(size=(n_chunks, n, max_rank), dtype=np.float32)
            * np.float32(1.0 / np.sqrt(n_chunks)))


def draw_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Any other bf16 tensor a test feeds in (e.g. the Y an expand adds to)."""
    return round_to_bf16_bits(_normal(seed, (6,) + tuple(int(s) for s in shape), shape, std))
