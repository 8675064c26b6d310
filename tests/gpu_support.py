"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
build pools from workloads, and evaluate the oracle on the same inputs.

Inputs come only from the `synth` generators; expected values only from
`oracle`.  Nothing here computes any part of the layer itself.
"""
import sys

import numpy as np
import pytest

import oracle as O

TOL = 2e-2  # max |Y - ref| <= TOL * (1 + |ref|): bf16 inputs, fp32 accumulation


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg: str) -> None:
    """Names the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_to_f64(t) -> np.ndarray:
    torch = torch_cuda()
    return O.widen_bf16(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def ids_dev(ids: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


def pages_needed(w, adapters=None):
    ids = w.adapter_ids() if adapters is None else adapters
    return sum(w.ranks[a] for a in ids) * w.n_proj


def make_pool(M, w, n_pages=None, adapters=None, max_adapters=None, max_rank=None):
    """A pool holding the workload's adapters (all projections)."""
    ids = w.adapter_ids() if adapters is None else adapters
    n_pages = pages_needed(w, ids) if n_pages is None else n_pages
    pool = M.Pool(w.din, w.dout, w.n_proj, max_adapters or w.max_adapters, max_rank or w.max_rank,
                  max(n_pages, 1))
    for a in ids:
        pool.load(a, w.ranks[a], w.scales[a], w.down_all_bits(a), w.up_all_bits(a))
    return pool


def oracle_adapters(w, proj=0, adapters=None):
    ids = w.adapter_ids() if adapters is None else adapters
    return {a: (float(w.scales[a]), O.widen_bf16(w.down_bits(a, proj)), O.widen_bf16(w.up_bits(a, proj)))
            for a in ids}


def assert_close(Y, ref, what: str, tol: float = TOL):
    err = O.max_scaled_error(Y, ref)
    assert err <= tol, f"{what}: max scaled error {err:.3e} > {tol}"
    return err
