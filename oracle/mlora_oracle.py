"""Plain CPU oracle for the heterogeneous multi-LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls this file; only tests/, the
smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
header, table or helper with the GPU path: the only thing both sides take
from elsewhere is the seeded inputs of the `synth` package.

What it computes, and where the pages define it
-----------------------------------------------
Pages cited (by address and section):
  * M031 card - xuujii.github.io/ai-infra-kb/details/M031.html, sections
    01..09 (a Chinese tutorial card on sharing one base among many LoRA
    adapters);
  * airsota card - airsota.com/?p=1825, sections one..seven (an interview
    card on multi-LoRA serving versus merging);
  * wiblog article - wiblog.cn "vLLM LoRA adapter batch scheduling", its
    sections on the baseline methods, on adapter-id mapping and on the
    Punica grouped matmul and in-batch fragmentation.

1. `linear` - the layer itself, per row and with no grouping:
       y_k = W0 x_k + s_a Up_a (Down_a x_k),  a = a(k)
   (M031 card section 02: one shared base product for the whole batch plus
   each row's own low-rank term, zero for a row with no adapter; airsota
   card section three, derivation 1, which writes the same per-query sum in
   row form with scale alpha/r).  Matrices use the column convention of the
   M031 card: W0 is [dout][din], Down is [r][din], Up is [dout][r]
   (the airsota card's A is Down^T and its B is Up^T: same algebra).
   The scale is applied after the Up product, as the M031 card's section 04
   identity writes it.  Arithmetic is float64 unless `dtype` says otherwise.
   A row whose id is neither -1 nor a resident adapter yields NaN: the
   pages leave this case open and a loud result is the reading taken.

2. `segments` - the row grouping the method performs before the low-rank
   products (M031 card section 02: rows of one adapter are gathered, the
   result goes back to each row's original position; section 03 fixes the
   group order P, R, Q for rows P, Q, R, S on A, B, A, none, i.e. ascending
   adapter order and original order inside a group).  Written as the
   textbook stable sort of rows by key, where key = adapter id for a row on
   a resident adapter, then all base-only rows, then all rows with an
   invalid id.

3. `shrink_rows` / `expand_rows` - the two halves of the low-rank term for
   one row (t = Down_a x_k and y += s_a Up_a t), the pieces the grouped
   path splits the branch into (wiblog article, Punica section: each group
   computes its BAx and writes back in original order).

4. `merge` - the merged alternative: W0 + sign * s_a * Up_a Down_a, the
   weight that serves adapter a's rows with the base product alone (M031
   card section 04; airsota card section three, derivation 2); sign = -1
   takes the term out again.

5. Accounting: `branch_flops` / `padded_flops` (M031 card section 03:
   2 * rows * r * (din + dout) per group, and the same with every row padded
   to the largest rank) and `adapter_bytes` (M031 card section 06: rank-r
   factors of one din x dout projection at 2 bytes per parameter).

Pins
----
tests/test_oracle_pins.py ties every function above to something other than
itself: the worked example's group order, write-back rows and FLOP counts
(M031 section 02/03), the page's pool sizes (section 06), the merge identity
(section 04; airsota section three, derivation 2), exact rational brute force
on tiny integer inputs, an exhaustive permutation search for the sort, and
planted mistakes that must fail the parity tolerance.  No function here is
"parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Iterable, Mapping, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "NONE", "STATUS_BAD_ID", "STATUS_NOT_RESIDENT", "Adapter",
    "widen_bf16", "row_keys", "segments", "linear", "shrink_rows", "expand_rows", "merge",
    "branch_flops", "padded_flops", "base_flops", "adapter_bytes", "within_tolerance",
    "max_scaled_error",
]

NONE = -1
STATUS_BAD_ID = 1        # an id < -1 or >= max_adapters appeared
STATUS_NOT_RESIDENT = 2  # an id in range named an adapter with no weights loaded

# (scale, Down [r][din], Up [dout][r]) of one adapter for one projection
Adapter = Tuple[float, np.ndarray, np.ndarray]


def widen_bf16(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float values (a bf16 is the top
    half of an IEEE float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(dtype)


def row_keys(row_adapter: Sequence[int], max_adapters: int,
             resident: Iterable[int]) -> Tuple[np.ndarray, int]:
    """Sort key of every row and the status bits of the batch.

    key = id for a row on a resident adapter; max_adapters for a base-only
    row (id -1); max_adapters + 1 for an invalid id.
    """
    res = set(int(a) for a in resident)
    keys = np.empty(len(row_adapter), dtype=np.int64)
    status = 0
    for k, a in enumerate(row_adapter):
        a = int(a)
        if a == NONE:
            keys[k] = max_adapters
        elif a < NONE or a >= max_adapters:
            keys[k] = max_adapters + 1
            status |= STATUS_BAD_ID
        elif a not in res:
            keys[k] = max_adapters + 1
            status |= STATUS_NOT_RESIDENT
        else:
            keys[k] = a
    return keys, status


def segments(row_adapter: Sequence[int], max_adapters: int,
             resident: Iterable[int]) -> Dict[str, object]:
    """Group rows by adapter: the stable sort of rows by key.

    Returns perm (sorted position -> original row), inv (its inverse),
    seg_adapter (distinct active ids, ascending), seg_off (first sorted
    position of each segment, plus n_act at the end), nseg, n_act, n_none,
    n_bad and status.
    """
    keys, status = row_keys(row_adapter, max_adapters, resident)
    n = len(keys)
    perm = sorted(range(n), key=lambda k: (int(keys[k]), k))
    inv = [0] * n
    for j, k in enumerate(perm):
        inv[k] = j
    seg_adapter, seg_off = [], []
    for j, k in enumerate(perm):
        key = int(keys[k])
        if key >= max_adapters:
            break
        if not seg_adapter or seg_adapter[-1] != key:
            seg_adapter.append(key)
            seg_off.append(j)
    n_act = int(sum(1 for key in keys if key < max_adapters))
    n_none = int(sum(1 for key in keys if key == max_adapters))
    seg_off.append(n_act)
    return dict(
        perm=np.array(perm, dtype=np.int32), inv=np.array(inv, dtype=np.int32),
        seg_adapter=np.array(seg_adapter, dtype=np.int32), seg_off=np.array(seg_off, dtype=np.int32),
        nseg=len(seg_adapter), n_act=n_act, n_none=n_none, n_bad=n - n_act - n_none,
        status=status)


def _row_class(a: int, adapters: Mapping[int, Adapter], max_adapters: int) -> str:
    if a == NONE:
        return "none"
    if a < NONE or a >= max_adapters or a not in adapters:
        return "bad"
    return "lora"


def shrink_rows(X: np.ndarray, row_adapter: Sequence[int], adapters: Mapping[int, Adapter],
                max_adapters: int, rows: Optional[Iterable[int]] = None,
                dtype=np.float64) -> Dict[int, np.ndarray]:
    """t_k = Down_a x_k for every row k on a resident adapter (unscaled)."""
    X = np.asarray(X, dtype=dtype)
    out = {}
    for k in (range(X.shape[0]) if rows is None else rows):
        a = int(row_adapter[k])
        if _row_class(a, adapters, max_adapters) == "lora":
            _, down, _ = adapters[a]
            out[k] = np.asarray(down, dtype=dtype) @ X[k]
    return out


def expand_rows(Y_in: np.ndarray, t: Mapping[int, np.ndarray], row_adapter: Sequence[int],
                adapters: Mapping[int, Adapter], max_adapters: int,
                dtype=np.float64) -> np.ndarray:
    """y_k = y_in_k + s_a Up_a t_k for rows on a resident adapter; NaN rows
    for invalid ids; base-only rows unchanged.  t is given per row."""
    Y = np.array(Y_in, dtype=dtype, copy=True)
    for k in range(Y.shape[0]):
        a = int(row_adapter[k])
        cls = _row_class(a, adapters, max_adapters)
        if cls == "lora":
            s, _, up = adapters[a]
            Y[k] = Y[k] + dtype(s) * (np.asarray(up, dtype=dtype) @ np.asarray(t[k], dtype=dtype))
        elif cls == "bad":
            Y[k] = np.nan
    return Y


def linear(X: np.ndarray, W0: np.ndarray, row_adapter: Sequence[int],
           adapters: Mapping[int, Adapter], max_adapters: int,
           rows: Optional[Sequence[int]] = None, base_batched: bool = False,
           dtype=np.float64) -> np.ndarray:
    """The multi-LoRA linear, one row at a time, with no grouping.

    rows selects which output rows to compute (all by default), in that
    order.  base_batched computes the shared base term of the selected rows
    as one matrix product (the M031 card's "all rows through W" step), which
    is the same arithmetic with a faster library call; the low-rank term is
    always per row.
    """
    X = np.asarray(X, dtype=dtype)
    W0 = np.asarray(W0, dtype=dtype)
    sel = list(range(X.shape[0])) if rows is None else [int(k) for k in rows]
    Y = np.empty((len(sel), W0.shape[0]), dtype=dtype)
    base = (X[sel] @ W0.T) if base_batched else None
    for i, k in enumerate(sel):
        y = base[i].copy() if base_batched else W0 @ X[k]
        a = int(row_adapter[k])
        cls = _row_class(a, adapters, max_adapters)
        if cls == "lora":
            s, down, up = adapters[a]
            t = np.asarray(down, dtype=dtype) @ X[k]
            y = y + dtype(s) * (np.asarray(up, dtype=dtype) @ t)
        elif cls == "bad":
            y[:] = np.nan
        Y[i] = y
    return Y


def merge(W0: np.ndarray, adapter: Adapter, sign: float = 1.0, dtype=np.float64) -> np.ndarray:
    """W0 + sign * s * (Up @ Down) for one adapter's (s, Down, Up), the
    merged weight of the M031 card's section 04 (a new array; W0 is not
    changed)."""
    s, down, up = adapter
    W0 = np.asarray(W0, dtype=dtype)
    return W0 + dtype(sign) * dtype(s) * (np.asarray(up, dtype=dtype) @ np.asarray(down, dtype=dtype))


def branch_flops(active_ranks: Iterable[int], din: int, dout: int) -> int:
    """Low-rank work of the grouped branch: every active row costs
    2 * r * (din + dout) (a multiply and an add per weight of Down and Up)."""
    return int(sum(2 * int(r) * (din + dout) for r in active_ranks))


def padded_flops(n_rows: int, max_rank: int, din: int, dout: int) -> int:
    """The same work when every row of the batch is padded to max_rank."""
    return int(2 * n_rows * max_rank * (din + dout))


def base_flops(n_rows: int, din: int, dout: int) -> int:
    return int(2 * n_rows * din * dout)


def adapter_bytes(din: int, dout: int, rank: int, bytes_per_param: int = 2) -> int:
    """Bytes of one adapter's factors for one din x dout projection."""
    return int(rank * (din + dout) * bytes_per_param)


def max_scaled_error(Y: np.ndarray, ref: np.ndarray) -> float:
    """max |Y - ref| / (1 + |ref|) over all elements (NaN-aware: a NaN
    where ref is not NaN, or vice versa, is an infinite error)."""
    Y = np.asarray(Y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_y, nan_r = np.isnan(Y), np.isnan(ref)
    if np.any(nan_y != nan_r):
        return float("inf")
    ok = ~nan_r
    if not np.any(ok):
        return 0.0
    return float(np.max(np.abs(Y[ok] - ref[ok]) / (1.0 + np.abs(ref[ok]))))


def within_tolerance(Y: np.ndarray, ref: np.ndarray, rtol: float = 2e-2) -> bool:
    """The parity bar for bf16 inputs with fp32 accumulation:
    max |Y - ref| <= rtol * (1 + |ref|) element-wise."""
    return max_scaled_error(Y, ref) <= rtol
