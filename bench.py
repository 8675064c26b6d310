#!/usr/bin/env python3
"""Throughput of the heterogeneous multi-LoRA linear on one MI355X.

One step = one batch through the whole layer: build the segments (group rows
by adapter) and apply the layer (the base GEMM Y = X W0^T and the low-rank
branch, shrink and expand), for the variant the library's planner picks, in
one mlora_forward call (--separate-build: mlora_build_segments, then
mlora_apply).
The steps of the timed region are replayed from a captured HIP graph, so the
number is the GPU's, not the Python launcher's.  Inputs are seeded synthetic
tensors already resident in HBM.  Consecutive steps rotate over distinct
copies of W0 and of the adapter pages (distinct projections of one pool), at
least 1 GiB in all, so that the 256 MB last-level cache cannot serve a step
from the previous one.

Prints ONE JSON line: tokens/s (whole batch rows per second of step time),
the dominant kernel's roofline fraction (its algorithmic bytes or flops per
launch over its average duration, from HIP events the library records on the
launch stream right after each of its kernel launches), per-kernel averages,
and the CPU oracle timed on the host cores as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "tokens/s per multi-LoRA linear (4096², r=16) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, published
RIDGE = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
KERNEL_SOURCES = {"seg_build": "seg_build.hip", "gemm_skinny": "base_gemm.hip", "gemm_ksplit": "base_gemm.hip",
                  "gemm_tiled": "base_gemm.hip", "gemm_big": "base_gemm.hip", "gemm_decode": "base_gemm.hip",
                  "gemm_decode+shrink_rows": "base_gemm.hip", "finish_part": "base_gemm.hip",
                  "gemm_decode+seg+shrink_rows": "base_gemm.hip", "gemm_mid+seg+shrink_rows": "base_gemm.hip",
                  "gemm_mid+shrink_rows": "base_gemm.hip",
                  "gemm_mid": "base_gemm.hip", "gemm_skinny_lora": "base_gemm.hip",
                  "gemm_ksplit_lora": "base_gemm.hip", "shrink": "lora_branch.hip", "expand": "lora_branch.hip",
                  "fused": "lora_branch.hip", "shrink_rows": "lora_branch.hip", "shrink_tiles": "lora_branch.hip",
                  "gemm_big_lora": "base_gemm.hip", "lora_prep": "lora_branch.hip", "finish_base": "base_gemm.hip"}
DEFAULT_WORKLOAD = "decode_3"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth.NAMED))
    ap.add_argument("--variant", default="auto", choices=["auto", "split", "fused", "rows"])
    ap.add_argument("--rotate-bytes", type=float, default=1.0, help="GiB of distinct weights to rotate over")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of from a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only --workload (by default the other workloads where a target is judged are timed "
                         "too and reported under \"configs\")")
    ap.add_argument("--config-steps", type=int, default=50, help="timed steps of each of the other workloads")
    ap.add_argument("--separate-build", action="store_true",
                    help="run each step as two library calls (build_segments, then apply) instead of forward")
    ap.add_argument("--copy-only", action="store_true", help="only run the HBM copy calibration kernel")
    ap.add_argument("--yardstick", action="store_true",
                    help="also time the vendor GEMM (torch linear) on the same rotated operands, for context")
    ap.add_argument("--compare-baselines", action="store_true",
                    help="also time the pages' naive baselines on the device: each adapter group served by its own "
                         "launches, and the branch with every adapter padded to the largest rank")
    ap.add_argument("--compare-paging", action="store_true",
                    help="also time the adapter paging lifecycle: one adapter's load from host memory, a step whose "
                         "adapter must be loaded first (miss) against one whose adapters are resident (hit), and "
                         "the step while a second stream reloads a spare adapter into the same pool")
    ap.add_argument("--compare-merged", action="store_true",
                    help="also time the merged alternative: merge/unmerge of one adapter into W0, the plain GEMM "
                         "on merged weights, and serving the batch adapter by adapter from merged weights")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work per launch (what the method must move / compute)
# ---------------------------------------------------------------------------

def segment_sizes(w):
    ids = w.row_adapter
    act = ids[(ids >= 0) & np.isin(ids, w.adapter_ids())]
    counts = np.bincount(act, minlength=w.max_adapters)
    segs = [(a, int(c), w.ranks[a]) for a, c in enumerate(counts) if c > 0]
    return segs, int(act.size)


def algorithmic(w, chunks):
    """{kernel: (bytes, flops)} per launch: what the step must move and
    compute, split over the library's kernels (scratch such as split-K
    partials is not counted)."""
    n, din, dout = w.n, w.din, w.dout
    segs, n_act = segment_sizes(w)
    sum_r = sum(r for _, _, r in segs)
    sum_nr = sum(c * r for _, c, r in segs)
    base = (2 * (dout * din + n * din + n * dout), 2 * n * din * dout)
    shrink_rows = (2 * sum_r * din + 2 * n_act * din + 4 * sum_nr, 2 * sum_nr * din)
    split_dense = (2 * (dout * din + n * din), 2 * n * din * dout)   # Y comes from the finish pass
    finish = (2 * sum_r * dout + 4 * sum_nr + 2 * n * dout, 2 * sum_nr * dout)
    gemm_lora = (base[0] + 2 * sum_r * dout + 4 * sum_nr, base[1] + 2 * sum_nr * dout)
    seg = (4 * n + 4 * 4 * n, 0)   # ids in; perm, inv, row keys and segment tables out
    # the shrink inside a GEMM launch works from the X rows that launch
    # already reads for the base product: only the Down rows and T are extra
    shrink_in_launch = (2 * sum_r * din + 4 * sum_nr, 2 * sum_nr * din)
    out = {
        "seg_build": seg,
        "shrink": (2 * sum_r * din + 2 * n_act * din + 4 * sum_nr * max(chunks, 1), 2 * sum_nr * din),
        "expand": (2 * sum_r * dout + 4 * n_act * dout + 4 * sum_nr * max(chunks, 1), 2 * sum_nr * dout),
        "fused": (2 * sum_r * (din + dout) + 2 * n_act * din + 4 * n_act * dout, 2 * sum_nr * (din + dout)),
        "shrink_rows": shrink_rows,
        "gemm_decode": split_dense, "gemm_mid": split_dense,
        "gemm_decode+shrink_rows": (split_dense[0] + shrink_in_launch[0], split_dense[1] + shrink_in_launch[1]),
        "gemm_mid+shrink_rows": (split_dense[0] + shrink_in_launch[0], split_dense[1] + shrink_in_launch[1]),
        "gemm_decode+seg+shrink_rows": (split_dense[0] + shrink_in_launch[0] + seg[0],
                                        split_dense[1] + shrink_in_launch[1]),
        "gemm_mid+seg+shrink_rows": (split_dense[0] + shrink_in_launch[0] + seg[0],
                                     split_dense[1] + shrink_in_launch[1]),
        "finish_part": finish,
        "finish_base": (2 * n * dout, 0),   # the base GEMM's partials summed (scratch) into Y
        "gemm_skinny_lora": gemm_lora, "gemm_ksplit_lora": gemm_lora, "gemm_big_lora": gemm_lora,
        # the large GEMM's low-rank operands: chunk partials in, bf16 t per row out; Up
        # pages in, the same Up with ranks contiguous out
        "lora_prep": (4 * sum_nr * max(chunks, 1) + 2 * sum_nr + 4 * sum_r * dout, sum_nr * max(chunks, 1)),
        "shrink_tiles": (2 * sum_r * din + 2 * n_act * din + 4 * sum_nr * max(chunks, 1), 2 * sum_nr * din),
    }
    for k in ("gemm_skinny", "gemm_ksplit", "gemm_tiled", "gemm_big"):
        out[k] = base
    return out


DENSE = ("gemm_skinny", "gemm_ksplit", "gemm_tiled", "gemm_big", "gemm_decode", "gemm_mid", "gemm_mid+shrink_rows",
         "gemm_decode+shrink_rows", "gemm_decode+seg+shrink_rows", "gemm_mid+seg+shrink_rows", "gemm_skinny_lora",
         "gemm_ksplit_lora",
         "gemm_big_lora")


def source_hash(kernel):
    """Hash of the kernel's source file and the headers every kernel shares."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, "lora_serving_mlora_amd", "csrc")
    src = KERNEL_SOURCES[kernel.split("#")[0]]
    shared = ("internal.h", "row_kernels.h") + (("seg_device.h",) if src in ("base_gemm.hip", "seg_build.hip") else ())
    for f in (src,) + shared:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the kernel source as it is now (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            rec = json.load(f).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# the merged alternative (M031 card section 04; airsota card section three)
# ---------------------------------------------------------------------------

def compare_merged(M, torch, w, pool, X, W0s, R, seg_ws, Y, work, variant, iters=50):
    """Times, with events on the launch stream and the same W0 rotation:
    the grouped layer on a batch whose rows all use one adapter against the
    plain GEMM on that adapter's merged weight (the overhead the pages put
    at 10-25 %); one merge and one unmerge; and the mixed batch served
    adapter by adapter from merged weights (merge, GEMM over its rows,
    unmerge) against the grouped layer."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        for i in range(min(iters, 2 * R)):
            fn(i)
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(iters):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / iters * 1e3

    n = w.n
    a0 = w.adapter_ids()[0]
    ids1 = torch.full((n,), a0, dtype=torch.int32, device="cuda")
    seg1 = M.build_segments(pool, ids1)
    grouped_one = timed(lambda i: M.apply(pool, i % R, X, W0s[i % R], seg1, Y=Y, work=work, variant=variant))
    Wm = [W.clone() for W in W0s]
    for p in range(R):
        M.merge(pool, a0, p, Wm[p], 1.0)
    merged_gemm = timed(lambda i: M.base_gemm(X, Wm[i % R], Y))
    merge_us = timed(lambda i: M.merge(pool, a0, i % R, Wm[i % R], 1.0 if i % 2 == 0 else -1.0))
    del Wm
    ids = w.row_adapter
    groups = [(a, torch.from_numpy(np.flatnonzero(ids == a)).cuda()) for a in w.adapter_ids() if (ids == a).any()]
    base_rows = torch.from_numpy(np.flatnonzero(ids < 0)).cuda()
    Xa = [(a, X.index_select(0, r).contiguous(), r) for a, r in groups]
    Xb = X.index_select(0, base_rows).contiguous() if len(base_rows) else None
    Ya = [torch.empty((len(r), w.dout), dtype=torch.bfloat16, device="cuda") for _, r in groups]
    Yb = torch.empty((len(base_rows), w.dout), dtype=torch.bfloat16, device="cuda") if len(base_rows) else None

    Wc = [W.clone() for W in W0s]  # merged in place: keep W0s untouched

    def merged_serving(i):
        p = i % R
        if Xb is not None:
            M.base_gemm(Xb, Wc[p], Yb)
        for (a, xa, _), ya in zip(Xa, Ya):
            M.merge(pool, a, p, Wc[p], 1.0)
            M.base_gemm(xa, Wc[p], ya)
            M.merge(pool, a, p, Wc[p], -1.0)

    ids_dev = torch.from_numpy(ids.astype(np.int32)).cuda()

    def grouped(i):
        M.build_segments(pool, ids_dev, seg_ws)
        M.apply(pool, i % R, X, W0s[i % R], seg_ws, Y=Y, work=work, variant=variant)

    grouped_mixed = timed(grouped)
    merged_mixed = timed(merged_serving)
    return {"adapter": int(a0), "rows": int(n),
            "one_adapter": {"grouped_apply_us": round(grouped_one, 3), "merged_gemm_us": round(merged_gemm, 3),
                            "grouped_over_merged_pct": round(100.0 * (grouped_one / merged_gemm - 1.0), 1)},
            "merge_or_unmerge_us": round(merge_us, 3),
            "mixed_batch": {"adapters": len(groups), "grouped_step_us": round(grouped_mixed, 3),
                            "merged_serving_us": round(merged_mixed, 3)},
            "timing": f"torch events on the launch stream around {iters} eager iterations, same W0 rotation; "
                      "merged serving = per adapter merge + GEMM over its rows + unmerge (base-only rows on W0)"}


# ---------------------------------------------------------------------------
# the pages' naive baselines on the device (wiblog article, baseline methods;
# M031 card section 03, padded FLOPs)
# ---------------------------------------------------------------------------

def compare_baselines(M, torch, w, pool, X, W0s, R, seg_ws, Y, work, variant, iters=30):
    """Times, with events on the launch stream and the same W0 rotation:
    the grouped layer (segments + apply); the batch served group by group,
    each adapter's rows through their own segment build and apply and the
    base-only rows through the plain GEMM (per-request application: many
    small launches); and the grouped layer on a pool where every adapter is
    zero-padded to the largest rank (what a padded dense branch computes:
    the same outputs, max_rank work per row)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, iters=iters):
        for i in range(min(iters, 2 * R)):
            fn(i)
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(iters):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / iters * 1e3

    ids = w.row_adapter
    ids_dev = torch.from_numpy(ids.astype(np.int32)).cuda()

    def grouped(i):
        M.build_segments(pool, ids_dev, seg_ws)
        M.apply(pool, i % R, X, W0s[i % R], seg_ws, Y=Y, work=work, variant=variant)

    t_grouped = timed(grouped)

    groups = []
    for a in w.adapter_ids():
        rows = np.flatnonzero(ids == a)
        if len(rows):
            r = torch.from_numpy(rows).cuda()
            xa = X.index_select(0, r).contiguous()
            ia = torch.full((len(rows),), a, dtype=torch.int32, device="cuda")
            groups.append((xa, ia, M.build_segments(pool, ia), torch.empty((len(rows), w.dout),
                          dtype=torch.bfloat16, device="cuda"), M.new_work(pool, len(rows))))
    base_rows = np.flatnonzero(ids < 0)
    xb = X.index_select(0, torch.from_numpy(base_rows).cuda()).contiguous() if len(base_rows) else None
    yb = torch.empty((len(base_rows), w.dout), dtype=torch.bfloat16, device="cuda") if len(base_rows) else None

    def per_group(i):
        p = i % R
        if xb is not None:
            M.base_gemm(xb, W0s[p], yb)
        for xa, ia, sa, ya, wa in groups:
            M.build_segments(pool, ia, sa)
            M.apply(pool, p, xa, W0s[p], sa, Y=ya, work=wa)

    t_serial = timed(per_group)

    # per-request serial application (wiblog article, baseline methods):
    # every request through its own layer call (segment build and layer for
    # its rows alone); its output stays in the request's own buffer
    reqs = []
    for rows in synth.request_rows(w):
        r = torch.from_numpy(rows).cuda()
        reqs.append((X.index_select(0, r).contiguous(), torch.from_numpy(ids[rows].astype(np.int32)).cuda(),
                     torch.empty(M.segments_bytes(len(rows)) // 4, dtype=torch.int32, device="cuda"),
                     torch.empty((len(rows), w.dout), dtype=torch.bfloat16, device="cuda"),
                     M.new_work(pool, len(rows))))

    def per_request(i):
        p = i % R
        for xr, ir, sr, yr, wr in reqs:
            M.forward(pool, p, xr, W0s[p], ir, seg_ws=sr, Y=yr, work=wr)

    t_per_request = timed(per_request, iters=max(3, min(iters, 3000 // max(len(reqs), 1))))

    # every adapter padded to the largest rank with zero factors
    rmax = max(w.ranks.values())
    n_pages = len(w.ranks) * rmax * R
    padded = M.Pool(w.din, w.dout, R, w.max_adapters, w.max_rank, n_pages)
    for a in w.adapter_ids():
        r = w.ranks[a]
        d = np.zeros((R, rmax, w.din), dtype=np.uint16)
        u = np.zeros((R, w.dout, rmax), dtype=np.uint16)
        for p in range(R):
            d[p, :r] = w.down_bits(a, p if w.n_proj > 1 else 0)
            u[p, :, :r] = w.up_bits(a, p if w.n_proj > 1 else 0)
        padded.load(a, rmax, w.scales[a], d, u)
    seg_p = M.build_segments(padded, ids_dev)
    work_p = M.new_work(padded, w.n)
    Yp = torch.empty_like(Y)

    def padded_step(i):
        M.build_segments(padded, ids_dev, seg_p)
        M.apply(padded, i % R, X, W0s[i % R], seg_p, Y=Yp, work=work_p, variant=variant)

    t_padded = timed(padded_step)
    del padded
    return {"grouped_step_us": round(t_grouped, 3),
            "per_group_launches_us": round(t_serial, 3), "groups": len(groups),
            "per_request_serial_us": round(t_per_request, 3), "requests": len(reqs),
            "padded_to_max_rank_us": round(t_padded, 3), "max_rank": rmax,
            "timing": f"torch events on the launch stream around {iters} eager iterations, same W0 rotation"}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def compare_paging(M, torch, w, pool, step_fn, spare_id, R, iters=20):
    """The host<->HBM paging lifecycle (M031 card sections 06-07; wiblog
    memory-cost section): the adapter of the batch's largest group is
    unloaded and loaded again from host memory (pinned staging; its R
    projections), and the same step is timed with and without a reload of
    a spare adapter (an id no row uses) on a second stream into the same
    pool."""
    import collections
    a = collections.Counter(int(x) for x in w.row_adapter if x >= 0).most_common(1)[0][0]
    rank = w.ranks[a]
    d = np.ascontiguousarray(np.repeat(w.down_bits(a, 0)[None], R, axis=0))
    u = np.ascontiguousarray(np.repeat(w.up_bits(a, 0)[None], R, axis=0))
    nbytes = 2 * R * rank * (w.din + w.dout)
    torch.cuda.synchronize()
    loads = []
    for _ in range(5):
        pool.unload(a)
        t0 = time.perf_counter()
        pool.load(a, rank, w.scales[a], d, u)
        torch.cuda.synchronize()
        loads.append(time.perf_counter() - t0)
    load_ms = float(np.median(loads)) * 1e3

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    for i in range(3):
        step_fn(i)
    hit_ms = timed(step_fn, iters)

    def miss(i):
        pool.unload(a)
        pool.load(a, rank, w.scales[a], d, u)
        step_fn(i)
    miss_ms = timed(miss, 5)

    copy = torch.cuda.Stream()
    pool.load(spare_id, rank, w.scales[a], d, u)

    def reload_spare(i):
        with torch.cuda.stream(copy):
            pool.unload(spare_id)
            pool.load(spare_id, rank, w.scales[a], d, u)

    def overlapped(i):
        reload_spare(i)
        step_fn(i)
    for i in range(2):
        overlapped(i)
    ov_ms = timed(overlapped, iters)
    spare_ms = timed(reload_spare, 5)
    return {"adapter": a, "adapter_bytes": nbytes, "projections": R,
            "load_ms": round(load_ms, 3), "load_gbps": round(nbytes / (load_ms * 1e-3) / 1e9, 2),
            "step_hit_us": round(hit_ms * 1e3, 2), "step_miss_us": round(miss_ms * 1e3, 2),
            "spare_reload_alone_us": round(spare_ms * 1e3, 2),
            "step_with_spare_reload_on_copy_stream_us": round(ov_ms * 1e3, 2),
            "timing": "host clock around synchronised loops of eager launches"}


def cpu_baseline(w, seconds):
    """The oracle as it stands, in fp32, on this host: the per-row loop over
    the workload's rows (projection 0).  Three runs with the BLAS library's
    own thread count and three with one thread, each about seconds / 6 long;
    the medians are reported (tokens/s = rows done / time)."""
    import oracle as O
    blas = {}
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = {"internal_api": info[0].get("internal_api"), "version": info[0].get("version"),
                "threading_layer": info[0].get("threading_layer")} if info else {}
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    X = O.widen_bf16(w.x_bits(), np.float32)
    W0 = O.widen_bf16(w.w0_bits(0), np.float32)
    ad = {a: (float(w.scales[a]), O.widen_bf16(w.down_bits(a, 0), np.float32),
              O.widen_bf16(w.up_bits(a, 0), np.float32)) for a in w.adapter_ids()}
    block = min(w.n, 64)

    def run(budget):
        rows_done, start, t0 = 0, 0, time.perf_counter()
        while True:
            rows = [(start + i) % w.n for i in range(block)]
            O.linear(X, W0, w.row_adapter, ad, w.max_adapters, rows=rows, dtype=np.float32)
            rows_done += block
            start = (start + block) % w.n
            el = time.perf_counter() - t0
            if el >= budget and rows_done >= block:
                return rows_done, el

    per = seconds / 6
    full = [run(per) for _ in range(3)]
    single = []
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            single = [run(per) for _ in range(3)]
    rate = lambda runs: float(np.median([r / el for r, el in runs]))
    rows_total = sum(r for r, _ in full)
    out = {"value": rate(full), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"3 runs of about {per:.1f} s ({rows_total} rows in all) of the {w.name} batch "
                     f"(projection 0), per-row fp32 numpy loop of the oracle, median; "
                     f"{os.cpu_count()} host cores, BLAS with {threads} threads",
           "runs_tokens_per_s": [round(r / el, 1) for r, el in full], "blas": blas}
    if single:
        out["value_1thread"] = rate(single)
        out["runs_1thread_tokens_per_s"] = [round(r / el, 1) for r, el in single]
    return out


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------

def copy_calibration(M, torch, gib=1.0, reps=10):
    """Achievable HBM rates: the library's streaming copy (1 GiB read + 1 GiB
    written per launch), its streaming read (1 GiB read) and the same read
    through LDS DMA (the ring GEMMs' operand path)."""
    nb = int(gib * 2 ** 30)
    src = torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_copy = timed(lambda: M.hbm_copy(dst, src))
    ms_read = timed(lambda: M.hbm_read(src, out))
    ms_read_lds = timed(lambda: M.hbm_read_lds(src, out))
    del src, dst
    return {"bytes_copied": 2 * nb, "copy_ms": ms_copy, "copy_gbps": 2 * nb / ms_copy / 1e6,
            "bytes_read": nb, "read_ms": ms_read, "read_gbps": nb / ms_read / 1e6,
            "read_lds_ms": ms_read_lds, "read_lds_gbps": nb / ms_read_lds / 1e6}


def run_workload(M, torch, name, steps, warmup, variant_arg="auto", rotate_bytes=1.0, separate_build=False,
                 no_graph=False, spare_adapter=False):
    """Builds the workload on the device and times K steps of it (segment
    build + layer for one projection per step, from a captured HIP graph),
    then the same steps eagerly with the library's launch timing.  Returns
    the measured figures and the objects the comparisons reuse."""
    w = synth.NAMED[name]()
    n = w.n
    # rotation: distinct projections of one pool, each with its own W0 copy
    per_proj = 2 * w.din * w.dout + 2 * sum(w.ranks.values()) * (w.din + w.dout)
    R = max(1, math.ceil(rotate_bytes * 2 ** 30 / per_proj))
    if w.n_proj > 1:
        R = w.n_proj   # the workload is a layer stack: rotate over its own projections
    print(f"[bench] workload {w.name}: n={n} din={w.din} dout={w.dout} adapters={len(w.ranks)} "
          f"rotation={R} projections", file=sys.stderr, flush=True)

    n_pages = sum(w.ranks.values()) * R
    max_adapters = w.max_adapters
    if spare_adapter:
        # one more id (no row uses it) and pages for a spare adapter
        max_adapters += 1
        n_pages += max(w.ranks.values()) * R
    pool = M.Pool(w.din, w.dout, R, max_adapters, w.max_rank, n_pages)
    for a in w.adapter_ids():
        if w.n_proj > 1:
            d, u = w.down_all_bits(a), w.up_all_bits(a)
        else:   # the same weights at R distinct addresses
            d = np.repeat(w.down_bits(a, 0)[None], R, axis=0)
            u = np.repeat(w.up_bits(a, 0)[None], R, axis=0)
        pool.load(a, w.ranks[a], w.scales[a], d, u)
    X = torch.from_numpy(w.x_bits().view(np.int16)).view(torch.bfloat16).cuda()
    if w.n_proj > 1:
        W0s = [torch.from_numpy(w.w0_bits(p).view(np.int16)).view(torch.bfloat16).cuda() for p in range(R)]
    else:
        W00 = torch.from_numpy(w.w0_bits(0).view(np.int16)).view(torch.bfloat16).cuda()
        W0s = [W00.clone() for _ in range(R)]
        del W00
    ids = torch.from_numpy(w.row_adapter.astype(np.int32)).cuda()
    seg_ws = M.build_segments(pool, ids)
    Y = torch.empty((n, w.dout), dtype=torch.bfloat16, device="cuda")
    variant, chunks = M.plan(pool, n, variant_arg)
    torch.cuda.synchronize()
    print(f"[bench] plan: variant={variant} shrink_chunks={chunks}", file=sys.stderr, flush=True)

    work = M.new_work(pool, n)

    if separate_build:
        def step(i):
            p = i % R
            M.build_segments(pool, ids, seg_ws)
            M.apply(pool, p, X, W0s[p], seg_ws, Y=Y, work=work, variant=variant)
    else:
        def step(i):
            # segment build + layer in one library call (one launch fewer
            # where the build rides in the GEMM launch)
            p = i % R
            M.forward(pool, p, X, W0s[p], ids, seg_ws=seg_ws, Y=Y, work=work, variant=variant)

    K, W = steps, warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps replayed from one captured HIP graph
    use_graph = not no_graph
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(K):
                    step(W + i)
            graph.replay()           # warm replay (untimed)
            torch.cuda.synchronize()
        except Exception as e:  # fall back to eager launches
            print(f"[bench] graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            graph, use_graph = None, False
            torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            step(W + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    print(f"[bench] timed {K} steps: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    # ---- per-kernel durations: the library records a HIP event on the launch
    # stream right after each of its kernel launches; the same K steps are
    # launched eagerly behind a spin kernel so the queue is full and host
    # launch gaps stay out of the intervals
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is not None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        spin(1_000_000)
        b.record()
        torch.cuda.synchronize()
        per_cycle_ms = max(a.elapsed_time(b), 1e-3) / 1_000_000
        spin_cycles = int(min(5e9, (0.05 + 100e-6 * K) * 1e3 / per_cycle_ms))
    torch.cuda.synchronize()
    if spin is not None:
        spin(spin_cycles)
    KT = min(K, 2048 // 8)
    M.timing_arm(2048)
    t2 = time.perf_counter()
    for i in range(KT):
        step(W + i)
    host_enqueue_s = time.perf_counter() - t2
    marks = M.timing_read()
    torch.cuda.synchronize()
    per_step = len(marks) // KT
    kernels = [marks[j][0] for j in range(per_step)]
    per_kernel_ms = {}
    for j, kname in enumerate(kernels):
        key = kname if kname not in per_kernel_ms else f"{kname}#{j}"
        per_kernel_ms[key] = float(np.mean([marks[i * per_step + j][1] for i in range(KT)]))
    kernel_sum_ms = float(np.mean([sum(m[1] for m in marks[i * per_step:(i + 1) * per_step]) for i in range(KT)]))
    queue_ok = spin is not None and host_enqueue_s * 1e3 < (0.05 + 100e-6 * K) * 1e3
    timing = ("kernel start/end HIP events stamped by the runtime on each library launch (hipExtLaunchKernel), "
              f"eager pass of {KT} steps behind a spin kernel "
              f"({'queue stayed full' if queue_ok else 'queue may have drained'})")
    if not bool(torch.isfinite(Y.float()).all()):
        print("[bench] warning: non-finite outputs", file=sys.stderr)

    algo = algorithmic(w, chunks)
    timed = {k: v for k, v in per_kernel_ms.items() if v}
    dom = max((k for k in timed if k != "seg_build"), key=lambda k: timed[k])
    b, f = algo[dom.split("#")[0]]
    t_s = timed[dom] * 1e-3
    mfma_bound = dom.split("#")[0] in DENSE and f / b > RIDGE
    if mfma_bound:
        ach, peak, unit = f / t_s / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"
    else:
        ach, peak, unit = b / t_s / 1e9, HBM_PEAK_GBS, "GB/s"
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "kernel": dom, "achieved": round(ach, 2),
                "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom, name),
                "algorithmic_bytes": b, "algorithmic_flops": f, "avg_us": round(timed[dom] * 1e3, 3),
                "timing": timing}

    ctx = dict(w=w, pool=pool, X=X, W0s=W0s, R=R, seg_ws=seg_ws, Y=Y, work=work, variant=variant, step=step,
               max_adapters=max_adapters, spin=spin, spin_cycles=spin_cycles if spin is not None else 0, K=K,
               use_graph=use_graph)
    meas = dict(n=n, ms_per_step=ms_per_step, per_kernel_ms=per_kernel_ms, kernel_sum_ms=kernel_sum_ms,
                roofline=roofline, chunks=chunks, variant=variant, R=R, use_graph=use_graph)
    return meas, ctx


def config_summary(name, meas):
    """The figures of one workload for the bench line."""
    n, t = meas["n"], meas["ms_per_step"] * 1e-3
    out = {"tokens_per_s": round(n / t, 1), "us_per_step": round(t * 1e6, 3), "n_tokens": n,
           "variant": meas["variant"], "launch": "hipgraph" if meas["use_graph"] else "eager",
           "per_kernel_us": {k: (round(v * 1e3, 3) if v else None) for k, v in meas["per_kernel_ms"].items()},
           "roofline": meas["roofline"]}
    if name == "layer_stack":
        # the step is one of the stack's 64 projections (all independent,
        # one X): the stack takes 64 steps
        out["stack_tokens_per_s"] = round(n / (64 * t), 1)
        out["stack_us"] = round(64 * t * 1e6, 2)
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no multi-GPU path; "
              "the layer shards by adapter-affine routing or by dout columns with no exchange inside the "
              "linear (see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    import lora_serving_mlora_amd as M
    M.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_only:
        cal = copy_calibration(M, torch)
        print(json.dumps({"copy_calibration": cal}))
        return

    meas, ctx = run_workload(M, torch, args.workload, args.steps, args.warmup, args.variant, args.rotate_bytes,
                             args.separate_build, args.no_graph, args.compare_paging)
    w, pool, X, W0s, R = ctx["w"], ctx["pool"], ctx["X"], ctx["W0s"], ctx["R"]
    seg_ws, Y, work, variant = ctx["seg_ws"], ctx["Y"], ctx["work"], ctx["variant"]
    n, K, W = w.n, args.steps, args.warmup
    ms_per_step = meas["ms_per_step"]

    yardstick = None
    if args.yardstick:
        # the vendor library's GEMM on the same operands and rotation, as a
        # point of comparison for the base GEMM only (not part of the path)
        import torch.nn.functional as F
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(min(K, 2 * R)):
            F.linear(X, W0s[i % R])
        torch.cuda.synchronize()
        if ctx["spin"] is not None:
            ctx["spin"](ctx["spin_cycles"])
        ev[0].record()
        for i in range(K):
            F.linear(X, W0s[i % R])
        ev[1].record()
        torch.cuda.synchronize()
        yardstick = round(ev[0].elapsed_time(ev[1]) / K * 1e3, 3)

    tokens_per_s = n / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": n, "din": w.din, "dout": w.dout,
                   "adapters": len(w.ranks), "ranks": sorted(set(w.ranks.values())),
                   "variant": variant, "shrink_chunks": meas["chunks"], "rotation_projections": R,
                   "step": "build_segments+apply" if args.separate_build else "forward",
                   "launch": "hipgraph" if meas["use_graph"] else "eager", "parallelism": "single-gpu"},
        "roofline": meas["roofline"],
        "per_kernel_us": {k: (round(v * 1e3, 3) if v else None) for k, v in meas["per_kernel_ms"].items()},
        "kernel_sum_us": round(meas["kernel_sum_ms"] * 1e3, 3),
        "gpu_name": torch.cuda.get_device_name(0),
    }
    if yardstick is not None:
        result["vendor_gemm_us"] = yardstick
    if args.compare_baselines:
        result["baseline_comparison"] = compare_baselines(M, torch, w, pool, X, W0s, R, seg_ws, Y, work, variant)
    if args.compare_merged:
        result["merged_comparison"] = compare_merged(M, torch, w, pool, X, W0s, R, seg_ws, Y, work, variant)
    if args.compare_paging:
        result["paging_comparison"] = (None if w.n_proj > 1 else
                                       compare_paging(M, torch, w, pool, ctx["step"], ctx["max_adapters"] - 1, R))
    del ctx, pool, X, W0s, seg_ws, Y, work
    torch.cuda.empty_cache()
    if not args.no_configs:
        # the other workloads where a target is judged, and the decode step
        # on a down projection (din 11008), each timed the same way (its own
        # seeded inputs, its own rotation) with fewer steps
        configs = {}
        for other in ("decode_frag", "prefill", "layer_stack", "decode_down"):
            if other == args.workload:
                continue
            m2, c2 = run_workload(M, torch, other, max(3, min(K, args.config_steps)), min(W, 5))
            configs[other] = config_summary(other, m2)
            del c2
            torch.cuda.empty_cache()
        result["configs"] = configs
    cal = copy_calibration(M, torch)
    result["hbm_copy_gbps"] = round(cal["copy_gbps"], 1)
    result["hbm_read_gbps"] = round(cal["read_gbps"], 1)
    result["hbm_read_lds_gbps"] = round(cal["read_lds_gbps"], 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
