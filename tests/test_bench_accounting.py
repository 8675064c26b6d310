"""Host logic of the bench: its algorithmic work per launch (the numerator
of every roofline fraction it reports), checked against a brute-force count
on a tiny batch, and its refusal of more than one GPU.

The count enumerates the distinct elements each step must touch and the
multiply-adds it must do, straight from the layer's definition: the base
product reads W0 and X and writes Y; the shrink reads the Down rows of each
adapter in use and the X rows of its tokens and writes one fp32 t per (row,
rank); the expand reads the Up columns and t and adds into Y (M031 card
section 02, one shared base product plus each row's low-rank branch;
wiblog article, Punica section, the shrink and expand split).  Rows without an adapter, or with one that is not resident, take no
part in the low-rank branch.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _count(w):
    resident = set(w.ranks)
    x_act, down, up, t, y_act = set(), set(), set(), set(), set()
    mac_shrink = mac_expand = 0
    for k, a in enumerate(w.row_adapter.tolist()):
        if a < 0 or a not in resident:
            continue
        r = w.ranks[a]
        for i in range(w.din):
            x_act.add((k, i))
        for o in range(w.dout):
            y_act.add((k, o))
        for j in range(r):
            t.add((k, j))
            for i in range(w.din):
                down.add((a, j, i))
                mac_shrink += 1
            for o in range(w.dout):
                up.add((a, o, j))
                mac_expand += 1
    return dict(x_act=len(x_act), down=len(down), up=len(up), t=len(t), y_act=len(y_act),
                mac_shrink=mac_shrink, mac_expand=mac_expand)


def _workload():
    # id 5 is not resident, id 3 is resident but unused, -1 rows are base-only
    ids = [0, 1, -1, 0, 2, 5, 1, 1, -1, 0, 2]
    return synth.custom("accounting", 3, 24, 40, ids, {0: 3, 1: 5, 2: 1, 3: 4}, max_adapters=6)


def test_low_rank_kernels_match_the_element_count():
    w = _workload()
    c = _count(w)
    algo = bench.algorithmic(w, chunks=1)
    assert algo["fused"] == (2 * (c["down"] + c["up"] + c["x_act"]) + 4 * c["y_act"],
                             2 * (c["mac_shrink"] + c["mac_expand"]))
    assert algo["shrink_rows"] == (2 * (c["down"] + c["x_act"]) + 4 * c["t"], 2 * c["mac_shrink"])
    assert algo["finish_part"] == (2 * c["up"] + 4 * c["t"] + 2 * w.n * w.dout, 2 * c["mac_expand"])
    assert algo["expand"] == (2 * c["up"] + 4 * c["t"] + 4 * c["y_act"], 2 * c["mac_expand"])
    for chunks in (1, 3):
        a = bench.algorithmic(w, chunks=chunks)
        assert a["shrink"] == (2 * (c["down"] + c["x_act"]) + 4 * c["t"] * chunks, 2 * c["mac_shrink"])


def test_base_and_combined_kernels_match_the_element_count():
    w = _workload()
    c = _count(w)
    algo = bench.algorithmic(w, chunks=1)
    w0, x, y = w.dout * w.din, w.n * w.din, w.n * w.dout
    dense = 0
    for _ in range(w.n):
        dense += w.din * w.dout
    for k in ("gemm_skinny", "gemm_ksplit", "gemm_tiled", "gemm_big"):
        assert algo[k] == (2 * (w0 + x + y), 2 * dense)
    # the split-K forms leave Y to the finish pass
    assert algo["gemm_decode"] == (2 * (w0 + x), 2 * dense)
    # the shrink inside the GEMM launch reads its X rows from what the base
    # product already reads: X counts once
    fused_in = algo["gemm_decode+shrink_rows"]
    assert fused_in == (2 * (w0 + x) + 2 * c["down"] + 4 * c["t"], 2 * (dense + c["mac_shrink"]))
    assert algo["gemm_mid+shrink_rows"] == fused_in
    # the decode launch that also builds the segments: ids in, the
    # workspace's per-row arrays out (perm, inv, key, item and tile entries)
    assert algo["gemm_decode+seg+shrink_rows"] == (fused_in[0] + algo["seg_build"][0], fused_in[1])
    assert algo["seg_build"] == (4 * w.n + 16 * w.n, 0)
    lora = algo["gemm_big_lora"]
    assert lora == (2 * (w0 + x + y) + 2 * c["up"] + 4 * c["t"], 2 * (dense + c["mac_expand"]))


def test_empty_branch_counts_nothing_low_rank():
    w = synth.custom("accounting_none", 4, 16, 8, [-1, -1, 7], {0: 2})
    algo = bench.algorithmic(w, chunks=2)
    assert algo["fused"] == (0, 0)
    assert algo["shrink_rows"] == (0, 0)
    assert algo["finish_part"] == (2 * w.n * w.dout, 0)


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU; asking for more exits with status 2 and says
    why, before touching any device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_run_workload_keeps_the_workload_name_for_the_traffic_lookup():
    """The measured-traffic lookup is keyed by (kernel, workload): nothing in
    run_workload may rebind its `name` parameter (a loop variable of that
    name once made every lookup miss)."""
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    fn = next(n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef) and n.name == "run_workload")
    assert "name" in [a.arg for a in fn.args.args]
    rebound = [n.lineno for n in ast.walk(fn)
               if isinstance(n, ast.Name) and n.id == "name" and isinstance(n.ctx, ast.Store)]
    assert rebound == [], f"`name` rebound at bench.py lines {rebound}"


def test_traffic_lookup_resolves_committed_records():
    """Every record in profiles/traffic.json is found under its own (kernel,
    workload) key whenever its source hash is current."""
    import json
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, rec in recs.items():
        kernel, workload = key.rsplit("/", 1)
        got = bench.measured_traffic(kernel, workload)
        want = rec["bytes_per_launch"] if rec["source_sha256_16"] == bench.source_hash(kernel) else None
        assert got == want, key

