"""The layer captured in a HIP graph: every replay (with eager work and
synchronisation between replays) must equal the eager result bitwise."""
import numpy as np
import pytest

import synth
from gpu_support import ids_dev, make_pool, say, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["split", "fused"])
def test_graph_replays_match_eager(variant):
    torch = torch_cuda()
    import lora_serving_mlora_amd as M
    w = synth.decode_fragmented()
    pool = make_pool(M, w)
    X, W0 = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    ids = ids_dev(w.row_adapter)
    seg = torch.empty(M.segments_bytes(w.n) // 4, dtype=torch.int32, device="cuda")
    Y = torch.empty((w.n, w.dout), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(max(M.work_bytes(pool, w.n), 256), dtype=torch.uint8, device="cuda")
    say(f"graph eager {variant}")
    M.build_segments(pool, ids, seg)
    M.apply(pool, 0, X, W0, seg, Y, work, variant)
    eager = Y.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    Y.zero_()
    seg.zero_()
    say(f"graph capture {variant}")
    with torch.cuda.graph(g):
        M.build_segments(pool, ids, seg)
        M.apply(pool, 0, X, W0, seg, Y, work, variant)
    for r in range(3):
        Y.fill_(7.0)                  # eager work between replays
        seg.zero_()
        torch.cuda.synchronize()
        say(f"graph replay {r} {variant}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"


@pytest.mark.parametrize("name", ["decode_3", "decode_frag", "layer_stack"])
def test_graph_replays_of_forward_match_eager(name):
    """The one-call step (segment build inside the GEMM launch at these
    sizes) as the bench times it: captured, replayed three times with eager
    work in between, each replay equal to the eager Y and workspace bitwise."""
    torch = torch_cuda()
    import lora_serving_mlora_amd as M
    w = synth.NAMED[name]()
    pool = make_pool(M, w)
    X, W0 = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    ids = ids_dev(w.row_adapter)
    # the builder leaves the unused tails of its tables unwritten: the same
    # sentinel under every run
    seg = torch.full((M.segments_bytes(w.n) // 4,), -7, dtype=torch.int32, device="cuda")
    Y = torch.empty((w.n, w.dout), dtype=torch.bfloat16, device="cuda")
    work = M.new_work(pool, w.n)
    say(f"graph eager forward {name}")
    M.forward(pool, 0, X, W0, ids, seg_ws=seg, Y=Y, work=work)
    eager, eager_seg = Y.clone(), seg.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say(f"graph capture forward {name}")
    with torch.cuda.graph(g):
        M.forward(pool, 0, X, W0, ids, seg_ws=seg, Y=Y, work=work)
    for r in range(3):
        Y.fill_(7.0)
        seg.fill_(-7)
        torch.cuda.synchronize()
        say(f"graph replay {r} forward {name}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
        assert torch.equal(seg, eager_seg), f"replay {r}: segment workspace differs"
