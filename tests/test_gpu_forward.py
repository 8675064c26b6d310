"""mlora_forward (segment build and the layer for one projection in one call)
through the C ABI: its Y and segment workspace against mlora_build_segments
followed by mlora_apply (bit for bit: the same kernels), and its Y against
the CPU oracle (M031 card, sections 02-03), on decode and medium shapes
where the segment build rides in the GEMM launch and on shapes that take
the two calls one after the other."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_support import assert_close, dev_to_f64, ids_dev, make_pool, oracle_adapters, say, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch_cuda()
    import lora_serving_mlora_amd as M
    return M


def _workload(seed, n, din, dout, ranks, n_proj=1, bad=False):
    ids = synth.random_ids(seed, n, sorted(ranks), 0.2)
    A = max(ranks) + 1
    if bad and n >= 4:
        # one id not resident, one past the table, one below -1
        ids[[0, n // 3, n - 1]] = [A, A + 7, -3]
        A += 1
    return synth.custom(f"fwd{seed}", seed, din, dout, ids, ranks, n_proj=n_proj, max_adapters=A,
                        max_rank=max(ranks.values()))


def _bits(t):
    torch = torch_cuda()
    return t.contiguous().view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _both(M, pool, w, proj, variant):
    """Y and seg_ws from forward, and from build_segments + apply, on
    workspaces filled with the same sentinel."""
    torch = torch_cuda()
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits(proj))
    ids = ids_dev(w.row_adapter)
    nb = M.segments_bytes(w.n) // 4
    seg_f = torch.full((nb,), -7, dtype=torch.int32, device="cuda")
    seg_a = torch.full((nb,), -7, dtype=torch.int32, device="cuda")
    Yf, _ = M.forward(pool, proj, Xd, W0d, ids, seg_ws=seg_f, work=M.new_work(pool, w.n), variant=variant)
    M.build_segments(pool, ids, seg_a)
    Ya = M.apply(pool, proj, Xd, W0d, seg_a, work=M.new_work(pool, w.n), variant=variant)
    torch.cuda.synchronize()
    return Yf, seg_f, Ya, seg_a


CASES = [
    # (seed, n, din, dout, ranks, bad ids): decode shapes (segment build inside the GEMM launch)
    (1, 1, 2048, 1000, {0: 16}, False),
    (2, 13, 4096, 136, {0: 16, 1: 3, 2: 64}, True),
    (3, 32, 4096, 4096, {0: 16, 1: 16, 2: 16}, False),
    (4, 48, 2048, 4104, {0: 8, 3: 1, 5: 33}, True),
    (5, 64, 4096, 4096, {i: 16 for i in range(40)}, True),
    # medium batches (65 .. 1024 rows): the segment build in the first
    # workgroup of the ring GEMM launch (direct ranking up to 256 rows, then
    # one radix pass, or two with more than 254 ids)
    (6, 65, 4096, 4096, {0: 16, 1: 3}, True),
    (9, 256, 4096, 1000, {0: 16, 1: 7, 2: 64}, True),
    (10, 300, 4096, 4096, {i: 16 for i in range(256)}, True),
    (11, 700, 2048, 512, {i: (16 if i % 3 else 64) for i in range(40)}, True),
    (12, 1024, 4096, 4096, {0: 16, 1: 8}, True),
    (17, 200, 2048, 1000, {0: 8, 1: 3, 2: 5}, True),
    (18, 520, 4096, 4096, {i: 16 for i in range(60)}, True),
    (19, 128, 1024, 4096, {0: 16, 1: 1}, False),
    # up to 256 rows the segment build's workgroup takes a share of the rows
    # too: 250 rows over 256 workgroups leaves it none, 257 rows takes the
    # other form
    (20, 250, 2048, 1000, {i: 16 for i in range(30)}, True),
    (21, 257, 2048, 1000, {i: 16 for i in range(30)}, True),
    # decode shapes with wider or ragged din (8 to 16 K slices; slices of
    # unequal depth)
    (13, 32, 11008, 4096, {0: 16, 1: 16, 2: 16}, True),
    (14, 64, 8192, 1000, {0: 8, 1: 64, 4: 3}, True),
    (15, 5, 2560, 520, {0: 16}, False),
    (16, 48, 16384, 264, {i: 16 for i in range(12)}, True),
    # two calls: din not a multiple of 128, unaligned dout
    (7, 20, 1000, 520, {0: 16, 1: 5}, True),
    (8, 9, 2048, 12, {0: 4}, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[1]}_k{c[2]}_n{c[3]}")
def test_forward_matches_build_then_apply_and_oracle(M, case):
    seed, n, din, dout, ranks, bad = case
    w = _workload(100 + seed, n, din, dout, ranks, bad=bad)
    pool = make_pool(M, w)
    say(f"forward n={n} din={din} dout={dout}")
    Yf, seg_f, Ya, seg_a = _both(M, pool, w, 0, "auto")
    assert np.array_equal(_bits(seg_f), _bits(seg_a)), "segment workspace differs"
    assert np.array_equal(_bits(Yf), _bits(Ya)), "Y differs from build_segments + apply"
    ref = O.linear(O.widen_bf16(w.x_bits()), O.widen_bf16(w.w0_bits(0)), w.row_adapter, oracle_adapters(w),
                   w.max_adapters, base_batched=True)
    assert_close(dev_to_f64(Yf), ref, f"forward n={n}")
    h = M.segments_header(seg_f)
    seg = O.segments(w.row_adapter, w.max_adapters, w.adapter_ids())
    assert h["n_act"] == seg["n_act"] and h["status"] == seg["status"]


@pytest.mark.parametrize("variant", ["rows", "split", "fused"])
def test_forward_every_variant(M, variant):
    w = _workload(120, 24, 4096, 1000, {0: 16, 1: 7, 2: 64}, bad=True)
    pool = make_pool(M, w)
    say(f"forward variant={variant}")
    Yf, seg_f, Ya, seg_a = _both(M, pool, w, 0, variant)
    assert np.array_equal(_bits(seg_f), _bits(seg_a))
    assert np.array_equal(_bits(Yf), _bits(Ya))


@pytest.mark.parametrize("n", [40, 300])
def test_forward_then_apply_on_other_projections(M, n):
    """The workspace forward builds (in the decode or the medium GEMM launch)
    serves apply on the batch's other projections."""
    w = _workload(130 + n, n, 4096, 264, {0: 5, 1: 12, 3: 2}, n_proj=3)
    pool = make_pool(M, w)
    X = w.x_bits()
    Xd = to_dev_bf16(X)
    say("forward + apply on projections 1, 2")
    _, seg_ws = M.forward(pool, 0, Xd, to_dev_bf16(w.w0_bits(0)), ids_dev(w.row_adapter))
    for p in (1, 2):
        Y = M.apply(pool, p, Xd, to_dev_bf16(w.w0_bits(p)), seg_ws)
        ref = O.linear(O.widen_bf16(X), O.widen_bf16(w.w0_bits(p)), w.row_adapter, oracle_adapters(w, p),
                       w.max_adapters, base_batched=True)
        assert_close(dev_to_f64(Y), ref, f"apply p{p} after forward")


def test_forward_launches(M):
    """Decode and medium shapes: two launches (GEMM with the segment build
    and the shrink, then the finish pass); din not a multiple of 128: the
    segment builder first."""
    torch = torch_cuda()
    w = synth.decode_3_adapters()
    pool = make_pool(M, w)
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    work = M.new_work(pool, w.n)
    Y, seg = M.forward(pool, 0, Xd, W0d, ids_dev(w.row_adapter), work=work)
    torch.cuda.synchronize()
    say("forward launch marks")
    M.timing_arm(8)
    M.forward(pool, 0, Xd, W0d, ids_dev(w.row_adapter), seg_ws=seg, Y=Y, work=work)
    assert [m[0] for m in M.timing_read()] == ["gemm_decode+seg+shrink_rows", "finish_part"]
    w2 = _workload(140, 65, 4096, 512, {0: 16})
    pool2 = make_pool(M, w2)
    M.timing_arm(8)
    M.forward(pool2, 0, to_dev_bf16(w2.x_bits()), to_dev_bf16(w2.w0_bits()), ids_dev(w2.row_adapter))
    assert [m[0] for m in M.timing_read()] == ["gemm_mid+seg+shrink_rows", "finish_part"]
    w3 = _workload(141, 100, 1000, 512, {0: 16})
    pool3 = make_pool(M, w3)
    M.timing_arm(8)
    M.forward(pool3, 0, to_dev_bf16(w3.x_bits()), to_dev_bf16(w3.w0_bits()), ids_dev(w3.row_adapter))
    names = [m[0] for m in M.timing_read()]
    assert names[0] == "seg_build" and len(names) >= 2, names


def test_forward_argument_errors_launch_nothing(M):
    torch = torch_cuda()
    w = _workload(150, 8, 2048, 64, {0: 4})
    pool = make_pool(M, w)
    Xd, W0d = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    ids = ids_dev(w.row_adapter)
    tiny = torch.zeros(256, dtype=torch.uint8, device="cuda")
    seg = torch.full((M.segments_bytes(w.n) // 4,), -7, dtype=torch.int32, device="cuda")
    say("forward argument errors")
    with pytest.raises(M.MloraError):
        M.forward(pool, 0, Xd, W0d, ids, seg_ws=seg, work=tiny, variant="rows")
    with pytest.raises(M.MloraError):
        M.forward(pool, 5, Xd, W0d, ids, seg_ws=seg)
    torch.cuda.synchronize()
    assert (seg == -7).all().item(), "a rejected call wrote the segment workspace"
