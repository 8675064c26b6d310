"""mlora_forward_static, the entry point for callers that cannot allocate
device memory: its scratch is the library's static device array, and it
must give exactly what mlora_forward gives with a caller-provided work
buffer (same kernels, same launch plan), on calls in a row of different
sizes (the second smaller, over the contents the first left), and the
oracle's result within the parity bar."""
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


def _check_against_forward(M, torch, pool, w, rows, what):
    X, W0 = w.x_bits()[rows], w.w0_bits()
    ids = w.row_adapter[rows]
    Xd, Wd, idd = to_dev_bf16(X), to_dev_bf16(W0), ids_dev(ids)
    # both workspaces start from the same contents: a small batch leaves
    # parts of the workspace (unused item and tile slots) unwritten
    segs = torch.full((M.segments_bytes(len(rows)) // 4,), -7, dtype=torch.int32, device="cuda")
    segf = segs.clone()
    say(f"forward_static {what} rows={len(rows)}")
    Ys, _ = M.forward_static(pool, 0, Xd, Wd, idd, seg_ws=segs)
    torch.cuda.synchronize()
    say(f"forward (work buffer) {what} rows={len(rows)}")
    Yf, _ = M.forward(pool, 0, Xd, Wd, idd, seg_ws=segf, work=M.new_work(pool, len(rows)))
    torch.cuda.synchronize()
    assert torch.equal(Ys.view(torch.int16), Yf.view(torch.int16)), f"{what}: Y differs from mlora_forward"
    assert torch.equal(segs, segf), f"{what}: segment workspace differs from mlora_forward"
    ref = O.linear(O.widen_bf16(X), O.widen_bf16(W0), ids, oracle_adapters(w), w.max_adapters, base_batched=True)
    assert_close(dev_to_f64(Ys), ref, f"forward_static {what}")


def test_static_scratch_matches_forward_on_calls_in_a_row(M):
    """Two calls in a row, the second with a smaller batch: the 256-row
    fragmented decode (its per-row plan takes 16.1 MiB of the scratch), then 13 rows of
    the 32-row decode; each compared with mlora_forward bit for bit and with
    the oracle."""
    torch = torch_cuda()
    wf = synth.decode_fragmented()
    pool_f = make_pool(M, wf)
    _check_against_forward(M, torch, pool_f, wf, np.arange(wf.n), "fragmented decode")
    w3 = synth.decode_3_adapters()
    pool_3 = make_pool(M, w3)
    _check_against_forward(M, torch, pool_3, w3, np.arange(13), "decode, first 13 rows")
    # and the full decode batch once more, over what the smaller call left
    _check_against_forward(M, torch, pool_3, w3, np.arange(w3.n), "decode, 32 rows")


def test_static_scratch_rejects_a_batch_beyond_its_size(M):
    """A batch whose launch plan needs more than the static scratch (here
    the split plan's low-rank operands for a pool of 64 adapter slots of
    rank up to 64 at dout = 11008, about 90 MB) is refused with EINVAL
    before anything is launched (the segment workspace stays as it was)."""
    torch = torch_cuda()
    n, din, dout = 4096, 256, 11008
    ids = np.zeros(n, dtype=np.int32)
    w = synth.custom("noalloc_big", 77, din, dout, ids, {0: 64}, max_adapters=64, max_rank=64)
    pool = make_pool(M, w)
    assert M.work_bytes(pool, n) > M.STATIC_SCRATCH_BYTES
    Xd, Wd = to_dev_bf16(w.x_bits()), to_dev_bf16(w.w0_bits())
    seg = torch.full((M.segments_bytes(n) // 4,), -7, dtype=torch.int32, device="cuda")
    say("forward_static beyond the scratch")
    with pytest.raises(M.MloraError) as e:
        M.forward_static(pool, 0, Xd, Wd, ids_dev(ids), seg_ws=seg)
    assert e.value.status == M.EINVAL
    torch.cuda.synchronize()
    assert (seg == -7).all().item()


def test_static_scratch_serves_the_prefill_batch(M):
    """The 4096-row prefill (split plan with the epilogue operands, 17 MB)
    fits the scratch: bit for bit what mlora_forward gives, and the oracle's
    result."""
    torch = torch_cuda()
    w = synth.prefill_hetero()
    pool = make_pool(M, w)
    _check_against_forward(M, torch, pool, w, np.arange(w.n), "prefill")
