"""The C-ABI library: it loads on a machine without a GPU and exports every
entry point include/mlora.h declares (no compute calls here)."""
import ctypes
import os
import re

import pytest

import lora_serving_mlora_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlora.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mlora_[a-z0-9_]+)\s*\(", src)) - {"mlora_status"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("mlora_pool_load", "mlora_build_segments", "mlora_apply", "mlora_shrink", "mlora_expand",
                 "mlora_fused", "mlora_base_gemm", "mlora_pool_create", "mlora_pool_unload"):
        assert must in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("libmlora.so not built")
    L = ctypes.CDLL(M.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(M.EXPORTS)


def test_host_only_calls():
    """Calls that touch no device: sizes, strings, argument errors."""
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("libmlora.so not built")
    L = M.lib()
    assert L.mlora_version().startswith(b"mlora")
    assert L.mlora_status_string(M.ENOSPC) == b"no free pages"
    # meta: 256-aligned regions rank, scale, two page tables
    A, P, R = 100, 64, 16
    pt = A * P * R * 4
    al = lambda x: (x + 255) // 256 * 256
    assert L.mlora_pool_meta_bytes(A, P, R) == al(4 * A) * 2 + al(pt) * 2
    assert L.mlora_pool_meta_bytes(0, 1, 1) == 0
    n = 4096
    items0 = (16 + 4 * n + 2) & ~1
    max_items = n + (n + 3) // 4 + 1
    assert L.mlora_segments_bytes(n) == al((items0 + 2 * max_items + n + 2 * n) * 4)
    assert L.mlora_shrink_max_chunks(4096) == 8 and L.mlora_shrink_max_chunks(4) == 1
    assert L.mlora_pool_create(None, None, None) == M.EINVAL
    assert b"NULL" in L.mlora_last_error()
    assert L.mlora_base_gemm(None, None, None, 0, 4, 4, None) == M.OK     # n = 0 is a no-op
    assert L.mlora_base_gemm(None, None, None, 1, 0, 4, None) == M.EINVAL
    assert L.mlora_hbm_copy(None, None, 16, None) == M.EINVAL
    assert L.mlora_hbm_read_lds(None, 1024, None, None) == M.EINVAL
    assert L.mlora_hbm_read_lds(ctypes.c_void_p(256), 1000, ctypes.c_void_p(256), None) == M.EINVAL  # not KiB
    assert L.mlora_hbm_read_lds(ctypes.c_void_p(256), 1 << 31, ctypes.c_void_p(256), None) == M.EINVAL
    # the layer's entry points reject a NULL pool before touching the device
    assert L.mlora_apply(None, 0, None, None, None, None, 1, None, 0, 0, None) == M.EINVAL
    assert L.mlora_forward(None, 0, None, None, None, None, None, 1, None, 0, 0, None) == M.EINVAL
    assert b"pool" in L.mlora_last_error()
    # launch timing: argument checks and an empty read touch no device
    assert L.mlora_timing_arm(0) == M.EINVAL
    assert L.mlora_timing_arm(2049) == M.EINVAL
    n_marked = ctypes.c_int32(-1)
    ms = (ctypes.c_float * 4)()
    assert L.mlora_timing_read(ms, 4, ctypes.byref(n_marked)) == M.OK and n_marked.value == 0
    assert L.mlora_timing_name(0) is None
