"""The C-ABI library without a GPU: it loads, exports every function include/l3.h
declares, and rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "l3.h")

l3 = pytest.importorskip("static_token_routed_amd", reason="libl3.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z][\w \*]*?\b(l3_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared()
    for must in ("l3_plan", "l3_forward", "l3_prefetch", "l3_route", "l3_status",
                 "l3_workspace_size", "l3_forward_staged"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(l3.LIB_PATH)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared()) == set(l3.EXPORTS)


def test_strerror_texts():
    for c in range(-7, 1):
        assert l3.l3_strerror(c)
    assert "unknown" in l3.l3_strerror(-99)


def _plan(off, v, k, dims=(64, 64, 64, 64), dtype="bf16", eps=1e-5):
    return l3.l3_plan(np.asarray(off, np.int64), len(off) - 1, v, k, *dims, dtype, eps)


@pytest.mark.parametrize("off,v,k,code", [
    ([0, 2, 2, 5], 5, 4, l3.L3_ERR_BAD_OFFSETS),    # d_t = 0
    ([0, 2, 7, 9], 9, 4, l3.L3_ERR_BAD_OFFSETS),    # d_t > k
    ([1, 2, 3, 5], 5, 4, l3.L3_ERR_BAD_OFFSETS),    # off[0] != 0
    ([0, 2, 3, 5], 6, 4, l3.L3_ERR_BAD_OFFSETS),    # off[vocab] != v
    ([0, 2, 3, 5], 5, 0, l3.L3_ERR_INVALID_ARG),    # k < 1
])
def test_plan_rejects_bad_offsets(off, v, k, code):
    with pytest.raises(l3.L3Error) as e:
        _plan(off, v, k)
    assert e.value.code == code


@pytest.mark.parametrize("dims,dtype,code", [
    ((100, 64, 64, 64), "bf16", l3.L3_ERR_UNSUPPORTED),   # d_in not a multiple of 64
    ((64, 96, 64, 64), "bf16", l3.L3_ERR_UNSUPPORTED),    # d_emb not a supported width
    ((8192, 64, 64, 64), "bf16", l3.L3_ERR_UNSUPPORTED),  # d_in above 4096
    ((512, 1024, 64, 64), "bf16", l3.L3_ERR_UNSUPPORTED),  # d_emb 1024 only with d_in = d_emb (tied)
    ((2048, 1536, 64, 64), "bf16", l3.L3_ERR_UNSUPPORTED), # d_emb not a supported width
    ((64, 64, 64, -1), "bf16", l3.L3_ERR_INVALID_ARG),
])
def test_plan_rejects_bad_dims(dims, dtype, code):
    with pytest.raises(l3.L3Error) as e:
        _plan([0, 2, 3, 5], 5, 4, dims, dtype)
    assert e.value.code == code


def test_null_and_size_checks():
    assert l3._lib.l3_plan(None, 3, 5, 4, None, None) == l3.L3_ERR_INVALID_ARG
    assert l3._lib.l3_forward(None, None, None, 1, *([None] * 8), 0, None) == l3.L3_ERR_INVALID_ARG
    assert l3._lib.l3_workspace_size(None, 10) == 0
    assert l3._lib.l3_plan_destroy(None) == l3.L3_OK
    assert l3._lib.l3_staging_destroy(None) == l3.L3_OK
    assert l3._lib.l3_gemm_bf16(None, None, None, 1, 64, 64, None, 0, None) == l3.L3_ERR_INVALID_ARG


def test_gemm_shape_and_alignment_checks():
    # rejected on the host: the pointers are never dereferenced
    g = l3._lib.l3_gemm_bf16
    a, b, c = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    w = ctypes.c_void_p(0x4000)
    big = 1 << 30
    assert g(a, b, c, 64, 64, 96, w, big, None) == l3.L3_ERR_UNSUPPORTED   # K not a multiple of 64
    assert g(a, b, c, 64, 96, 64, w, big, None) == l3.L3_ERR_UNSUPPORTED   # N not a multiple of 64
    assert g(ctypes.c_void_p(0x1008), b, c, 64, 64, 64, w, big, None) == l3.L3_ERR_INVALID_ARG
    assert g(a, b, ctypes.c_void_p(0x3002), 64, 64, 64, w, big, None) == l3.L3_ERR_INVALID_ARG
    assert g(a, b, c, 64, 64, 64, ctypes.c_void_p(0x4004), big, None) == l3.L3_ERR_INVALID_ARG
    # small M needs the split-K workspace: S = ceil(K / 256) fp32 slabs of M x N
    need = l3.l3_gemm_workspace_size(64, 8192, 2048)
    assert need == 8 * 64 * 8192 * 4
    assert l3.l3_gemm_workspace_size(1, 64, 64) == 64 * 4
    assert l3.l3_gemm_workspace_size(513, 1024, 4096) == 0   # large M: no workspace
    assert g(a, b, c, 64, 8192, 2048, None, 0, None) == l3.L3_ERR_CAPACITY
    assert g(a, b, c, 64, 8192, 2048, w, need - 1, None) == l3.L3_ERR_CAPACITY


@pytest.mark.parametrize("dims,dtype,max_d", [
    ((2048, 512, 2048, 2048), "bf16", 512),   # the paper's widths at the k = 512 cap
    ((4096, 512, 4096, 4096), "bf16", 512),
    ((1024, 256, 1024, 1024), "bf16", 128),
    ((192, 64, 128, 64), "bf16", 90),
    ((100, 37, 72, 52), "f32", 96),
])
def test_workspace_size_covers_every_smaller_batch(dims, dtype, max_d):
    """A workspace sized for n_max serves every batch of 1 .. n_max tokens.  Small bf16
    batches carry split-row partials whose size grows with n * max_d until they switch
    off, so the per-token need is largest just below that point: the size function
    must be non-decreasing in n across it."""
    size = lambda n: l3.l3_workspace_size_dims(*dims, dtype, max_d, n)
    sizes = np.array([size(n) for n in range(0, 1300)])
    assert np.all(sizes[1:] > 0)
    assert np.all(np.diff(sizes) >= 0), int(np.argmax(np.diff(sizes) < 0))
    for n_max in (512, 1024, 4096):
        assert size(n_max) >= sizes[1:min(n_max, 1299) + 1].max()
    if dtype == "bf16" and dims[0] == 2048:
        # the split-row partials: 256 tokens x 128 chunks of 4 rows x d_emb fp32 alone
        assert size(256) >= 256 * 128 * 512 * 4
        assert size(512) >= size(256)


def test_workspace_size_dims_rejects():
    assert l3.l3_workspace_size_dims(100, 64, 64, 64, "bf16", 8, 10) == 0   # unsupported dims
    assert l3.l3_workspace_size_dims(64, 64, 64, 64, "bf16", 0, 10) == 0    # max_d < 1
    assert l3.l3_workspace_size_dims(64, 64, 64, 64, "bf16", 8, -1) == 0
