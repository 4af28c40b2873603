"""The C ABI on the CPU: the library loads, exports every entry point that
include/dflash.h declares, and host-side validation rejects bad calls with
the documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

from block_diffusion_speculative_amd import _lib
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd.engine import cdims

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dflash.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdflash.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_abi_version(lib):
    assert lib.dflash_abi_version() == 1
    assert lib.dflash_status_str(-4) == b"workspace too small"
    assert lib.dflash_status_str(-7) == b"unsupported"


def test_sizes(lib):
    d = cdims(C.QWEN3_8B_DRAFT)
    assert lib.dflash_packed_bytes(0, 151936, 4096) == 151936 * 4096 * 2
    assert lib.dflash_packed_bytes(1, 17, 20) == 2 * 2 * 1024     # padded to 32 rows x 32 cols fp32
    assert lib.dflash_packed_bytes(5, 16, 16) == 0
    assert lib.dflash_kv_bytes(ctypes.byref(d), 2080, 1) == 5 * 8 * 2080 * 128 * 2
    ws = lib.dflash_workspace_bytes(ctypes.byref(d), 1, 17)
    assert ws > (1 << 20)
    assert lib.dflash_workspace_bytes(ctypes.byref(d), 0, 17) == 0
    assert lib.dflash_workspace_bytes(ctypes.byref(d), 65, 17) == 0


def test_views_inside_workspace(lib):
    d = cdims(C.QWEN3_8B_DRAFT)
    total = lib.dflash_workspace_bytes(ctypes.byref(d), 4, 68)
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    for what, count, layer in [(0, 68, 0), (1, 4, -1), (1, 4, 4), (2, 4, 0), (3, 4, 4)]:
        assert lib.dflash_workspace_view(ctypes.byref(d), what, count, layer, ctypes.byref(off), ctypes.byref(nb)) == 0
        assert off.value >= (1 << 20) and off.value + nb.value <= total
    assert lib.dflash_workspace_view(ctypes.byref(d), 1, 4, 5, ctypes.byref(off), ctypes.byref(nb)) == _lib.DFLASH_ERR_SHAPE
    for bad in (4, 9):
        assert lib.dflash_workspace_view(ctypes.byref(d), bad, 4, 0, ctypes.byref(off), ctypes.byref(nb)) == _lib.DFLASH_ERR_SHAPE


def _bad_dims(**kw):
    base = C.QWEN3_8B_DRAFT.__dict__.copy()
    d = cdims(C.QWEN3_8B_DRAFT)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, _lib.DFLASH_ERR_DTYPE),
    ("hidden", 100, _lib.DFLASH_ERR_SHAPE),
    ("hidden", 96, _lib.DFLASH_ERR_UNSUPPORTED),
    ("hidden", 8256, _lib.DFLASH_ERR_UNSUPPORTED),
    ("head_dim", 80, _lib.DFLASH_ERR_SHAPE),
    ("head_dim", 96, _lib.DFLASH_ERR_UNSUPPORTED),
    ("n_q_heads", 30, _lib.DFLASH_ERR_SHAPE),
    ("n_q_heads", 136, _lib.DFLASH_ERR_UNSUPPORTED),
    ("n_layers", 0, _lib.DFLASH_ERR_SHAPE),
    ("n_layers", 17, _lib.DFLASH_ERR_UNSUPPORTED),
    ("block_size", 17, _lib.DFLASH_ERR_SHAPE),
    ("block_size", 0, _lib.DFLASH_ERR_SHAPE),
    ("mask_id", 151936, _lib.DFLASH_ERR_SHAPE),
    ("intermediate", 100, _lib.DFLASH_ERR_SHAPE),
])
def test_bad_dims_rejected(lib, field, value, code):
    d = _bad_dims(**{field: value})
    r = lib.dflash_verify_accept(ctypes.byref(d), 16, 16, 16, 1, 16, 16, 16, 16, 1 << 30, None)
    assert r == code
    assert lib.dflash_last_error()


def test_null_and_alignment_rejected(lib):
    d = cdims(C.QWEN3_8B_DRAFT)
    r = lib.dflash_verify_accept(ctypes.byref(d), None, 16, 16, 1, 16, 16, 16, 16, 1 << 30, None)
    assert r == _lib.DFLASH_ERR_NULL
    r = lib.dflash_verify_accept(ctypes.byref(d), 24, 16, 16, 1, 16, 16, 16, 16, 1 << 30, None)
    assert r == _lib.DFLASH_ERR_ALIGN
    r = lib.dflash_verify_accept(ctypes.byref(d), 16, 16, 16, 0, 16, 16, 16, 16, 1 << 30, None)
    assert r == _lib.DFLASH_ERR_SHAPE
    r = lib.dflash_verify_accept(ctypes.byref(d), 16, 16, 16, 1, 16, 16, 16, 16, 1024, None)
    assert r == _lib.DFLASH_ERR_WORKSPACE
    r = lib.dflash_pack_matrix(0, 16, 16, 20, 16, None)   # 40-byte row pitch
    assert r == _lib.DFLASH_ERR_ALIGN
    r = lib.dflash_pack_matrix(3, 16, 16, 32, 16, None)
    assert r == _lib.DFLASH_ERR_DTYPE


def test_kv_and_inject_validation(lib):
    d = cdims(C.QWEN3_8B_DRAFT)
    layers = (_lib.Layer * 5)()
    for i in range(5):
        layers[i] = _lib.Layer(16, 16, 16, 16, 16, 16)
    w = _lib.Weights(16, 16, 16, 16, 16, ctypes.cast(layers, ctypes.POINTER(_lib.Layer)))
    kv = _lib.KV(16, 16, 16, 16, 2080, 1)
    big = 1 << 34
    # capacity not a multiple of 32
    bad = _lib.KV(16, 16, 16, 16, 2081, 1)
    assert lib.dflash_inject_kv(ctypes.byref(d), ctypes.byref(w), ctypes.byref(bad), 16, 16, 1, 9, 16, big, None) == _lib.DFLASH_ERR_SHAPE
    # batch above max_batch
    assert lib.dflash_inject_kv(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, 16, 2, 9, 16, big, None) == _lib.DFLASH_ERR_SHAPE
    # missing cu_new
    assert lib.dflash_inject_kv(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, None, 1, 9, 16, big, None) == _lib.DFLASH_ERR_NULL
    # workspace too small
    assert lib.dflash_inject_kv(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, 16, 1, 9, 16, 4096, None) == _lib.DFLASH_ERR_WORKSPACE
    # missing layer weight
    layers[2] = _lib.Layer(16, None, 16, 16, 16, 16)
    assert lib.dflash_draft_forward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, 1, 16, 16, big, None) == _lib.DFLASH_ERR_NULL
    # zero rows: nothing to do
    layers[2] = _lib.Layer(16, 16, 16, 16, 16, 16)
    assert lib.dflash_inject_kv(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), None, 16, 1, 0, 16, big, None) == 0
