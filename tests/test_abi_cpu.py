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


def _drafter_structs(n_layers=5, capacity=2080, max_batch=1):
    layers = (_lib.Layer * n_layers)()
    for i in range(n_layers):
        layers[i] = _lib.Layer(16, 16, 16, 16, 16, 16)
    w = _lib.Weights(16, 16, 16, 16, 16, ctypes.cast(layers, ctypes.POINTER(_lib.Layer)))
    kv = _lib.KV(16, 16, 16, 16, capacity, max_batch)
    return layers, w, kv


def test_target_pass_validation(lib):
    """dflash_target_forward rejects bad row counts, feature layers, batches
    and workspaces before any HIP call; dflash_target_workspace_bytes is 0
    outside its ranges."""
    td = cdims(C.QWEN3_8B_TARGET)
    layers, w, kv = _drafter_structs(36, 4096, 2)
    big = 1 << 40
    fl = (ctypes.c_int32 * 3)(5, 11, 17)
    call = lambda batch, rows, feats, n, ws=big: lib.dflash_target_forward(
        ctypes.byref(td), ctypes.byref(w), ctypes.byref(kv), 16, None, batch, rows, feats, n, 16, 16, 16, ws, None)
    assert lib.dflash_target_workspace_bytes(ctypes.byref(td), 1, 17) > (1 << 20)
    assert lib.dflash_target_workspace_bytes(ctypes.byref(td), 1, 33) == 0
    assert lib.dflash_target_workspace_bytes(ctypes.byref(td), 0, 17) == 0
    assert call(1, 0, fl, 3) == _lib.DFLASH_ERR_SHAPE
    assert call(1, 33, fl, 3) == _lib.DFLASH_ERR_SHAPE
    assert call(3, 17, fl, 3) == _lib.DFLASH_ERR_SHAPE          # above kv->max_batch
    assert call(1, 17, fl, 17) == _lib.DFLASH_ERR_SHAPE         # n_feat above 16
    assert call(1, 17, None, 3) == _lib.DFLASH_ERR_NULL
    dup = (ctypes.c_int32 * 3)(5, 11, 5)
    assert call(1, 17, dup, 3) == _lib.DFLASH_ERR_SHAPE
    out = (ctypes.c_int32 * 3)(5, 11, 36)
    assert call(1, 17, out, 3) == _lib.DFLASH_ERR_SHAPE
    assert call(1, 17, fl, 3, ws=4096) == _lib.DFLASH_ERR_WORKSPACE
    layers[7] = _lib.Layer(16, 16, None, 16, 16, 16)
    assert call(1, 17, fl, 3) == _lib.DFLASH_ERR_NULL
    assert lib.dflash_kv_commit(ctypes.byref(td), ctypes.byref(kv), 16, 3, 17, None) == _lib.DFLASH_ERR_SHAPE
    assert lib.dflash_kv_commit(ctypes.byref(td), ctypes.byref(kv), 16, 1, -1, None) == _lib.DFLASH_ERR_SHAPE
    assert lib.dflash_kv_commit(ctypes.byref(td), ctypes.byref(kv), None, 1, 17, None) == _lib.DFLASH_ERR_NULL


def test_tree_validation(lib):
    """Draft trees: topk in [1, 8], nodes in [1, 31] and within the
    continuations of the block, walk sizes in [1, 32], batches in range."""
    d = cdims(C.QWEN3_8B_DRAFT)
    layers, w, kv = _drafter_structs()
    big = 1 << 40
    tree = lambda batch, topk, nodes: lib.dflash_draft_tree(
        ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, batch, topk, nodes, 16, 16, 16, 16, big, None)
    assert tree(1, 0, 8) == _lib.DFLASH_ERR_SHAPE
    assert tree(1, 9, 8) == _lib.DFLASH_ERR_SHAPE
    assert tree(1, 4, 0) == _lib.DFLASH_ERR_SHAPE
    assert tree(1, 4, 32) == _lib.DFLASH_ERR_SHAPE
    assert tree(0, 4, 8) == _lib.DFLASH_ERR_SHAPE
    assert tree(65, 4, 8) == _lib.DFLASH_ERR_SHAPE
    d4 = cdims(C.QWEN3_8B_DRAFT.with_block(4))
    # K = 1 over 4 slots: 4 continuations, so 5 nodes cannot exist
    assert lib.dflash_draft_tree(ctypes.byref(d4), ctypes.byref(w), ctypes.byref(kv), 16, 1, 1, 5, 16, 16, 16,
                                 16, big, None) == _lib.DFLASH_ERR_SHAPE
    acc = lambda batch, n: lib.dflash_tree_accept(ctypes.byref(d), 16, 16, 16, 16, batch, n, 16, 16, 16, 16, 16,
                                                  big, None)
    assert acc(1, 0) == _lib.DFLASH_ERR_SHAPE
    assert acc(1, 33) == _lib.DFLASH_ERR_SHAPE
    assert acc(65, 8) == _lib.DFLASH_ERR_SHAPE
    assert lib.dflash_tree_accept(ctypes.byref(d), 16, 16, 16, 16, 1, 8, 16, 16, 16, None, 16, big,
                                  None) == _lib.DFLASH_ERR_NULL
    td = cdims(C.QWEN3_8B_TARGET)
    _, _, tkv = _drafter_structs(36, 4096, 2)
    path = lambda batch, n: lib.dflash_kv_commit_path(ctypes.byref(td), ctypes.byref(tkv), 16, 16, batch, n, None)
    assert path(1, 33) == _lib.DFLASH_ERR_SHAPE
    assert path(3, 8) == _lib.DFLASH_ERR_SHAPE
    assert path(1, 0) == _lib.DFLASH_ERR_SHAPE


def test_anchor_and_sampling_validation(lib):
    """Anchored drafting takes 1-64 blocks; sampling needs a positive finite
    temperature and its uniforms."""
    d = cdims(C.QWEN3_8B_DRAFT)
    layers, w, kv = _drafter_structs()
    big = 1 << 40
    anchors = lambda nb, pos=16: lib.dflash_draft_anchors(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16,
                                                        pos, 16, nb, 16, 16, big, None)
    assert anchors(0) == _lib.DFLASH_ERR_SHAPE
    assert anchors(65) == _lib.DFLASH_ERR_SHAPE
    assert anchors(4, None) == _lib.DFLASH_ERR_NULL
    sample = lambda t, u=16: lib.dflash_draft_sample(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 16, 1, t,
                                                     u, 16, 16, 16, big, None)
    for t in (0.0, -1.0, float("inf"), float("nan")):
        assert sample(t) == _lib.DFLASH_ERR_SHAPE, t
    assert sample(1.0, None) == _lib.DFLASH_ERR_NULL
    ver = lambda t, batch=1, ua=16: lib.dflash_verify_sample(ctypes.byref(d), 16, 16, 16, 16, batch, t, ua, 16, 16,
                                                             16, 16, 16, big, None)
    assert ver(0.0) == _lib.DFLASH_ERR_SHAPE
    assert ver(1.0, batch=0) == _lib.DFLASH_ERR_SHAPE
    assert ver(1.0, ua=None) == _lib.DFLASH_ERR_NULL
    assert lib.dflash_verify_sample(ctypes.byref(d), 16, 16, 16, 16, 1, 1.0, 16, 16, 16, 16, 16, 16, 4096,
                                    None) == _lib.DFLASH_ERR_WORKSPACE
