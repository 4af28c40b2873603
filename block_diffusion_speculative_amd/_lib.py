"""ctypes binding of libdflash.so: the same names as include/dflash.h.

Argument marshalling only.  Loading fails loudly when the library has not
been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_BF16 = 0
DFLASH_F32 = 1
DFLASH_OK = 0
DFLASH_ERR_NULL = -1
DFLASH_ERR_SHAPE = -2
DFLASH_ERR_DTYPE = -3
DFLASH_ERR_WORKSPACE = -4
DFLASH_ERR_ALIGN = -5
DFLASH_ERR_HIP = -6
DFLASH_ERR_UNSUPPORTED = -7
DFLASH_STATUS_CAPACITY = 1
DFLASH_STATUS_TOKEN = 2
DFLASH_STATUS_ANCHOR = 4
DFLASH_STATUS_TREE = 8
VIEW_FUSED, VIEW_HIDDEN, VIEW_MID, VIEW_ATTN = range(4)

EXPORTED = [
    "dflash_packed_bytes", "dflash_pack_matrix", "dflash_pack_qkv", "dflash_pack_gate_up",
    "dflash_pack_lm_head",
    "dflash_kv_bytes", "dflash_kv_import", "dflash_kv_export",
    "dflash_workspace_bytes", "dflash_workspace_init", "dflash_workspace_view",
    "dflash_inject_kv", "dflash_draft_forward", "dflash_draft_anchors", "dflash_draft_sample",
    "dflash_target_workspace_bytes", "dflash_target_forward", "dflash_kv_commit",
    "dflash_draft_tree", "dflash_tree_accept", "dflash_kv_commit_path",
    "dflash_verify_sample", "dflash_verify_accept", "dflash_verify_accept_noalloc",
    "dflash_status_str", "dflash_last_error", "dflash_abi_version", "dflash_build_id",
]


class Dims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("n_layers", c_int32), ("intermediate", c_int32),
                ("vocab", c_int32), ("n_feat_layers", c_int32), ("block_size", c_int32),
                ("mask_id", c_int32), ("rope_theta", c_float), ("rms_eps", c_float),
                ("dtype", c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("w_qkv", c_void_p), ("w_o", c_void_p),
                ("mlp_norm", c_void_p), ("w_gate_up", c_void_p), ("w_down", c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("w_fc", c_void_p), ("fc_norm", c_void_p), ("embed", c_void_p),
                ("final_norm", c_void_p), ("lm_head", c_void_p), ("layers", POINTER(Layer))]


class KV(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("ctx_len", c_void_p), ("status", c_void_p),
                ("capacity", c_int32), ("max_batch", c_int32)]


class DflashError(RuntimeError):
    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libdflash.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_diffusion_speculative_amd.csrc.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "dflash_packed_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "dflash_pack_matrix": (c_int32, [c_int32, P, c_int32, c_int32, P, P]),
        "dflash_pack_qkv": (c_int32, [POINTER(Dims), P, P, P, P, P]),
        "dflash_pack_gate_up": (c_int32, [POINTER(Dims), P, P, P, P]),
        "dflash_pack_lm_head": (c_int32, [c_int32, P, c_int32, c_int32, P, P]),
        "dflash_kv_bytes": (c_size_t, [POINTER(Dims), c_int32, c_int32]),
        "dflash_kv_import": (c_int32, [POINTER(Dims), POINTER(KV), P, P, P]),
        "dflash_kv_export": (c_int32, [POINTER(Dims), POINTER(KV), P, P, P]),
        "dflash_workspace_bytes": (c_size_t, [POINTER(Dims), c_int32, c_int32]),
        "dflash_workspace_init": (c_int32, [P, c_size_t, P]),
        "dflash_workspace_view": (c_int32, [POINTER(Dims), c_int32, c_int32, c_int32,
                                            POINTER(c_size_t), POINTER(c_size_t)]),
        "dflash_inject_kv": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P, P,
                                       c_int32, c_int32, P, c_size_t, P]),
        "dflash_draft_forward": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P,
                                           c_int32, P, P, c_size_t, P]),
        "dflash_draft_anchors": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P, P, P,
                                           c_int32, P, P, c_size_t, P]),
        "dflash_target_workspace_bytes": (c_size_t, [POINTER(Dims), c_int32, c_int32]),
        "dflash_target_forward": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P, P, c_int32,
                                            c_int32, P, c_int32, P, P, P, c_size_t, P]),
        "dflash_draft_tree": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P, c_int32, c_int32,
                                        c_int32, P, P, P, P, c_size_t, P]),
        "dflash_tree_accept": (c_int32, [POINTER(Dims), P, P, P, P, c_int32, c_int32, P, P, P, P, P,
                                         c_size_t, P]),
        "dflash_kv_commit_path": (c_int32, [POINTER(Dims), POINTER(KV), P, P, c_int32, c_int32, P]),
        "dflash_kv_commit": (c_int32, [POINTER(Dims), POINTER(KV), P, c_int32, c_int32, P]),
        "dflash_draft_sample": (c_int32, [POINTER(Dims), POINTER(Weights), POINTER(KV), P, c_int32,
                                          c_float, P, P, P, P, c_size_t, P]),
        "dflash_verify_sample": (c_int32, [POINTER(Dims), P, P, P, P, c_int32, c_float, P, P, P, P, P,
                                           P, c_size_t, P]),
        "dflash_verify_accept": (c_int32, [POINTER(Dims), P, P, P, c_int32, P, P, P, P,
                                           c_size_t, P]),
        "dflash_verify_accept_noalloc": (c_int32, [POINTER(Dims), P, P, P, c_int32, P, P, P, P]),
        "dflash_status_str": (c_char_p, [c_int32]),
        "dflash_last_error": (c_char_p, []),
        "dflash_abi_version": (c_int32, []),
        "dflash_build_id": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def build_id() -> str:
    """Digest of the sources the loaded library was built from."""
    return load().dflash_build_id().decode()


def is_fresh() -> bool:
    """Whether the loaded library was built from the sources now in the tree."""
    from .csrc.build import source_digest
    return build_id() == source_digest()


def file_is_fresh(path: str = LIB_PATH) -> bool:
    """The same question answered from the library file's bytes (the digest
    is compiled in as a string), without loading it: usable before the GPU
    runtime is initialised."""
    from .csrc.build import source_digest
    with open(path, "rb") as fh:
        return source_digest().encode() in fh.read()


def last_error() -> str:
    return load().dflash_last_error().decode()


def check(name: str, code: int) -> None:
    if code != DFLASH_OK:
        raise DflashError(name, code, last_error())


def call(name: str, *args) -> int:
    """Call an entry point that returns a status code; raise on failure."""
    code = getattr(load(), name)(*args)
    check(name, code)
    return code
