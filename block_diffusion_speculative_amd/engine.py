"""Device-side state for one drafter: packed weights, KV cache and workspace
in HBM (allocated through PyTorch), and thin calls into libdflash.so.

Every step of the path runs in the library's HIP kernels; this module only
allocates memory, uploads inputs and marshals pointers.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from .configs import Dims, kv_capacity
from .inputs import Weights


def cdims(d: Dims) -> _lib.Dims:
    return _lib.Dims(d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.n_layers,
                     d.intermediate, d.vocab, d.n_feat_layers, d.block_size, d.mask_id,
                     float(d.rope_theta), float(d.rms_eps),
                     _lib.DFLASH_BF16 if d.dtype == "bf16" else _lib.DFLASH_F32)


def torch_dtype(d: Dims) -> torch.dtype:
    return torch.bfloat16 if d.dtype == "bf16" else torch.float32


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def upload(arr, dtype: torch.dtype, device, chunk_rows: int = 1 << 14) -> torch.Tensor:
    """Host float32 (storage-representable values) -> device tensor of dtype
    (a tensor already on the device is converted in place of a copy)."""
    if isinstance(arr, torch.Tensor):
        return arr.to(device=device, dtype=dtype).contiguous()
    arr = np.ascontiguousarray(arr)
    out = torch.empty(arr.shape, dtype=dtype, device=device)
    if arr.ndim == 1:
        out.copy_(torch.from_numpy(arr))
        return out
    for r0 in range(0, arr.shape[0], chunk_rows):
        out[r0:r0 + chunk_rows].copy_(torch.from_numpy(arr[r0:r0 + chunk_rows]))
    return out


def pack_layers(lib, cd, dims: Dims, layers, dt, device, sp):
    """Pack a stack of decoder layers (q/k/v, o, gate/up, down and the norm
    gains) on the device; returns the tensors and the ctypes layer array."""
    dcode = cd.dtype
    H = dims.hidden
    out = []
    for lw in layers:
        wq = upload(lw["wq"], dt, device)
        wk = upload(lw["wk"], dt, device)
        wv = upload(lw["wv"], dt, device)
        qkv = torch.empty(lib.dflash_packed_bytes(dcode, dims.qkv_rows, H), dtype=torch.uint8, device=device)
        _lib.call("dflash_pack_qkv", ctypes.byref(cd), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(),
                  qkv.data_ptr(), sp)
        del wq, wk, wv
        wg = upload(lw["w_gate"], dt, device)
        wu = upload(lw["w_up"], dt, device)
        gu = torch.empty(lib.dflash_packed_bytes(dcode, 2 * dims.intermediate, H), dtype=torch.uint8,
                         device=device)
        _lib.call("dflash_pack_gate_up", ctypes.byref(cd), wg.data_ptr(), wu.data_ptr(), gu.data_ptr(), sp)
        del wg, wu
        packed = {}
        for name, key in (("w_o", "wo"), ("w_down", "w_down")):
            src = upload(lw[key], dt, device)
            dst = torch.empty(lib.dflash_packed_bytes(dcode, *lw[key].shape), dtype=torch.uint8, device=device)
            _lib.call("dflash_pack_matrix", dcode, src.data_ptr(), lw[key].shape[0], lw[key].shape[1],
                      dst.data_ptr(), sp)
            packed[name] = dst
        out.append({"attn_norm": upload(lw["attn_norm"], dt, device),
                    "mlp_norm": upload(lw["mlp_norm"], dt, device),
                    "w_qkv": qkv, "w_gate_up": gu, **packed})
    arr = (_lib.Layer * len(out))()
    for i, L in enumerate(out):
        arr[i] = _lib.Layer(L["attn_norm"].data_ptr(), L["w_qkv"].data_ptr(), L["w_o"].data_ptr(),
                            L["mlp_norm"].data_ptr(), L["w_gate_up"].data_ptr(), L["w_down"].data_ptr())
    return out, arr


class Target:
    """The target model's device state for its verify pass: packed layers,
    embedding and final norm, its own KV cache and a workspace (the lm_head
    is the drafter's shared one, applied by the verify call)."""

    def __init__(self, dims: Dims, weights, max_batch: int, capacity: int, max_rows: int = 17,
                 device="cuda:0"):
        self.lib = _lib.load()
        self.dims = dims
        self.cd = cdims(dims)
        self.dt = torch_dtype(dims)
        self.device = torch.device(device)
        self.max_batch, self.capacity, self.max_rows = max_batch, capacity, max_rows
        sp = _stream_ptr(None)
        self.embed = upload(weights.embed, self.dt, self.device)
        self.final_norm = upload(weights.final_norm, self.dt, self.device)
        self.layers, self._layer_arr = pack_layers(self.lib, self.cd, dims, weights.layers, self.dt,
                                                   self.device, sp)
        self.cw = _lib.Weights(None, None, self.embed.data_ptr(), self.final_norm.data_ptr(), None,
                               ctypes.cast(self._layer_arr, ctypes.POINTER(_lib.Layer)))
        kvb = self.lib.dflash_kv_bytes(ctypes.byref(self.cd), capacity, max_batch)
        if kvb == 0:
            raise ValueError("invalid KV cache shape")
        self.k_cache = torch.zeros(kvb, dtype=torch.uint8, device=self.device)
        self.v_cache = torch.zeros(kvb, dtype=torch.uint8, device=self.device)
        self.ctx_len = torch.zeros(max_batch, dtype=torch.int32, device=self.device)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.ckv = _lib.KV(self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.ctx_len.data_ptr(),
                           self.status.data_ptr(), capacity, max_batch)
        self.ws_bytes = self.lib.dflash_target_workspace_bytes(ctypes.byref(self.cd), max_batch, max_rows)
        if self.ws_bytes == 0:
            raise ValueError("invalid target workspace request")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        _lib.call("dflash_workspace_init", self.ws.data_ptr(), self.ws_bytes, sp)

    def forward(self, tokens: torch.Tensor, batch: int, rows: int, feat_layers: Sequence[int],
                out_hidden: torch.Tensor, out_feats: Optional[torch.Tensor], stream=None,
                parents: Optional[torch.Tensor] = None):
        fl = (ctypes.c_int32 * max(1, len(feat_layers)))(*feat_layers)
        _lib.call("dflash_target_forward", ctypes.byref(self.cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(tokens), _ptr(parents), batch, rows, fl, len(feat_layers), _ptr(out_hidden),
                  _ptr(out_feats), self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def commit(self, accept_len: torch.Tensor, batch: int, max_commit: int, stream=None):
        _lib.call("dflash_kv_commit", ctypes.byref(self.cd), ctypes.byref(self.ckv), _ptr(accept_len), batch,
                  max_commit, _stream_ptr(stream))

    def commit_path(self, path: torch.Tensor, accept_len: torch.Tensor, batch: int, n: int, stream=None):
        _lib.call("dflash_kv_commit_path", ctypes.byref(self.cd), ctypes.byref(self.ckv), _ptr(path),
                  _ptr(accept_len), batch, n, _stream_ptr(stream))

    def kv_import(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        _lib.call("dflash_kv_import", ctypes.byref(self.cd), ctypes.byref(self.ckv), k.data_ptr(),
                  v.data_ptr(), _stream_ptr(stream))

    def set_ctx_len(self, lens: Sequence[int]):
        t = torch.as_tensor(np.asarray(lens, dtype=np.int32))
        self.ctx_len[:len(t)].copy_(t)

    def read_status(self) -> int:
        return int(self.status.item())


class Drafter:
    """Packed drafter weights + draft KV cache + workspace on one GPU."""

    def __init__(self, dims: Dims, weights: Weights, max_batch: int, capacity: int,
                 max_rows: int, device="cuda:0", keep_plain: bool = False, max_blocks: int = 0):
        self.lib = _lib.load()
        self.dims = dims
        self.cd = cdims(dims)
        self.dt = torch_dtype(dims)
        self.device = torch.device(device)
        self.max_batch = max_batch
        self.capacity = capacity
        self.max_rows = max_rows
        d = dims
        sp = _stream_ptr(None)
        dcode = self.cd.dtype

        def pack_matrix(arr):
            src = upload(arr, self.dt, self.device)
            nb = self.lib.dflash_packed_bytes(dcode, arr.shape[0], arr.shape[1])
            dst = torch.empty(nb, dtype=torch.uint8, device=self.device)
            _lib.call("dflash_pack_matrix", dcode, src.data_ptr(), arr.shape[0], arr.shape[1],
                      dst.data_ptr(), sp)
            return dst, (src if keep_plain else None)

        def pack_lm_head(arr):
            src = upload(arr, self.dt, self.device)
            nb = self.lib.dflash_packed_bytes(dcode, arr.shape[0], arr.shape[1])
            dst = torch.empty(nb, dtype=torch.uint8, device=self.device)
            _lib.call("dflash_pack_lm_head", dcode, src.data_ptr(), arr.shape[0], arr.shape[1],
                      dst.data_ptr(), sp)
            return dst, (src if keep_plain else None)

        self.plain = {}
        self.w_fc, self.plain["w_fc"] = pack_matrix(weights.w_fc)
        self.lm_head, self.plain["lm_head"] = pack_lm_head(weights.lm_head)
        self.fc_norm = upload(weights.fc_norm, self.dt, self.device)
        self.final_norm = upload(weights.final_norm, self.dt, self.device)
        self.embed = upload(weights.embed, self.dt, self.device)
        self.layers = []
        H, hd = d.hidden, d.head_dim
        for lw in weights.layers:
            wq = upload(lw["wq"], self.dt, self.device)
            wk = upload(lw["wk"], self.dt, self.device)
            wv = upload(lw["wv"], self.dt, self.device)
            qkv = torch.empty(self.lib.dflash_packed_bytes(dcode, d.qkv_rows, H), dtype=torch.uint8,
                              device=self.device)
            _lib.call("dflash_pack_qkv", ctypes.byref(self.cd), wq.data_ptr(), wk.data_ptr(),
                      wv.data_ptr(), qkv.data_ptr(), sp)
            wg = upload(lw["w_gate"], self.dt, self.device)
            wu = upload(lw["w_up"], self.dt, self.device)
            gu = torch.empty(self.lib.dflash_packed_bytes(dcode, 2 * d.intermediate, H),
                             dtype=torch.uint8, device=self.device)
            _lib.call("dflash_pack_gate_up", ctypes.byref(self.cd), wg.data_ptr(), wu.data_ptr(),
                      gu.data_ptr(), sp)
            wo, _ = pack_matrix(lw["wo"])
            wd, _ = pack_matrix(lw["w_down"])
            self.layers.append({
                "attn_norm": upload(lw["attn_norm"], self.dt, self.device),
                "mlp_norm": upload(lw["mlp_norm"], self.dt, self.device),
                "w_qkv": qkv, "w_gate_up": gu, "w_o": wo, "w_down": wd,
            })
            del wq, wk, wv, wg, wu
        self._layer_arr = (_lib.Layer * d.n_layers)()
        for i, L in enumerate(self.layers):
            self._layer_arr[i] = _lib.Layer(L["attn_norm"].data_ptr(), L["w_qkv"].data_ptr(),
                                            L["w_o"].data_ptr(), L["mlp_norm"].data_ptr(),
                                            L["w_gate_up"].data_ptr(), L["w_down"].data_ptr())
        self.cw = _lib.Weights(self.w_fc.data_ptr(), self.fc_norm.data_ptr(), self.embed.data_ptr(),
                               self.final_norm.data_ptr(), self.lm_head.data_ptr(),
                               ctypes.cast(self._layer_arr, ctypes.POINTER(_lib.Layer)))
        kvb = self.lib.dflash_kv_bytes(ctypes.byref(self.cd), capacity, max_batch)
        if kvb == 0:
            raise ValueError("invalid KV cache shape")
        self.k_cache = torch.zeros(kvb, dtype=torch.uint8, device=self.device)
        self.v_cache = torch.zeros(kvb, dtype=torch.uint8, device=self.device)
        self.ctx_len = torch.zeros(max_batch, dtype=torch.int32, device=self.device)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.ckv = _lib.KV(self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.ctx_len.data_ptr(),
                           self.status.data_ptr(), capacity, max_batch)
        # the workspace holds the largest draft call: max_batch sequences, or
        # max_blocks anchored blocks
        self.max_blocks = max(max_batch, max_blocks)
        self.ws_bytes = self.lib.dflash_workspace_bytes(ctypes.byref(self.cd), self.max_blocks, max_rows)
        if self.ws_bytes == 0:
            raise ValueError("invalid workspace request")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        _lib.call("dflash_workspace_init", self.ws.data_ptr(), self.ws_bytes, sp)

    # ------------------------------------------------------------ the step
    def inject(self, feats: torch.Tensor, cu_new: torch.Tensor, batch: int, rows: int, stream=None):
        _lib.call("dflash_inject_kv", ctypes.byref(self.cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(feats), _ptr(cu_new), batch, rows, self.ws.data_ptr(), self.ws_bytes,
                  _stream_ptr(stream))

    def dims_for(self, block_size: Optional[int] = None) -> _lib.Dims:
        """The drafter's dims, with another block size for this call (any
        B <= the drafter's: its workspace is sized for that)."""
        if block_size is None or block_size == self.dims.block_size:
            return self.cd
        if not 1 <= block_size <= self.dims.block_size:
            raise ValueError(f"block size {block_size} outside [1, {self.dims.block_size}]")
        cd = cdims(self.dims.with_block(block_size))
        return cd

    def draft(self, last_tok: torch.Tensor, out: torch.Tensor, batch: int, stream=None,
              block_size: Optional[int] = None):
        cd = self.dims_for(block_size)
        _lib.call("dflash_draft_forward", ctypes.byref(cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(last_tok), batch, _ptr(out), self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def draft_anchors(self, anchor_seq: torch.Tensor, anchor_pos: torch.Tensor, anchor_tok: torch.Tensor,
                      out: torch.Tensor, nblocks: int, stream=None, block_size: Optional[int] = None):
        cd = self.dims_for(block_size)
        _lib.call("dflash_draft_anchors", ctypes.byref(cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(anchor_seq), _ptr(anchor_pos), _ptr(anchor_tok), nblocks, _ptr(out),
                  self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def draft_sample(self, last_tok: torch.Tensor, temperature: float, u_draft: torch.Tensor,
                     out: torch.Tensor, draft_logits: torch.Tensor, batch: int, stream=None,
                     block_size: Optional[int] = None):
        cd = self.dims_for(block_size)
        _lib.call("dflash_draft_sample", ctypes.byref(cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(last_tok), batch, float(temperature), _ptr(u_draft), _ptr(out), _ptr(draft_logits),
                  self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def verify_sample(self, target_hidden: torch.Tensor, draft: torch.Tensor, draft_logits: torch.Tensor,
                      temperature: float, u_accept: torch.Tensor, u_resid: torch.Tensor,
                      target_logits: torch.Tensor, accept_len: torch.Tensor, next_tok: torch.Tensor,
                      batch: int, stream=None, block_size: Optional[int] = None):
        cd = self.dims_for(block_size)
        _lib.call("dflash_verify_sample", ctypes.byref(cd), self.lm_head.data_ptr(), _ptr(target_hidden),
                  _ptr(draft), _ptr(draft_logits), batch, float(temperature), _ptr(u_accept), _ptr(u_resid),
                  _ptr(target_logits), _ptr(accept_len), _ptr(next_tok), self.ws.data_ptr(), self.ws_bytes,
                  _stream_ptr(stream))

    def draft_tree(self, last_tok: torch.Tensor, topk: int, nodes: int, draft_logits: torch.Tensor,
                   tree_tok: torch.Tensor, tree_parent: torch.Tensor, batch: int, stream=None):
        _lib.call("dflash_draft_tree", ctypes.byref(self.cd), ctypes.byref(self.cw), ctypes.byref(self.ckv),
                  _ptr(last_tok), batch, topk, nodes, _ptr(draft_logits), _ptr(tree_tok), _ptr(tree_parent),
                  self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def tree_accept(self, target_hidden: torch.Tensor, tree_tok: torch.Tensor, tree_parent: torch.Tensor,
                    batch: int, n: int, target_argmax: torch.Tensor, accept_len: torch.Tensor,
                    bonus: torch.Tensor, path: torch.Tensor, stream=None):
        _lib.call("dflash_tree_accept", ctypes.byref(self.cd), self.lm_head.data_ptr(), _ptr(target_hidden),
                  _ptr(tree_tok), _ptr(tree_parent), batch, n, _ptr(target_argmax), _ptr(accept_len), _ptr(bonus),
                  _ptr(path), self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    def verify(self, target_hidden: torch.Tensor, draft: torch.Tensor, target_argmax: torch.Tensor,
               accept_len: torch.Tensor, bonus: torch.Tensor, batch: int, stream=None,
               block_size: Optional[int] = None):
        cd = self.dims_for(block_size)
        _lib.call("dflash_verify_accept", ctypes.byref(cd), self.lm_head.data_ptr(),
                  _ptr(target_hidden), _ptr(draft), batch, _ptr(target_argmax), _ptr(accept_len),
                  _ptr(bonus), self.ws.data_ptr(), self.ws_bytes, _stream_ptr(stream))

    # ------------------------------------------------------------ helpers
    def view(self, what: int, count: int, layer: int = 0, block_size: Optional[int] = None) -> torch.Tensor:
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        _lib.call("dflash_workspace_view", ctypes.byref(self.dims_for(block_size)), what, count, layer,
                  ctypes.byref(off), ctypes.byref(nb))
        return self.ws[off.value:off.value + nb.value].view(torch.float32)

    def kv_plain_shape(self):
        d = self.dims
        return (d.n_layers, self.max_batch, d.n_kv_heads, self.capacity, d.head_dim)

    def kv_import(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        assert k.shape == self.kv_plain_shape() and k.dtype == self.dt and k.is_contiguous()
        assert v.shape == self.kv_plain_shape() and v.dtype == self.dt and v.is_contiguous()
        _lib.call("dflash_kv_import", ctypes.byref(self.cd), ctypes.byref(self.ckv), k.data_ptr(),
                  v.data_ptr(), _stream_ptr(stream))

    def kv_export(self, stream=None):
        k = torch.empty(self.kv_plain_shape(), dtype=self.dt, device=self.device)
        v = torch.empty(self.kv_plain_shape(), dtype=self.dt, device=self.device)
        _lib.call("dflash_kv_export", ctypes.byref(self.cd), ctypes.byref(self.ckv), k.data_ptr(),
                  v.data_ptr(), _stream_ptr(stream))
        return k, v

    def bind_ctx_len(self, ctx_len: Optional[torch.Tensor] = None):
        """Point the cache's per-sequence context lengths at another int32
        device array of max_batch entries (None: back to the drafter's own).
        The K/V rows stay shared; only where lengths are read and committed
        changes."""
        t = self.ctx_len if ctx_len is None else ctx_len
        assert t.dtype == torch.int32 and t.device == self.device and t.numel() >= self.ckv.max_batch
        self.ckv.ctx_len = t.data_ptr()
        self._bound_ctx = t   # keep the array alive while bound

    def set_ctx_len(self, lens: Sequence[int]):
        t = torch.as_tensor(np.asarray(lens, dtype=np.int32))
        self.ctx_len[:len(t)].copy_(t)

    def read_status(self) -> int:
        return int(self.status.item())

    def clear_status(self):
        self.status.zero_()
