"""Runs one draft-and-verify step on the GPU (through the C ABI) and in the
fp64 oracle from the same seeded inputs, and compares the results.

The oracle never sees a value produced by the GPU path: every oracle input
comes from the seeded generator, and the planted verification targets are
built from the oracle's own drafted tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle.dflash_oracle as O
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I

REL_TOL = 2e-2        # hidden / attention outputs (bf16 inputs, fp32 accumulation)
GAP = 1e-2            # token ids must match where the oracle's top-1/top-2 gap exceeds this


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref|| / ||ref||."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    return float(np.max(num / den))


HEAD = 128            # channels per attention head: the per-head error segment


def rel_err_heads(got: np.ndarray, ref: np.ndarray, seg: int = HEAD) -> float:
    """max over rows and over each row's ``seg``-channel segments of
    ||got - ref|| / ||ref||: localises an error confined to one head or one
    rotary pair that a whole-row norm would dilute.  Rows narrower than
    ``seg`` are taken whole."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    w = g.shape[-1]
    s = seg if w % seg == 0 else w
    g = g.reshape(-1, s)
    r = r.reshape(-1, s)
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    return float(np.max(num / den))


@dataclass
class TokenReport:
    compared: int = 0
    below_gap: int = 0
    mismatched: List[tuple] = field(default_factory=list)

    def add(self, got: np.ndarray, want: np.ndarray, gaps: np.ndarray, tag: str):
        got = np.asarray(got).reshape(-1)
        want = np.asarray(want).reshape(-1)
        gaps = np.asarray(gaps).reshape(-1)
        for i in range(len(want)):
            if gaps[i] > GAP:
                self.compared += 1
                if got[i] != want[i]:
                    self.mismatched.append((tag, i, int(got[i]), int(want[i]), float(gaps[i])))
            else:
                self.below_gap += 1


@dataclass
class Case:
    dims: C.Dims
    weights: I.Weights
    batch: int
    ctx: np.ndarray            # context length per sequence before the step
    capacity: int
    seed: int
    kv_mode: str               # "inject" or "import"
    prefill: Optional[List[np.ndarray]] = None
    kv_plain: Optional[tuple] = None


def build_case(dims: C.Dims, batch: int, ctx: Sequence[int], seed: int, kv_mode: str = "inject",
               capacity: Optional[int] = None, gain_std: float = 0.0,
               weights: Optional[I.Weights] = None) -> Case:
    ctx = np.asarray(ctx, dtype=np.int32)
    cap = capacity or C.kv_capacity(int(ctx.max()))
    w = weights or I.make_weights(dims, seed, gain_std=gain_std)
    case = Case(dims, w, batch, ctx, cap, seed, kv_mode)
    if kv_mode == "inject":
        case.prefill = [I.prefill_features(dims, seed, s, int(ctx[s])) for s in range(batch)]
    else:
        shape = (dims.n_layers, batch, dims.n_kv_heads, cap, dims.head_dim)
        k = np.zeros(shape, dtype=np.float32)
        v = np.zeros(shape, dtype=np.float32)
        for l in range(dims.n_layers):
            for s in range(batch):
                ks, vs = I.kv_entries(dims, seed, l, s, int(ctx[s]))
                k[l, s, :, :ctx[s]] = ks
                v[l, s, :, :ctx[s]] = vs
        case.kv_plain = (k, v)
    return case


def oracle_prefill(case: Case, seqs: Sequence[int]) -> O.OracleCache:
    """Oracle cache holding only the sequences in ``seqs`` (in that order)."""
    d = case.dims
    cache = O.OracleCache.empty(d, len(seqs), case.capacity)
    if case.kv_mode == "inject":
        O.inject(d, case.weights, cache, [case.prefill[s] for s in seqs])
    else:
        k, v = case.kv_plain
        for i, s in enumerate(seqs):
            cache.k[:, i] = k[:, s]
            cache.v[:, i] = v[:, s]
            cache.length[i] = case.ctx[s]
    return cache


def step_inputs(case: Case, step: int, new_rows: Sequence[int]):
    d = case.dims
    feats = [I.features(d, case.seed, step, s, int(new_rows[s])) for s in range(case.batch)]
    last = I.last_tokens(d, case.seed, step, case.batch)
    return feats, last


def oracle_step(case: Case, step: int, new_rows: Sequence[int], seqs: Sequence[int],
                accept_p: float) -> Dict:
    """Oracle inject + draft for ``seqs``; then planted targets from the
    oracle's drafted tokens and the oracle's verify + accept."""
    d = case.dims
    feats, last = step_inputs(case, step, new_rows)
    cache = oracle_prefill(case, seqs)
    fused = O.inject(d, case.weights, cache, [feats[s] for s in seqs])
    dr = O.draft_forward(d, case.weights, cache, last[list(seqs)])
    L_plant = I.planted_accept(case.seed, step, case.batch, accept_p, d.block_size)
    return {"cache": cache, "fused": fused, "draft": dr, "last": last, "feats": feats,
            "planted_L": L_plant}


def planted_verify_inputs(case: Case, step: int, oracle_tokens_all: np.ndarray, planted_L: np.ndarray):
    """Target hidden states for all sequences; ``oracle_tokens_all`` [b, B]
    holds the oracle's drafted tokens (random stand-ins for sequences the
    oracle did not run are drawn by the caller from the generator)."""
    return I.planted_targets(case.dims, case.seed, step, case.weights.lm_head, oracle_tokens_all, planted_L)


# ------------------------------------------------------------------- GPU side

class GpuRunner:
    """Owns a Drafter for one case and runs the three entry points."""

    def __init__(self, case: Case, max_rows: Optional[int] = None, max_blocks: int = 0):
        import torch
        from block_diffusion_speculative_amd.engine import Drafter, upload
        self.torch = torch
        self.case = case
        d = case.dims
        self.max_rows = max_rows or max(int(case.ctx.sum()) if case.kv_mode == "inject" else 0, 17 * case.batch)
        self.drafter = Drafter(d, case.weights, case.batch, case.capacity, self.max_rows, max_blocks=max_blocks)
        self.upload = upload
        dev = self.drafter.device
        if case.kv_mode == "inject":
            self.inject([f for f in case.prefill])
        else:
            k, v = case.kv_plain
            kt = upload(k.reshape(-1, d.head_dim), self.drafter.dt, dev).reshape(k.shape)
            vt = upload(v.reshape(-1, d.head_dim), self.drafter.dt, dev).reshape(v.shape)
            self.drafter.kv_import(kt, vt)
            self.drafter.set_ctx_len(case.ctx)
        torch.cuda.synchronize()

    def inject(self, feats: List[np.ndarray]):
        torch = self.torch
        d = self.case.dims
        rows = [f.shape[0] for f in feats]
        cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        total = int(cu[-1])
        cu_t = torch.as_tensor(cu).to(self.drafter.device)
        if total == 0:
            self.drafter.inject(None, cu_t, self.case.batch, 0)
            return
        allf = np.concatenate(feats, axis=0)
        ft = self.upload(allf, self.drafter.dt, self.drafter.device)
        self.drafter.inject(ft, cu_t, self.case.batch, total)
        torch.cuda.synchronize()

    def draft(self, last: np.ndarray) -> np.ndarray:
        torch = self.torch
        b, B = self.case.batch, self.case.dims.block_size
        lt = torch.as_tensor(np.asarray(last, dtype=np.int32)).to(self.drafter.device)
        out = torch.full((b, B), -1, dtype=torch.int32, device=self.drafter.device)
        self.drafter.draft(lt, out, b)
        torch.cuda.synchronize()
        self.last_draft = out
        return out.cpu().numpy()

    def verify(self, target_hidden: np.ndarray, draft: np.ndarray):
        torch = self.torch
        b, B, H = self.case.batch, self.case.dims.block_size, self.case.dims.hidden
        th = self.upload(target_hidden.reshape(b * (B + 1), H), self.drafter.dt,
                         self.drafter.device).reshape(b, B + 1, H)
        dr = torch.as_tensor(np.asarray(draft, dtype=np.int32)).to(self.drafter.device)
        ta = torch.full((b, B + 1), -1, dtype=torch.int32, device=self.drafter.device)
        al = torch.full((b,), -1, dtype=torch.int32, device=self.drafter.device)
        bo = torch.full((b,), -1, dtype=torch.int32, device=self.drafter.device)
        self.drafter.verify(th, dr, ta, al, bo, b)
        torch.cuda.synchronize()
        return ta.cpu().numpy(), al.cpu().numpy(), bo.cpu().numpy()

    def fused_view(self, rows: int):
        from block_diffusion_speculative_amd import _lib
        if rows == 0:
            return None
        return self.drafter.view(_lib.VIEW_FUSED, rows, 0).reshape(rows, -1).cpu().numpy()

    def views(self):
        from block_diffusion_speculative_amd import _lib
        d = self.case.dims
        b, B = self.case.batch, d.block_size
        M = b * B
        out = {"attn": [], "mid": [], "hidden": []}
        for l in range(d.n_layers):
            out["attn"].append(self.drafter.view(_lib.VIEW_ATTN, b, l).reshape(M, -1).cpu().numpy())
            out["mid"].append(self.drafter.view(_lib.VIEW_MID, b, l).reshape(M, -1).cpu().numpy())
        for l in range(-1, d.n_layers):
            out["hidden"].append(self.drafter.view(_lib.VIEW_HIDDEN, b, l).reshape(M, -1).cpu().numpy())
        return out

    def kv_plain(self):
        k, v = self.drafter.kv_export()
        return k.float().cpu().numpy(), v.float().cpu().numpy()

    def kv_rows(self, seq: int, lo: int, hi: int):
        """Cache positions [lo, hi) of one sequence, every layer and head:
        K and V as [n_layers, n_kv, hi - lo, head_dim] (sliced on the device,
        so a full-size cache never crosses to the host)."""
        k, v = self.drafter.kv_export()
        ks = k[:, seq, :, lo:hi].float().cpu().numpy()
        vs = v[:, seq, :, lo:hi].float().cpu().numpy()
        del k, v
        return ks, vs

    def ctx_len(self):
        return self.drafter.ctx_len.cpu().numpy()
