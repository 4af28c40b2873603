"""Seeded synthetic inputs for the draft-and-verify step.

This module is shared by the tests, the benchmark and the checks against the
fp64 oracle.  It holds random-number generation, bf16 rounding of the draws
and the planting of verification targets; none of the method's arithmetic
(projections, attention, norms, argmax, acceptance) is computed here.

Every tensor comes from its own ``numpy.random.PCG64`` stream keyed by
``SeedSequence([seed, tensor_id, *sub_ids, chunk])``, so the values do not
depend on generation order or on the number of worker threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import Dims, Workload

WEIGHT_STD = 0.02
FEATURE_STD = 1.0
TARGET_SCALE = 4.0
TARGET_NOISE_STD = 0.1
KV_STD = 1.28          # std of an injected K/V entry: 0.02 * sqrt(4096)

_CHUNK = 1 << 22       # elements per independent random stream

# Tensor ids: one per kind; per-layer tensors add the layer index.
TID = {
    "w_fc": 1, "fc_norm": 2, "embed": 3, "final_norm": 4, "lm_head": 5,
    "attn_norm": 10, "wq": 11, "wk": 12, "wv": 13, "wo": 14,
    "mlp_norm": 15, "w_gate": 16, "w_up": 17, "w_down": 18,
    "features": 30, "prefill": 31, "last_tok": 32, "accept": 33,
    "targets": 34, "target_noise": 35, "ctx_len": 36, "new_rows": 37,
    "kv_k": 40, "kv_v": 41,
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def stream(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(i) for i in ids])))


def round_bf16_(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 value (ties to even), in
    place.  Inputs are finite by construction."""
    assert x.dtype == np.float32
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of a float32 array whose values are
    already bf16-representable."""
    assert x.dtype == np.float32
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, ids: Sequence[int], shape, std: float, dtype: str,
           mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, rounded to ``dtype`` ("bf16"
    rounds to bf16 values; "f32" keeps float32)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        if lo >= hi:
            return
        g = stream(seed, *ids, c)
        seg = out[lo:hi]
        g.standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= np.float32(std)
        if mean != 0.0:
            seg += np.float32(mean)
        if dtype == "bf16":
            round_bf16_(seg)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _gain(seed, ids, n, dtype, gain_std):
    if gain_std == 0.0:
        return np.ones(n, dtype=np.float32)
    return normal(seed, ids, (n,), gain_std, dtype, mean=1.0)


@dataclass
class Weights:
    """Drafter weights as float32 arrays holding storage-type values
    (bf16-representable for bf16 drafters).  Matrices are [out, in]."""

    w_fc: np.ndarray
    fc_norm: np.ndarray
    embed: np.ndarray
    final_norm: np.ndarray
    lm_head: np.ndarray
    layers: List[Dict[str, np.ndarray]]


def make_weights(dims: Dims, seed: int, gain_std: float = 0.0) -> Weights:
    """All matrices ~ N(0, 0.02^2); RMSNorm gains 1 (or 1 + N(0, gain_std^2))."""
    H, d, I, V = dims.hidden, dims.head_dim, dims.intermediate, dims.vocab
    dt = dims.dtype
    layers = []
    for l in range(dims.n_layers):
        layers.append({
            "attn_norm": _gain(seed, (TID["attn_norm"], l), H, dt, gain_std),
            "wq": normal(seed, (TID["wq"], l), (dims.n_q_heads * d, H), WEIGHT_STD, dt),
            "wk": normal(seed, (TID["wk"], l), (dims.n_kv_heads * d, H), WEIGHT_STD, dt),
            "wv": normal(seed, (TID["wv"], l), (dims.n_kv_heads * d, H), WEIGHT_STD, dt),
            "wo": normal(seed, (TID["wo"], l), (H, dims.n_q_heads * d), WEIGHT_STD, dt),
            "mlp_norm": _gain(seed, (TID["mlp_norm"], l), H, dt, gain_std),
            "w_gate": normal(seed, (TID["w_gate"], l), (I, H), WEIGHT_STD, dt),
            "w_up": normal(seed, (TID["w_up"], l), (I, H), WEIGHT_STD, dt),
            "w_down": normal(seed, (TID["w_down"], l), (H, I), WEIGHT_STD, dt),
        })
    return Weights(
        w_fc=normal(seed, (TID["w_fc"],), (H, dims.feat_dim), WEIGHT_STD, dt),
        fc_norm=_gain(seed, (TID["fc_norm"],), H, dt, gain_std),
        embed=normal(seed, (TID["embed"],), (V, H), WEIGHT_STD, dt),
        final_norm=_gain(seed, (TID["final_norm"],), H, dt, gain_std),
        lm_head=normal(seed, (TID["lm_head"],), (V, H), WEIGHT_STD, dt),
        layers=layers,
    )


@dataclass
class TargetWeights:
    """The target's weights for its verify pass (the lm_head is the
    drafter's shared one)."""

    embed: np.ndarray
    final_norm: np.ndarray
    layers: List[Dict[str, np.ndarray]]


# Tensor ids of the target's weights: the drafter's ids + TARGET_TID.
TARGET_TID = 100


def make_target_weights(dims: Dims, seed: int, gain_std: float = 0.0) -> TargetWeights:
    """Target layers of the drafter's layer type, ~N(0, 0.02^2), gains 1,
    from streams of their own (ids offset by TARGET_TID)."""
    H, d, I, V = dims.hidden, dims.head_dim, dims.intermediate, dims.vocab
    dt = dims.dtype
    T = TARGET_TID
    layers = []
    for l in range(dims.n_layers):
        layers.append({
            "attn_norm": _gain(seed, (T + TID["attn_norm"], l), H, dt, gain_std),
            "wq": normal(seed, (T + TID["wq"], l), (dims.n_q_heads * d, H), WEIGHT_STD, dt),
            "wk": normal(seed, (T + TID["wk"], l), (dims.n_kv_heads * d, H), WEIGHT_STD, dt),
            "wv": normal(seed, (T + TID["wv"], l), (dims.n_kv_heads * d, H), WEIGHT_STD, dt),
            "wo": normal(seed, (T + TID["wo"], l), (H, dims.n_q_heads * d), WEIGHT_STD, dt),
            "mlp_norm": _gain(seed, (T + TID["mlp_norm"], l), H, dt, gain_std),
            "w_gate": normal(seed, (T + TID["w_gate"], l), (I, H), WEIGHT_STD, dt),
            "w_up": normal(seed, (T + TID["w_up"], l), (I, H), WEIGHT_STD, dt),
            "w_down": normal(seed, (T + TID["w_down"], l), (H, I), WEIGHT_STD, dt),
        })
    return TargetWeights(
        embed=normal(seed, (T + TID["embed"],), (V, H), WEIGHT_STD, dt),
        final_norm=_gain(seed, (T + TID["final_norm"],), H, dt, gain_std),
        layers=layers,
    )


def target_tokens(dims: Dims, seed: int, step: int, batch: int, rows: int) -> np.ndarray:
    """Token ids of a target pass, uniform over [0, vocab - 1)."""
    g = stream(seed, TID["last_tok"] + TARGET_TID, step)
    return g.integers(0, dims.vocab - 1, size=(batch, rows), dtype=np.int64).astype(np.int32)


# ----------------------------------------------------------------- features

def features(dims: Dims, seed: int, step: int, seq: int, rows: int) -> np.ndarray:
    """Target features for ``rows`` newly accepted positions of one sequence:
    [rows, n_feat_layers * hidden], layer-major concatenation, ~N(0, 1)."""
    return normal(seed, (TID["features"], step, seq), (rows, dims.feat_dim), FEATURE_STD, dims.dtype)


def prefill_features(dims: Dims, seed: int, seq: int, rows: int) -> np.ndarray:
    return normal(seed, (TID["prefill"], seq), (rows, dims.feat_dim), FEATURE_STD, dims.dtype)


def last_tokens(dims: Dims, seed: int, step: int, batch: int) -> np.ndarray:
    """Last accepted token per sequence, uniform over [0, vocab - 1)."""
    g = stream(seed, TID["last_tok"], step)
    return g.integers(0, dims.vocab - 1, size=batch, dtype=np.int64).astype(np.int32)


def context_lengths(w: Workload, seed: int) -> np.ndarray:
    lo, hi = w.ctx
    if lo == hi:
        return np.full(w.batch, lo, dtype=np.int32)
    g = stream(seed, TID["ctx_len"])
    return g.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)


def new_row_counts(w: Workload, seed: int, step: int,
                   prev_accept: Optional[np.ndarray] = None) -> np.ndarray:
    """Rows injected per sequence this step: a seeded U{lo..hi} when the
    workload fixes a range, else the previous step's accepted length plus
    one (one row on the first step)."""
    if w.new_rows is not None:
        lo, hi = w.new_rows
        g = stream(seed, TID["new_rows"], step)
        return g.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)
    if prev_accept is None:
        return np.ones(w.batch, dtype=np.int32)
    return (np.asarray(prev_accept, dtype=np.int32) + 1)


def kv_entries(dims: Dims, seed: int, layer: int, seq: int, rows: int):
    """Directly generated cache contents for one (layer, sequence):
    K and V of shape [n_kv_heads, rows, head_dim], ~N(0, KV_STD^2)."""
    shape = (dims.n_kv_heads, rows, dims.head_dim)
    k = normal(seed, (TID["kv_k"], layer, seq), shape, KV_STD, dims.dtype)
    v = normal(seed, (TID["kv_v"], layer, seq), shape, KV_STD, dims.dtype)
    return k, v


# ------------------------------------------------------- planted acceptance

def geometric_mean_accept(p: float, B: int) -> float:
    """E[min(G, B)] for G geometric on {0, 1, ...} with P(G = k) = (1-p)^k p."""
    q = 1.0 - p
    return q * (1.0 - q ** B) / p


def geom_p_for_mean(mean: float, B: int = 16) -> float:
    """Geometric parameter whose truncated mean at B equals ``mean``."""
    if not (0.0 < mean < B):
        raise ValueError("mean must lie in (0, B)")
    lo, hi = 1e-9, 1.0 - 1e-12
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if geometric_mean_accept(mid, B) > mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def workload_geom_p(w: Workload) -> float:
    if w.geom_p is not None:
        return w.geom_p
    return geom_p_for_mean(w.mean_accept, 16)


def planted_accept(seed: int, step: int, batch: int, p: float, B: int) -> np.ndarray:
    """Planted accept length per sequence: min(G, B), G ~ Geometric(p) on {0,1,...}."""
    g = stream(seed, TID["accept"], step)
    G = g.geometric(p, size=batch) - 1
    return np.minimum(G, B).astype(np.int32)


def _uniform_except(g: np.random.Generator, V: int, excluded: int) -> int:
    u = int(g.integers(0, V - 1))
    return u + 1 if u >= excluded else u


def planted_targets(dims: Dims, seed: int, step: int, lm_head: np.ndarray,
                    draft: np.ndarray, accept: np.ndarray):
    """Target tokens t[b, B+1] and target final hidden states
    h[b, B+1, H] = 4 * lm_head[t] + N(0, 0.1^2), rounded to the storage type.

    t_j equals the drafted token d_j for j < L; t_L differs from d_L when
    L < B; t_j for L < j < B differs from d_j; t_B is uniform.  ``draft``
    is taken as given (the caller supplies the oracle's drafted tokens)."""
    B, V, H = dims.block_size, dims.vocab, dims.hidden
    draft = np.asarray(draft, dtype=np.int64).reshape(-1, B)
    batch = draft.shape[0]
    t = np.zeros((batch, B + 1), dtype=np.int32)
    for s in range(batch):
        g = stream(seed, TID["targets"], step, s)
        L = int(accept[s])
        for j in range(B):
            if j < L:
                t[s, j] = draft[s, j]
            else:
                t[s, j] = _uniform_except(g, V, int(draft[s, j]))
        t[s, B] = int(g.integers(0, V))
    noise = normal(seed, (TID["target_noise"], step), (batch, B + 1, H), TARGET_NOISE_STD, "f32")
    hid = np.float32(TARGET_SCALE) * lm_head[t.reshape(-1)].reshape(batch, B + 1, H) + noise
    hid = hid.astype(np.float32)
    if dims.dtype == "bf16":
        round_bf16_(hid)
    return t, hid
