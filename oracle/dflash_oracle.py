"""Plain fp64 reference of one DFlash draft-and-verify step (numpy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (page title, then section):

* [Report/KP]  "DFlash, Diffusion LLMs, dLLM, MTP and Speculative Decoding:
  A Deep Research Report", "Key points": target-context features from
  several layers are injected into the K/V projections of every draft layer
  and kept in the draft KV cache; the drafter fills a block of 16 masked
  positions in one forward pass.
* [Report/Why]  same page, "Why DFlash beats EAGLE-3", item 3, and the
  MTP-vs-diffusion comparison table: attention is bidirectional inside the
  block.
* [Term/WF]  "Term: DFlash speculative decoding", "DFlash: architecture and
  workflow": anchor at the frontier, one drafting pass, the target computes
  logits at every block position and checks the draft against its argmax,
  the longest contiguous accepted prefix is emitted and decoding falls back
  to the target for the next token.
* [Term/Math]  same page, "Mathematical view of acceptance and speedup":
  S ~= C_AR / (C_DF / E[L]).
* [Forum]  "LLMs hit ludicrous speed: diffusion decoding and dMoE supercharge
  AI inference, shattering old benchmarks", the DDTree paragraph: a draft
  tree built best-first from per-position distributions and verified in one
  target pass under an ancestor-only attention mask.

Readings where the pages are silent (each is listed with its reason in the
design notes): one drafting pass (T = 1); B drafted tokens, one per block
slot, slot 0 holding the last accepted token; B + 1 verify rows so the
fallback ("bonus") token always exists; rotate-half RoPE with
omega_i = theta^(-2i/d) on q and k of the block and on k of injected rows;
contiguous GQA grouping; softmax scale 1/sqrt(d) with no mask; RMSNorm with
eps inside the square root and a per-channel gain; SwiGLU MLP; no biases;
the injected context c = RMSNorm(W_fc [f_0 .. f_{n-1}]) is projected by each
layer's own W_k / W_v; block K/V are not stored in the cache; ties in argmax
go to the lowest index.

Everything is computed in float64 from the stored input values (bf16 inputs
arrive as exactly-representable float32 values and are widened, never
re-rounded).  Large matrices are widened one row chunk at a time.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

_CHUNK_ROWS = 8192


# --------------------------------------------------------------- primitives

def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T for W stored [out, in] (the PyTorch Linear convention).

    ``x`` is [..., in]; W is widened to fp64 in row chunks so that a
    151936 x 4096 matrix never exists in fp64 all at once."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape[:-1] + (w.shape[0],), dtype=np.float64)
    for r0 in range(0, w.shape[0], _CHUNK_ROWS):
        wc = np.asarray(w[r0:r0 + _CHUNK_ROWS], dtype=np.float64)
        out[..., r0:r0 + wc.shape[0]] = x @ wc.T
    return out


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.

    ``x`` is [n, heads, d]; ``positions`` is [n].  Channel i < d/2 is paired
    with channel i + d/2 and the pair is rotated by the angle
    position * theta^(-2i/d).  theta == 0 disables the rotation."""
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Unmasked softmax attention with grouped K/V heads.

    q: [Bq, n_q, d]; k, v: [T, n_kv, d].  Query head h reads K/V head
    h // (n_q / n_kv).  Every query sees every key (bidirectional inside the
    block and the whole injected context, [Report/Why], [Term/WF])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nkv, d = q.shape[1], k.shape[1], q.shape[2]
    group = nq // nkv
    out = np.empty_like(q)
    for h in range(nq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)          # [Bq, T]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def argmax_lowest(logits: np.ndarray):
    """Index of the maximum along the last axis, lowest index on ties, and
    the gap between the largest and second-largest logit (0 on a tie)."""
    logits = np.asarray(logits, dtype=np.float64)
    idx = np.argmax(logits, axis=-1)          # numpy returns the first maximum
    top1 = np.take_along_axis(logits, idx[..., None], axis=-1)[..., 0]
    masked = logits.copy()
    np.put_along_axis(masked, idx[..., None], -np.inf, axis=-1)
    top2 = masked.max(axis=-1)
    return idx.astype(np.int64), top1 - top2


def accept(draft: np.ndarray, target_argmax: np.ndarray):
    """Greedy acceptance ([Term/WF] stages three and four).

    draft: [b, B]; target_argmax: [b, B+1].  L is the length of the longest
    prefix on which the drafted tokens equal the target's argmax; the
    fallback token is the target's argmax at the first mismatch (row B when
    the whole block matches)."""
    draft = np.asarray(draft)
    tgt = np.asarray(target_argmax)
    b, B = draft.shape
    L = np.zeros(b, dtype=np.int64)
    bonus = np.zeros(b, dtype=np.int64)
    for s in range(b):
        n = 0
        while n < B and draft[s, n] == tgt[s, n]:
            n += 1
        L[s] = n
        bonus[s] = tgt[s, n]
    return L, bonus


def speedup(c_ar: float, c_df: float, mean_accept: float) -> float:
    """S ~= C_AR / (C_DF / E[L]) ([Term/Math])."""
    return c_ar / (c_df / mean_accept)


# ------------------------------------------------------------------ the step

@dataclass
class OracleCache:
    """Draft KV cache in fp64: k, v are [n_layers, batch, n_kv, capacity, d];
    ``length`` holds the number of valid positions per sequence."""

    k: np.ndarray
    v: np.ndarray
    length: np.ndarray

    @classmethod
    def empty(cls, dims, batch: int, capacity: int) -> "OracleCache":
        shape = (dims.n_layers, batch, dims.n_kv_heads, capacity, dims.head_dim)
        return cls(np.zeros(shape), np.zeros(shape), np.zeros(batch, dtype=np.int64))


def _get(w, name):
    return getattr(w, name) if not isinstance(w, dict) else w[name]


def inject(dims, weights, cache: OracleCache, feats: Sequence[np.ndarray],
           pos_offset: int = 0) -> List[np.ndarray]:
    """KV injection ([Report/KP]).

    For sequence s with new feature rows F_s [n_s, n_f * H] written at cache
    slots len_s + i (rotary position len_s + i + pos_offset):
    c = RMSNorm(W_fc F_s) * g_fc; for every layer l, K = RoPE(W_k^l c, P) and
    V = W_v^l c are written at those slots.  Returns the fused context rows c
    per sequence (for inspection)."""
    nkv, d = dims.n_kv_heads, dims.head_dim
    fused = []
    for s, F in enumerate(feats):
        n = F.shape[0]
        start = int(cache.length[s])
        if start + n > cache.k.shape[3]:
            raise ValueError("cache capacity exceeded")
        u = linear(F, _get(weights, "w_fc"))
        c = rms_norm(u, _get(weights, "fc_norm"), dims.rms_eps)
        pos = np.arange(start, start + n) + pos_offset
        for l, lw in enumerate(_get(weights, "layers")):
            k = linear(c, lw["wk"]).reshape(n, nkv, d)
            v = linear(c, lw["wv"]).reshape(n, nkv, d)
            k = rope(k, pos, dims.rope_theta)
            cache.k[l, s, :, start:start + n, :] = k.transpose(1, 0, 2)
            cache.v[l, s, :, start:start + n, :] = v.transpose(1, 0, 2)
        cache.length[s] = start + n
        fused.append(c)
    return fused


def draft_forward(dims, weights, cache: OracleCache, last_tok: np.ndarray,
                  keep_logits: bool = False, pos_offset: int = 0) -> Dict[str, np.ndarray]:
    """One block-diffusion drafting pass ([Report/KP], [Term/WF] stage two).

    The block holds the last accepted token followed by B-1 mask tokens at
    positions len_s .. len_s + B - 1.  Each layer: RMSNorm, q/k/v
    projections, RoPE on q and k, attention over the injected context K/V of
    that layer followed by the block's own K/V (no mask), output projection
    and residual, RMSNorm, SwiGLU MLP and residual.  A final RMSNorm and the
    shared lm_head give logits whose lowest-index argmax is the drafted
    token of each slot.

    Returns tokens [b, B], gaps [b, B], per-layer attention outputs
    (pre-projection, [L][b, B, n_q*d]), the residual after the attention
    half and after each full layer, and the final normed hidden."""
    last_tok = np.asarray(last_tok, dtype=np.int64)
    toks = np.full((last_tok.shape[0], dims.block_size), dims.mask_id, dtype=np.int64)
    toks[:, 0] = last_tok
    return draft_block(dims, weights, cache, toks, keep_logits, pos_offset)


def draft_anchors(dims, weights, cache: OracleCache, anchor_seq, anchor_pos, anchor_tok,
                  keep_logits: bool = False) -> Dict[str, np.ndarray]:
    """Drafting passes over blocks with explicit anchors ([Term/WF] stage
    one: anchor positions at the decoding frontier and at additional points
    when several blocks are drafted concurrently).

    Block a belongs to cached sequence anchor_seq[a]; its anchor position
    p = anchor_pos[a] is the number of that sequence's cached positions it
    sees, so slot 0 holds anchor_tok[a] at position p, the mask slots follow
    at p + 1 .. p + B - 1, and attention covers cached positions [0, p) and
    the block's own slots.  A block anchored at the frontier (p equal to the
    cached length) is the ordinary drafting pass.  Blocks are independent of
    one another; several may share a sequence.  Returns the draft_forward
    outputs stacked over blocks."""
    outs = []
    for a in range(len(anchor_tok)):
        s, p = int(anchor_seq[a]), int(anchor_pos[a])
        if not 0 <= p <= int(cache.length[s]):
            raise ValueError("an anchor lies beyond its sequence's cached positions")
        view = OracleCache(cache.k[:, s:s + 1], cache.v[:, s:s + 1], np.array([p], dtype=np.int64))
        outs.append(draft_forward(dims, weights, view, np.array([anchor_tok[a]]), keep_logits))
    res: Dict[str, np.ndarray] = {}
    for key in outs[0]:
        if isinstance(outs[0][key], list):
            res[key] = [np.concatenate([o[key][l] for o in outs], axis=0) for l in range(len(outs[0][key]))]
        else:
            res[key] = np.concatenate([o[key] for o in outs], axis=0)
    return res


def draft_block(dims, weights, cache: OracleCache, toks: np.ndarray,
                keep_logits: bool = False, pos_offset: int = 0) -> Dict[str, np.ndarray]:
    """The drafting pass over an arbitrary block of token ids [b, B]
    (``draft_forward`` supplies [last token, mask, ..., mask])."""
    toks = np.asarray(toks, dtype=np.int64)
    b, B = toks.shape
    H, nq, nkv, d = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    embed = _get(weights, "embed")
    layers = _get(weights, "layers")
    h = np.asarray(embed[toks.reshape(-1)], dtype=np.float64).reshape(b, B, H)
    attn_outs, mids, hiddens = [], [], [h.copy()]
    for l, lw in enumerate(layers):
        a = rms_norm(h, lw["attn_norm"], dims.rms_eps)
        q = linear(a, lw["wq"]).reshape(b, B, nq, d)
        k = linear(a, lw["wk"]).reshape(b, B, nkv, d)
        v = linear(a, lw["wv"]).reshape(b, B, nkv, d)
        o = np.empty((b, B, nq, d))
        for s in range(b):
            C = int(cache.length[s])
            pos = np.arange(C, C + B) + pos_offset
            qs = rope(q[s], pos, dims.rope_theta)
            ks = rope(k[s], pos, dims.rope_theta)
            keys = np.concatenate([cache.k[l, s, :, :C, :].transpose(1, 0, 2), ks], axis=0)
            vals = np.concatenate([cache.v[l, s, :, :C, :].transpose(1, 0, 2), v[s]], axis=0)
            o[s] = attention(qs, keys, vals)
        o = o.reshape(b, B, nq * d)
        attn_outs.append(o)
        h = h + linear(o, lw["wo"])
        mids.append(h.copy())
        a = rms_norm(h, lw["mlp_norm"], dims.rms_eps)
        act = silu(linear(a, lw["w_gate"])) * linear(a, lw["w_up"])
        h = h + linear(act, lw["w_down"])
        hiddens.append(h.copy())
    z = rms_norm(h, _get(weights, "final_norm"), dims.rms_eps)
    logits = linear(z, _get(weights, "lm_head"))
    tokens, gaps = argmax_lowest(logits)
    out = {"tokens": tokens, "gaps": gaps, "attn_out": attn_outs, "mid": mids,
           "hidden": hiddens, "final": z}
    if keep_logits:
        out["logits"] = logits
    return out


def verify(dims, lm_head: np.ndarray, target_hidden: np.ndarray):
    """Target argmax at every block row ([Term/WF] stage three).

    target_hidden is the target's final (post-norm) hidden state at the
    B + 1 rows of its pass over [x, d_0 .. d_{B-1}], shape [b, B+1, H].
    Returns the lowest-index argmax [b, B+1] and the top-1/top-2 gaps."""
    th = np.asarray(target_hidden, dtype=np.float64)
    logits = linear(th, lm_head)
    return argmax_lowest(logits)



# ------------------------------------------------------- temperature sampling

def gumbel(u: np.ndarray) -> np.ndarray:
    """Gumbel noise -log(-log u) of uniforms u in (0, 1)."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u))


def sample_categorical(log_weights: np.ndarray, u: np.ndarray):
    """A draw from the distribution proportional to exp(log_weights) along
    the last axis, by the Gumbel-max property: the lowest-index argmax of
    log_weights + gumbel(u).  Entries with weight 0 carry -inf.  Returns the
    index and the top-1/top-2 gap of the perturbed values."""
    return argmax_lowest(np.asarray(log_weights, dtype=np.float64) + gumbel(u))


def log_softmax(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    return x - m - np.log(np.exp(x - m).sum(axis=-1, keepdims=True))


def draft_sample(dims, weights, cache: OracleCache, last_tok, temperature: float, u):
    """The drafting pass with each slot's token drawn from the drafter's
    distribution q_j = softmax(l_j / T) ([Term/WF] stage two: the masked
    positions are filled with sampled tokens).  u: uniforms [b, B, V].
    Returns the draft_forward outputs plus "tokens" / "gaps" of the sampled
    draw and the logits."""
    dr = draft_forward(dims, weights, cache, last_tok, keep_logits=True)
    tok, gaps = sample_categorical(dr["logits"] / float(temperature), u)
    dr["tokens"], dr["gaps"] = tok, gaps
    return dr


def speculative_verify(draft, q_logits, p_logits, temperature: float, u_accept, u_resid):
    """Speculative-sampling verification ([Term/WF] stage three: each
    drafted token is checked against the target by an acceptance criterion,
    the accepted prefix is emitted and the target supplies the next token).

    Reading of the criterion: the standard speculative-sampling rule.  With
    q_j = softmax(q_logits_j / T) (drafter) and p_j = softmax(p_logits_j / T)
    (target), drafted token d_j is accepted when u_accept_j <= p_j(d_j) /
    q_j(d_j), slot by slot; at the first rejected slot j the next token is
    drawn from max(0, p_j - q_j) (normalised), and after B accepted slots
    from p_B.  Draws use sample_categorical with u_resid.

    draft [b, B], q_logits [b, B, V], p_logits [b, B+1, V], u_accept [b, B],
    u_resid [b, V].  Returns (accept_len [b], next_tok [b], margins [b]: the
    smallest |log(p/q) - log u| over the decisions taken, and gaps [b]: the
    top-1/top-2 gap of the final draw)."""
    draft = np.asarray(draft)
    b, B = draft.shape
    L = np.zeros(b, dtype=np.int64)
    nxt = np.zeros(b, dtype=np.int64)
    margins = np.full(b, np.inf)
    gaps = np.zeros(b)
    T = float(temperature)
    for s in range(b):
        lq = log_softmax(np.asarray(q_logits[s], dtype=np.float64) / T)
        lp = log_softmax(np.asarray(p_logits[s], dtype=np.float64) / T)
        j = 0
        while j < B:
            d = int(draft[s, j])
            diff = (lp[j, d] - lq[j, d]) - np.log(float(u_accept[s, j]))
            margins[s] = min(margins[s], abs(diff))
            if diff >= 0.0:
                j += 1
            else:
                break
        if j < B:
            w = np.maximum(0.0, np.exp(lp[j]) - np.exp(lq[j]))
            with np.errstate(divide="ignore"):
                logw = np.where(w > 0.0, np.log(np.where(w > 0.0, w, 1.0)), -np.inf)
        else:
            logw = lp[B]
        t, gap = sample_categorical(logw, u_resid[s])
        L[s], nxt[s], gaps[s] = j, int(t), float(gap)
    return L, nxt, margins, gaps


# ----------------------------------------------------- target verify pass

def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, C: int) -> np.ndarray:
    """Softmax attention of n new queries over C cached keys followed by
    the n new keys, causal over the new ones: query i (position C + i) sees
    keys 0 .. C + i.  q: [n, n_q, d]; k, v: [C + n, n_kv, d]; grouped K/V
    heads as in ``attention``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, nq, d = q.shape
    group = nq // k.shape[1]
    out = np.empty_like(q)
    for i in range(n):
        T = C + i + 1
        for h in range(nq):
            g = h // group
            s = (k[:T, g, :] @ q[i, h, :]) / np.sqrt(d)
            p = np.exp(s - s.max())
            out[i, h, :] = (p / p.sum()) @ v[:T, g, :]
    return out


def target_feature_layers(n_layers: int, n_feat: int) -> List[int]:
    """Reading of which target layers feed the drafter: n_feat layers spread
    evenly through the depth, the residual stream after layer
    floor((k + 1) * n_layers / (n_feat + 1)) (1-based) for k = 0 .. n_feat - 1,
    returned 0-based."""
    return [(k + 1) * n_layers // (n_feat + 1) - 1 for k in range(n_feat)]


def target_forward(tdims, tweights, cache: OracleCache, tokens, feat_layers, parents=None) -> Dict[str, np.ndarray]:
    """The target's causal pass over n new tokens per sequence ([Term/WF]
    stage three: the target computes its own logits at every block position;
    [Report/KP]: the drafter is conditioned on hidden features from several
    target layers).

    The target is read as a decoder of the drafter's layer type (RMSNorm,
    q/k/v with RoPE, grouped attention, o_proj and residual, RMSNorm, SwiGLU
    and residual) with causal attention.  tokens [b, n] sit at positions
    C_s .. C_s + n - 1 (C_s the cached length); their K/V are written to the
    cache at those positions, the cached length is left as it was (the
    caller commits the accepted rows).  With parents [b, n] (a draft tree,
    parents[s][0] = -1, parents before children) row i is a tree node: its
    rotary position is C_s + depth(i) and it sees the cached positions and
    its ancestors and itself only (the ancestor-only mask of the DDTree
    paragraph); without, the rows form a chain (causal).  Returns the final normalised hidden
    states "hidden" [b, n, H] (what the verify head multiplies by W_lm), the
    features [b, n, len(feat_layers) * H] (the residual stream after each
    listed layer, layer-major) and the residual after every layer."""
    tokens = np.asarray(tokens, dtype=np.int64)
    b, n = tokens.shape
    H, nq, nkv, d = tdims.hidden, tdims.n_q_heads, tdims.n_kv_heads, tdims.head_dim
    h = np.asarray(_get(tweights, "embed")[tokens.reshape(-1)], dtype=np.float64).reshape(b, n, H)
    resid = []
    for l, lw in enumerate(_get(tweights, "layers")):
        a = rms_norm(h, lw["attn_norm"], tdims.rms_eps)
        q = linear(a, lw["wq"]).reshape(b, n, nq, d)
        k = linear(a, lw["wk"]).reshape(b, n, nkv, d)
        v = linear(a, lw["wv"]).reshape(b, n, nkv, d)
        o = np.empty((b, n, nq, d))
        for s in range(b):
            C = int(cache.length[s])
            if C + n > cache.k.shape[3]:
                raise ValueError("cache capacity exceeded")
            pos = np.arange(C, C + n)
            if parents is not None:
                par = np.asarray(parents[s])
                depth = np.zeros(n, dtype=np.int64)
                for i in range(1, n):
                    depth[i] = depth[par[i]] + 1
                pos = C + depth
            qs = rope(q[s], pos, tdims.rope_theta)
            ks = rope(k[s], pos, tdims.rope_theta)
            cache.k[l, s, :, C:C + n, :] = ks.transpose(1, 0, 2)
            cache.v[l, s, :, C:C + n, :] = v[s].transpose(1, 0, 2)
            keys = cache.k[l, s, :, :C + n, :].transpose(1, 0, 2)
            vals = cache.v[l, s, :, :C + n, :].transpose(1, 0, 2)
            if parents is None:
                o[s] = causal_attention(qs, keys, vals, C)
            else:
                o[s] = masked_attention(qs, keys, vals, C, tree_mask(parents[s]))
        h = h + linear(o.reshape(b, n, nq * d), lw["wo"])
        a = rms_norm(h, lw["mlp_norm"], tdims.rms_eps)
        h = h + linear(silu(linear(a, lw["w_gate"])) * linear(a, lw["w_up"]), lw["w_down"])
        resid.append(h.copy())
    feats = [resid[l] for l in feat_layers]
    z = rms_norm(h, _get(tweights, "final_norm"), tdims.rms_eps)
    features = np.concatenate(feats, axis=-1) if feats else np.zeros((b, n, 0))
    return {"hidden": z, "features": features, "residual": resid}


def commit(cache: OracleCache, accept_len) -> None:
    """After verification the accepted prefix and the target's own next
    token stay in the target cache: the cached length grows by L + 1."""
    cache.length += np.asarray(accept_len, dtype=np.int64) + 1


# ------------------------------------------------------------ draft trees

def topk_logprobs(logits: np.ndarray, K: int):
    """The K most probable tokens of each row (highest log-softmax first,
    lowest index on ties) and their log-probabilities.  logits [..., V]."""
    lp = log_softmax(logits)
    order = np.argsort(-lp, axis=-1, kind="stable")[..., :K]
    return order.astype(np.int64), np.take_along_axis(lp, order, axis=-1)


def build_tree(draft_logits: np.ndarray, anchor: int, K: int, N: int):
    """A draft tree from the drafter's per-position distributions by a
    best-first heap ([Forum] the DDTree paragraph: multiple continuations
    from per-position distributions, selected best-first, verified in one
    target pass).

    Reading: the block's slots are drafted independently in one pass, so a
    continuation t_1 .. t_k (slot j proposing the (j+1)-th token after the
    anchor) scores sum_j log q_j(t_j); the tree holds the N continuations of
    highest score over the top-K tokens of each slot.  Every prefix scores
    at least as much as its extensions, so these form a tree rooted at the
    anchor.  The heap pops continuations in score order; after popping
    (prefix, token of rank r at depth k) it pushes the prefix's next sibling
    (rank r + 1) and the popped node's first child (rank 0 at depth k + 1).
    Ties go to the smaller depth, then the smaller ranks.

    draft_logits [B, V].  Returns node tokens [N+1] (node 0 the anchor),
    parents [N+1] (-1 for the root), depths [N+1] and scores [N+1]; nodes
    are numbered in pop order, so a parent precedes its children."""
    import heapq
    B = draft_logits.shape[0]
    tok, lp = topk_logprobs(draft_logits, K)
    tokens, parent, depth, score = [int(anchor)], [-1], [0], [0.0]
    ranks = [()]
    heap = [(-float(lp[0, 0]), 1, (0,), 0)]        # (-score, depth, ranks, parent node)
    while heap and len(tokens) < N + 1:
        neg, dep, rk, par = heapq.heappop(heap)
        node = len(tokens)
        tokens.append(int(tok[dep - 1, rk[-1]]))
        parent.append(par)
        depth.append(dep)
        score.append(-neg)
        ranks.append(rk)
        if rk[-1] + 1 < K:                          # next sibling
            heapq.heappush(heap, (-(score[par] + float(lp[dep - 1, rk[-1] + 1])), dep, rk[:-1] + (rk[-1] + 1,), par))
        if dep < B:                                 # first child
            heapq.heappush(heap, (-(-neg + float(lp[dep, 0])), dep + 1, rk + (0,), node))
    return (np.array(tokens, dtype=np.int64), np.array(parent, dtype=np.int64),
            np.array(depth, dtype=np.int64), np.array(score))


def tree_mask(parent) -> np.ndarray:
    """allowed[i, j]: node j is node i or one of its ancestors."""
    n = len(parent)
    allowed = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            allowed[i, j] = True
            j = int(parent[j])
    return allowed


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, C: int, allowed: np.ndarray) -> np.ndarray:
    """Attention of n new queries over C cached keys (all seen) and the n
    new keys, new key j seen by query i where allowed[i, j].  Causal
    attention is the lower-triangular case."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, nq, d = q.shape
    group = nq // k.shape[1]
    out = np.empty_like(q)
    for i in range(n):
        keys = np.concatenate([np.arange(C), C + np.nonzero(allowed[i])[0]])
        for h in range(nq):
            g = h // group
            s = (k[keys, g, :] @ q[i, h, :]) / np.sqrt(d)
            p = np.exp(s - s.max())
            out[i, h, :] = (p / p.sum()) @ v[keys, g, :]
    return out


def tree_accept(tokens, parent, target_argmax):
    """Greedy acceptance over a tree ([Term/WF] stages three and four):
    from the root, follow the child whose token is the target's argmax at
    the current node (the lowest-numbered such child), as long as there is
    one.  Returns the accepted length L (the depth reached), the fallback
    token (the target's argmax at the last accepted node) and the path of
    nodes [0, n_1, .., n_L]."""
    node, path = 0, [0]
    while True:
        g = int(target_argmax[node])
        kids = [c for c in range(len(tokens)) if int(parent[c]) == node and int(tokens[c]) == g]
        if not kids:
            break
        node = kids[0]
        path.append(node)
    return len(path) - 1, int(target_argmax[node]), np.array(path, dtype=np.int64)


def commit_path(cache: OracleCache, seq: int, path) -> None:
    """Keep a tree pass's accepted path in the target cache: the K/V rows of
    path node k (written at slot C + node) move to C + k, and the cached
    length grows by len(path)."""
    C = int(cache.length[seq])
    rows = C + np.asarray(path, dtype=np.int64)
    cache.k[:, seq, :, C:C + len(path)] = cache.k[:, seq][:, :, rows].copy()
    cache.v[:, seq, :, C:C + len(path)] = cache.v[:, seq][:, :, rows].copy()
    cache.length[seq] = C + len(path)
