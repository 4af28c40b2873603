"""Precision budget of the drafting pass: which activations may be rounded
to a single bf16 plane (a script, not a test; run on the CPU).

    python tests/precision_budget.py [--seeds 0,1,2] [--workload qwen3-8b-b1]

It repeats the oracle's drafting pass in fp64 with the GPU path's roundings
applied at chosen points, each either exact, a single bf16 plane, or a hi +
lo pair of bf16 planes (x = hi + lo, about 16 mantissa bits), and prints the
per-row relative errors of the attention outputs and of the residual stream
against the exact oracle, and every drafted token that flips while the
oracle's top-1/top-2 gap exceeds 1e-2.  (An error the whole-row norm
keeps small can still be large in one head: the GPU tests also bound the
error of every 128-channel segment, which a single-plane QKV input exceeds
at the batch-1 shape, 2.15% at layer 4, so every GEMM input stays two
planes.)  The rounding points are the inputs
of the QKV, o_proj, gate/up and down projections, the block's q (hi + lo in
the attention), the block's own K/V (always one plane, as in the cache), the
attention probabilities P, and the final normalised hidden state that the
draft head reads (one plane).  The numbers behind the GPU path's choice of
planes come from this script.
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle.dflash_oracle as O  # noqa: E402
from block_diffusion_speculative_amd import configs as C  # noqa: E402
from block_diffusion_speculative_amd import inputs as I  # noqa: E402
import harness as Hn  # noqa: E402


def to_bf16(x):
    y = np.asarray(x, dtype=np.float32).copy()
    I.round_bf16_(y)
    return y.astype(np.float64)


def rnd(x, mode):
    """'x': exact; 'b': one bf16 plane; 'h': hi + lo bf16 planes of the
    fp32 value (what the GPU stores)."""
    if mode == "x":
        return np.asarray(x, np.float64)
    x32 = np.asarray(x, np.float32).astype(np.float64)
    hi = to_bf16(x32)
    return hi if mode == "b" else hi + to_bf16(x32 - hi)


def attention_rounded(q, k, v, mq, mp):
    nq, nkv, d = q.shape[1], k.shape[1], q.shape[2]
    group = nq // nkv
    out = np.empty_like(q)
    q = rnd(q, mq)
    for h in range(nq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (rnd(p, mp) @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def draft_rounded(dims, weights, cache, toks, M):
    b, B = toks.shape
    H, nq, nkv, d = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    h = np.asarray(weights.embed[toks.reshape(-1)], np.float64).reshape(b, B, H)
    res = {"attn_out": [], "hidden": []}

    def norm_in(x, g, mode):   # the producer rounds x * g; the consumer scales by 1/rms
        ms = np.mean(x * x, axis=-1, keepdims=True)
        return rnd(x * g, mode) / np.sqrt(ms + dims.rms_eps)

    for l, lw in enumerate(weights.layers):
        a = norm_in(h, lw["attn_norm"], M["qkv"])
        q = O.linear(a, lw["wq"]).reshape(b, B, nq, d)
        k = O.linear(a, lw["wk"]).reshape(b, B, nkv, d)
        v = O.linear(a, lw["wv"]).reshape(b, B, nkv, d)
        o = np.empty((b, B, nq, d))
        for s in range(b):
            Cs = int(cache.length[s])
            pos = np.arange(Cs, Cs + B)
            ks = rnd(O.rope(k[s], pos, dims.rope_theta), "b")
            keys = np.concatenate([cache.k[l, s, :, :Cs, :].transpose(1, 0, 2), ks], 0)
            vals = np.concatenate([cache.v[l, s, :, :Cs, :].transpose(1, 0, 2), rnd(v[s], "b")], 0)
            o[s] = attention_rounded(O.rope(q[s], pos, dims.rope_theta), keys, vals, "h", M["p"])
        o = o.reshape(b, B, nq * d)
        res["attn_out"].append(o)
        h = h + O.linear(rnd(o, M["o"]), lw["wo"])
        a = norm_in(h, lw["mlp_norm"], M["gu"])
        act = O.silu(O.linear(a, lw["w_gate"])) * O.linear(a, lw["w_up"])
        h = h + O.linear(rnd(act, M["dn"]), lw["w_down"])
        res["hidden"].append(h.copy())
    z = norm_in(h, weights.final_norm, "b")
    res["tokens"], _ = O.argmax_lowest(O.linear(z, weights.lm_head))
    return res


CONFIGS = {
    "all two planes": dict(qkv="h", p="h", o="h", gu="h", dn="h"),
    "QKV input one plane": dict(qkv="b", p="h", o="h", gu="h", dn="h"),
    "QKV + o_proj inputs one plane": dict(qkv="b", p="h", o="b", gu="h", dn="h"),
    "gate/up input one plane": dict(qkv="h", p="h", o="h", gu="b", dn="h"),
    "down input one plane": dict(qkv="h", p="h", o="h", gu="h", dn="b"),
    "every GEMM input one plane": dict(qkv="b", p="h", o="b", gu="b", dn="b"),
    "everything one plane": dict(qkv="b", p="b", o="b", gu="b", dn="b"),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="qwen3-8b-b1")
    ap.add_argument("--seeds", default="0,1,2")
    args = ap.parse_args()
    w = C.get(args.workload)
    dims = w.dims
    weights = I.make_weights(dims, 0)
    ctx = [int(c) for c in I.context_lengths(w, 0)[:1]]
    for seed in [int(x) for x in args.seeds.split(",")]:
        case = Hn.build_case(dims, 1, ctx, seed=seed, kv_mode="import", weights=weights)
        cache = Hn.oracle_prefill(case, [0])
        toks = np.full((1, dims.block_size), dims.mask_id, np.int64)
        toks[0, 0] = I.last_tokens(dims, seed, 0, 1)[0]
        t0 = time.time()
        ref = O.draft_block(dims, weights, cache, toks)
        print(f"seed {seed}, context {ctx[0]} (oracle step {time.time() - t0:.1f} s)", flush=True)
        for name, M in CONFIGS.items():
            r = draft_rounded(dims, weights, cache, toks, M)
            ea = max(Hn.rel_err_rows(r["attn_out"][l], ref["attn_out"][l]) for l in range(dims.n_layers))
            eh = max(Hn.rel_err_rows(r["hidden"][l], ref["hidden"][l + 1]) for l in range(dims.n_layers))
            flips = [(i, round(float(g), 4)) for i, g in enumerate(ref["gaps"].reshape(-1))
                     if g > 1e-2 and r["tokens"].reshape(-1)[i] != ref["tokens"].reshape(-1)[i]]
            print(f"  {name:38s} attention {ea:.2e}  residual {eh:.2e}  flips above the gap {flips}", flush=True)


if __name__ == "__main__":
    main()
