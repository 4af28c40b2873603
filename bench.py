#!/usr/bin/env python3
"""Benchmark of one DFlash draft-and-verify step on one MI355X.

A step is the whole hot path for one batch: KV injection of the newly
accepted rows, the drafting pass over a B = 16 block and greedy verification
with acceptance.  The default workload is the Qwen3-8B-shaped drafter at
batch 1 with a 2048-position injected context.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--extras LIST | --no-extras]

Prints one JSON line.  Inputs are seeded and synthetic; weights are random
with the drafter's shapes.  Every step first rewinds ctx_len to the
configured context, so each timed step runs at the same shape.  After the
headline workload, the other measured workloads (batch 32 with ragged
contexts, batch 4 over 16384 cached positions, and the hidden-5120 drafter
at block sizes 4, 8 and 16) are timed in the same run and reported under
"workloads" in the same line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
EV_EVERY = 10                  # timed steps per sampled verify-head launch
VERIFY_PROBES = 16             # bracketed verify-only launches after the timed region
# Cost model of the speedup ("Term: DFlash speculative decoding", section
# "Mathematical view of acceptance and speedup": S ~ C_AR * E[L] / C_DF).
# The target itself is not built here: its pass is modeled as streaming the
# bf16 weights of an 8-billion-parameter model (the pages' Qwen3-8B) once at
# the HBM rate the verify head measures in the same run.
TARGET_PARAMS = 8.0e9
# The oracle leg repeats whole steps until this much host time (at most
# CPU_SAMPLE_MAX steps; at least one).
CPU_SAMPLE_S = 10.0
CPU_SAMPLE_MAX = 20
# Calibrated HBM bytes of the verify head per workload, with the kernel
# sources they were measured on (files that name no sources were taken on
# the skinny GEMM's).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_verify_head_{}.md")
TRAFFIC_SOURCES = ["gemm.hip", "gemm_util.hpp", "common.hpp", "kernels.hpp", "api.hip"]
# The library's routing rule for the heads (a CPU test pins both sides of
# it): skinny up to HEAD_TILED_MIN_ROWS rows while two row tiles of
# activations fit the registers (k chunks of at most 16 tiles of 32 bf16
# columns per wavefront, i.e. hidden <= 4096), else up to STEP_TILED_MIN_ROWS.
HEAD_TILED_MIN_ROWS = 32
STEP_TILED_MIN_ROWS = 17
# Workloads timed after the headline one: (name, block size), fewer steps.
EXTRAS = [("qwen3-8b-b32", 16), ("qwen3-8b-long", 16), ("larger-b8", 4), ("larger-b8", 8),
          ("larger-b8", 16)]
EXTRA_STEPS, EXTRA_WARMUP = 10, 3
# Workloads that also time a temperature-1 step (sampled drafting and
# speculative-sampling verification).
SAMPLING_WORKLOADS = ("qwen3-8b-b1", "qwen3-8b-b32")
# Multi-anchor drafting and the block-size policy are timed at batch 1.
ANCHOR_WORKLOADS = ("qwen3-8b-b1",)
ANCHOR_BLOCKS = (1, 2, 4, 8)
POLICY_BLOCKS = (4, 8, 16)
# Workloads that also time the 36-layer target's verify pass and an
# autoregressive target step (the measured cost model).
TARGET_WORKLOADS = ("qwen3-8b-b1", "qwen3-8b-b32")


def time_graph(args, torch, b: int, rewind, run, outs):
    """The same step captured once in a HIP graph and replayed: warmup
    replays, then `steps` timed replays.  The replays' outputs must equal the
    eager step's (the step is deterministic)."""
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rewind()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rewind()
        run()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    ms = g0.elapsed_time(g1) / args.steps
    match = all(bool(torch.equal(o, r)) for o, r in zip(outs, ref))
    return {"ms_per_step": round(ms, 4), "value": round(b * 1000.0 / ms, 2), "outputs_match": match}


def measured_traffic(workload: str):
    """HBM bytes per verify-head launch from the committed FETCH_SIZE /
    WRITE_SIZE counter summary of this workload, if there is one and the
    kernel sources it lists are the ones it was measured on; else None."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    import hashlib
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "sources", "sources_sha256"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in vals.get("sources", " ".join(TRAFFIC_SOURCES)).split():
        with open(os.path.join(ROOT, "block_diffusion_speculative_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("sources_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_model(d, batch, ctx, rows):
    """Algorithmic HBM bytes and flops of one step.  Weights are counted once
    per step, except the lm_head, which the draft head and the verify head
    each stream (a target pass lies between them).  The K/V projection
    weights of injection are the drafter's own and are counted once."""
    es = 2 if d.dtype == "bf16" else 4
    H, I, V, hd = d.hidden, d.intermediate, d.vocab, d.head_dim
    nqd = d.n_q_heads * hd
    per_layer = (d.qkv_rows * H + H * nqd + 2 * I * H + H * I)
    w_bytes = (H * d.feat_dim + d.n_layers * per_layer + 2 * V * H) * es
    ctx_after = np.asarray(ctx) + np.asarray(rows)
    kv_read = int(np.sum(ctx_after)) * d.n_layers * 2 * d.n_kv_heads * hd * es
    kv_write = int(np.sum(rows)) * d.n_layers * 2 * d.n_kv_heads * hd * es
    io = int(np.sum(rows)) * d.feat_dim * es + batch * (d.block_size + 1) * H * es
    B = d.block_size
    M = batch * B
    R = int(np.sum(rows))
    flops = 2 * (R * H * d.feat_dim + R * H * d.n_layers * 2 * d.n_kv_heads * hd)
    flops += 2 * M * d.n_layers * per_layer + 2 * M * V * H + 2 * batch * (B + 1) * V * H
    flops += sum(4 * d.n_q_heads * B * (int(c) + B) * hd * d.n_layers for c in ctx_after)
    return {"bytes": w_bytes + kv_read + kv_write + io, "weight_bytes": w_bytes,
            "kv_bytes": kv_read + kv_write, "flops": flops}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def head_kernel_label(lm_rows: int, hidden: int = 4096) -> str:
    """The kernels that run the verify head at this many rows and this bf16
    hidden size (the library's skinny/tiled routing rule)."""
    k_tiles = (hidden + 31) // 32
    limit = HEAD_TILED_MIN_ROWS if (k_tiles + 7) // 8 <= 16 else STEP_TILED_MIN_ROWS
    if lm_rows > limit:
        return ("gemm_tiled_kernel<bf16, ARGMAX> + argmax_finish_kernel "
                "(verify lm_head + argmax, then the accept scan)")
    return "gemm_kernel<bf16, ARGMAX> (verify lm_head + argmax + accept)"


def copy_ceiling(torch, dev, mib: int = 1024, reps: int = 5):
    """HBM rate of a plain device copy of `mib` MiB (read + write bytes over
    the mean HIP-event time of `reps` copies): a measured ceiling beside the
    8 TB/s nameplate."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"GBs": round(2 * n / (ms * 1e-3) / 1e9, 1), "bytes_moved": 2 * n, "ms": round(ms, 4),
            "method": f"torch copy_ of {mib} MiB on the device, read + write bytes / mean event time of {reps}"}


def time_sampling(torch, dr, b, B, V, feats_t, cu, R, last_t, th, rewind, steps, greedy_ms):
    """The same step at temperature 1: inject, sampled drafting
    (dflash_draft_sample) and speculative-sampling verification
    (dflash_verify_sample), the uniforms drawn on the device beforehand
    (seeded inputs).  Returns its time per step next to the greedy one."""
    dev = dr.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    grid = float(1 << 24)
    unif = lambda *shape: (torch.randint(0, 1 << 24, shape, device=dev, generator=gen).float() + 0.5) / grid
    u_draft, u_acc, u_res = unif(b * B, V), unif(b, B), unif(b, V)
    dlog = torch.empty((b * B, V), dtype=torch.float32, device=dev)
    tlog = torch.empty((b * (B + 1), V), dtype=torch.float32, device=dev)
    out = torch.empty((b, B), dtype=torch.int32, device=dev)
    al = torch.empty(b, dtype=torch.int32, device=dev)
    nx = torch.empty(b, dtype=torch.int32, device=dev)

    def step():
        rewind()
        dr.inject(feats_t, cu, b, R)
        dr.draft_sample(last_t, 1.0, u_draft, out, dlog, b)
        dr.verify_sample(th, out, dlog, 1.0, u_acc, u_res, tlog, al, nx, b)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"temperature": 1.0, "ms_per_step": round(ms, 4), "value": round(b * 1000.0 / ms, 2),
            "unit": "block-steps/s", "vs_greedy_step": round(ms / greedy_ms, 4), "steps": steps,
            "mean_accept_len": float(al.float().mean().item()),
            "note": "inject + dflash_draft_sample + dflash_verify_sample; logits of both heads in HBM "
                    "(fp32), uniforms generated on the device before timing; includes one rewind of the "
                    "context lengths per step"}


def time_anchors(torch, dr, d, b, ctx, last, steps):
    """Drafting over several anchored blocks of one sequence per call
    (dflash_draft_anchors): the frontier block and blocks anchored 16, 32,
    ... positions before it, each attending to the context before its anchor.
    Every block of a call shares the one weight stream, so the pass time grows
    far slower than the block count."""
    dev = dr.device
    es = 2 if d.dtype == "bf16" else 4
    H, hd, V = d.hidden, d.head_dim, d.vocab
    per_layer = (d.qkv_rows * H + H * d.n_q_heads * hd + 3 * d.intermediate * H) * es
    out = {}
    for A in ANCHOR_BLOCKS:
        if A > dr.max_blocks:
            continue
        pos = [int(ctx[0]) - 16 * a for a in range(A)]
        seq_t = torch.zeros(A, dtype=torch.int32, device=dev)
        pos_t = torch.as_tensor(np.asarray(pos, dtype=np.int32)).to(dev)
        tok_t = torch.full((A,), int(last[0]), dtype=torch.int32, device=dev)
        o = torch.empty((A, d.block_size), dtype=torch.int32, device=dev)
        for _ in range(3):
            dr.draft_anchors(seq_t, pos_t, tok_t, o, A)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            dr.draft_anchors(seq_t, pos_t, tok_t, o, A)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        byts = d.n_layers * per_layer + V * H * es + sum(pos) * d.n_layers * 2 * d.n_kv_heads * hd * es
        out[str(A)] = {"ms_per_call": round(ms, 4), "blocks_per_s": round(A * 1000.0 / ms, 1),
                       "drafted_tokens_per_s": round(A * d.block_size * 1000.0 / ms, 1),
                       "algorithmic_bytes": int(byts),
                       "hbm_frac": round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
    return {"blocks": out, "anchors": "sequence 0; the frontier and anchors 16, 32, ... positions before it",
            "note": "one dflash_draft_anchors call per timed pass (embedding, 5 layers, draft head with argmax); "
                    "bytes = the drafter's layer weights and W_lm once plus each block's context K/V"}


def time_block_policy(torch, dr, d, b, rows, feats_t, last_t, th, rewind, p_acc, seed, steps):
    """Adaptive block size: the whole step (inject + draft + verify) timed at
    each candidate B (injecting min(n, B + 1) rows per sequence, the most a
    step of that size commits), then the policy's choice from the planted
    accept lengths of 64 steps at B = 16."""
    from block_diffusion_speculative_amd import inputs as I
    from block_diffusion_speculative_amd.policy import BlockSizePolicy, expected_accept
    dev = dr.device
    Bmax = d.block_size
    cu_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    times = {}
    for Bc in POLICY_BLOCKS:
        if Bc > Bmax:
            continue
        r_b = np.minimum(rows, Bc + 1)
        idx = np.concatenate([np.arange(cu_h[s], cu_h[s] + r_b[s]) for s in range(b)])
        f_b = feats_t[torch.as_tensor(idx).to(dev)].contiguous()
        cu_b = torch.as_tensor(np.concatenate([[0], np.cumsum(r_b)]).astype(np.int32)).to(dev)
        R_b = int(np.sum(r_b))
        th_b = th[:, :Bc + 1].contiguous()
        o = torch.empty((b, Bc), dtype=torch.int32, device=dev)
        tg = torch.empty((b, Bc + 1), dtype=torch.int32, device=dev)
        al = torch.empty(b, dtype=torch.int32, device=dev)
        bo = torch.empty(b, dtype=torch.int32, device=dev)

        def step():
            rewind()
            dr.inject(f_b, cu_b, b, R_b)
            dr.draft(last_t, o, b, block_size=Bc)
            dr.verify(th_b, o, tg, al, bo, b, block_size=Bc)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        times[Bc] = e0.elapsed_time(e1) / steps
    pol = BlockSizePolicy(times, prior_steps=0.0)
    for k in range(64):
        pol.observe_many(I.planted_accept(seed, 1000 + k, b, p_acc, Bmax), Bmax)
    p_hat = pol.p_hat()
    per_b = {str(Bc): {"ms_per_step": round(t, 4),
                       "committed_tokens_per_s": round(b * (expected_accept(p_acc, Bc) + 1.0) * 1000.0 / t, 1)}
             for Bc, t in times.items()}
    return {"per_block_size": per_b, "p_planted": round(p_acc, 5), "p_estimated": round(p_hat, 5),
            "chosen_block_size": pol.choose(),
            "note": "committed tokens/s = batch x (E[min(G, B)] + 1) / step time at the planted geometric p; "
                    "the choice maximises the same rate at the p estimated from 64 planted steps at B = 16; "
                    "each step includes one rewind of the context lengths"}


def device_target_weights(torch, td, seed, dev):
    """Seeded random target weights generated on the device (bf16 values of
    N(0, 0.02^2) draws, unit gains): the 36-layer target is only timed, and
    host generation of its seven billion values would dominate the run."""
    from block_diffusion_speculative_amd.inputs import TargetWeights
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    H, d, I_, V = td.hidden, td.head_dim, td.intermediate, td.vocab
    rn = lambda *shape: (torch.randn(shape, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    ones = lambda: torch.ones(H, device=dev, dtype=torch.bfloat16)
    layers = [{"attn_norm": ones(), "wq": rn(td.n_q_heads * d, H), "wk": rn(td.n_kv_heads * d, H),
               "wv": rn(td.n_kv_heads * d, H), "wo": rn(H, td.n_q_heads * d), "mlp_norm": ones(),
               "w_gate": rn(I_, H), "w_up": rn(I_, H), "w_down": rn(H, I_)} for _ in range(td.n_layers)]
    return TargetWeights(embed=rn(V, H), final_norm=ones(), layers=layers)


def time_target(torch, dr, d, b, ctx, B, verify_bytes, step_ms, e_l, steps):
    """The target's side of a decode step, measured: its causal verify pass
    over the B + 1 block rows (dflash_target_forward) and an autoregressive
    step (the same pass over one row followed by the lm_head argmax, the
    verify call at block size 1).  Then the pages' speedup model S ~ C_AR E /
    C_DF ("Term: DFlash speculative decoding", "Mathematical view of
    acceptance and speedup") on measured costs: C_AR the autoregressive step,
    C_DF this draft step plus the target's verify pass."""
    from block_diffusion_speculative_amd import configs as C
    from block_diffusion_speculative_amd.engine import Target
    td = C.QWEN3_8B_TARGET
    dev = dr.device
    t0 = time.time()
    cap = C.kv_capacity(int(np.max(ctx)) + 32)
    # workspace for the 17-row verify pass and the 32-node tree pass
    tg = Target(td, device_target_weights(torch, td, 77, dev), b, cap, max_rows=32, device=dev)
    shape = (td.n_layers, b, td.n_kv_heads, cap, td.head_dim)
    gen = torch.Generator(device=dev)
    gen.manual_seed(78)
    kv = [(torch.randn(shape, device=dev, generator=gen) * 1.28).to(torch.bfloat16) for _ in range(2)]
    tg.kv_import(kv[0], kv[1])
    del kv
    tg.set_ctx_len(ctx)
    feat_layers = [(k + 1) * td.n_layers // (td.n_feat_layers + 1) - 1 for k in range(td.n_feat_layers)]
    toks = torch.randint(0, td.vocab - 1, (b, B + 1), device=dev, generator=gen, dtype=torch.int32)
    hid = torch.empty((b, B + 1, td.hidden), dtype=torch.bfloat16, device=dev)
    feats = torch.empty((b, B + 1, td.n_feat_layers * td.hidden), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] target (36 layers) set up in {time.time() - t0:.1f}s")

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # the pass leaves ctx_len alone, so every repetition runs at the same shape
    t_verify_pass = timed(lambda: tg.forward(toks, b, B + 1, feat_layers, hid, feats))
    t_one = timed(lambda: tg.forward(toks[:, :1].contiguous(), b, 1, [], hid[:, :1], None))
    th2 = hid[:, :2].contiguous()
    d2 = torch.zeros((b, 1), dtype=torch.int32, device=dev)
    ta = torch.empty((b, 2), dtype=torch.int32, device=dev)
    al = torch.empty(b, dtype=torch.int32, device=dev)
    bo = torch.empty(b, dtype=torch.int32, device=dev)
    t_head = timed(lambda: dr.verify(th2, d2, ta, al, bo, b, block_size=1))
    # a DDTree step's device work: the draft tree (drafting pass with its
    # logits, top-4 per slot, 31 nodes best-first), the target's pass over
    # the 32 tree nodes, the walk and the path commit
    K, N = 4, 31
    dlog = torch.empty((b * B, d.vocab), dtype=torch.float32, device=dev)
    tt = torch.empty((b, N + 1), dtype=torch.int32, device=dev)
    tp = torch.empty((b, N + 1), dtype=torch.int32, device=dev)
    thid = torch.empty((b, N + 1, td.hidden), dtype=torch.bfloat16, device=dev)
    tfeat = torch.empty((b, N + 1, td.n_feat_layers * td.hidden), dtype=torch.bfloat16, device=dev)
    tta = torch.empty((b, N + 1), dtype=torch.int32, device=dev)
    tpath = torch.empty((b, N + 1), dtype=torch.int32, device=dev)
    last = torch.zeros(b, dtype=torch.int32, device=dev)
    t_tree_draft = timed(lambda: dr.draft_tree(last, K, N, dlog, tt, tp, b))
    t_tree_pass = timed(lambda: tg.forward(tt, b, N + 1, feat_layers, thid, tfeat, parents=tp))
    t_tree_accept = timed(lambda: dr.tree_accept(thid, tt, tp, b, N + 1, tta, al, bo, tpath))
    status = tg.read_status()
    del tg
    torch.cuda.empty_cache()
    H, I_ = td.hidden, td.intermediate
    layer_bytes = ((td.n_q_heads + 2 * td.n_kv_heads) * td.head_dim * H + H * td.n_q_heads * td.head_dim
                   + 3 * I_ * H) * 2
    kv_bytes = int(np.sum(ctx) + b * (B + 1)) * td.n_layers * 2 * td.n_kv_heads * td.head_dim * 2
    pass_bytes = td.n_layers * layer_bytes + kv_bytes
    c_ar = t_one + t_head
    c_df = step_ms + t_verify_pass
    return {
        "target": "Qwen3-8B-shaped: the drafter's layer type, 36 layers, hidden 4096, 32/8 heads, "
                  "intermediate 12288, shared lm_head; seeded random weights",
        "verify_pass_ms": round(t_verify_pass, 4), "verify_pass_rows": B + 1,
        "verify_pass_GBs": round(pass_bytes / (t_verify_pass * 1e-3) / 1e9, 1),
        "verify_pass_hbm_frac": round(pass_bytes / (t_verify_pass * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "verify_pass_algorithmic_bytes": pass_bytes,
        "ar_step_ms": round(c_ar, 4), "ar_pass_one_row_ms": round(t_one, 4), "lm_head_argmax_ms": round(t_head, 4),
        "C_AR_ms": round(c_ar, 4), "C_DF_ms": round(c_df, 4),
        "S_with_E_L": round(c_ar * e_l / c_df, 3), "S_with_E_L_plus_bonus": round(c_ar * (e_l + 1) / c_df, 3),
        "E_L_planted": round(e_l, 4), "status": status,
        "ddtree_step": {"topk": K, "nodes": N + 1, "draft_tree_ms": round(t_tree_draft, 4),
                        "target_tree_pass_ms": round(t_tree_pass, 4), "tree_accept_ms": round(t_tree_accept, 4),
                        "note": "the drafting pass with its logits, top-K and the best-first build; the 36-layer "
                                "target over the tree nodes under the ancestor mask; lm_head argmax and walk"},
        "source": "S = C_AR * E / C_DF, C_AR = one-row target pass + lm_head argmax, "
                  "C_DF = draft step + the target's (B+1)-row verify pass, all measured",
    }


def run_workload(args, torch, name: str, block: int, steps: int, warmup: int, cpu_leg: str):
    """Times one workload: `warmup` untimed steps, then `steps` timed ones
    (inject + draft + verify with acceptance).  cpu_leg: "full" runs whole
    oracle steps of the workload for the CPU baseline, "one" one sequence of
    it, "" none.  Returns the result dict."""
    from block_diffusion_speculative_amd import configs as C
    from block_diffusion_speculative_amd import inputs as I
    from block_diffusion_speculative_amd.engine import Drafter, upload

    w = C.get(name)
    d = w.dims.with_block(block) if block else w.dims
    B = d.block_size
    b = w.batch
    seed = args.seed
    t0 = time.time()
    weights = I.make_weights(d, seed)
    log(f"[bench] {name} B={B}: weights generated in {time.time() - t0:.1f}s")
    ctx = I.context_lengths(w, seed)
    if w.new_rows is not None:
        rows = I.new_row_counts(w, seed, 0)
    else:
        # a step commits at most B + 1 rows (B accepted drafts and the fallback token)
        rows = np.full(b, min(int(round(w.mean_accept)) + 1, B + 1), dtype=np.int32)
    cap = C.kv_capacity(int(ctx.max()))
    p_acc = I.workload_geom_p(w)

    # Context K/V generated directly (seeded bf16 values), one step of injection on top.
    shape = (d.n_layers, b, d.n_kv_heads, cap, d.head_dim)
    k_plain = np.zeros(shape, dtype=np.float32)
    v_plain = np.zeros(shape, dtype=np.float32)
    for l in range(d.n_layers):
        for s in range(b):
            ks, vs = I.kv_entries(d, seed, l, s, int(ctx[s]))
            k_plain[l, s, :, :ctx[s]] = ks
            v_plain[l, s, :, :ctx[s]] = vs
    feats = [I.features(d, seed, 0, s, int(rows[s])) for s in range(b)]
    last = I.last_tokens(d, seed, 0, b)
    L_plant = I.planted_accept(seed, 0, b, p_acc, B)

    cpu = None
    oracle_tokens = None
    oracle_gaps = None
    oseqs = list(range(b)) if cpu_leg == "full" else ([0] if cpu_leg == "one" else [])
    if oseqs:
        import oracle.dflash_oracle as O
        # Whole oracle steps (inject, draft, verify, accept) on a fresh copy
        # of the context each time, repeated until about CPU_SAMPLE_S seconds
        # of work; the copies and the planted verify targets (input recipe,
        # not the method) stay outside the timed parts.
        log(f"[bench] oracle steps on the host ({len(oseqs)} of {b} sequences) ...")
        secs = []
        while not secs or (sum(secs) < CPU_SAMPLE_S and len(secs) < CPU_SAMPLE_MAX):
            cache = O.OracleCache(k_plain[:, oseqs].astype(np.float64), v_plain[:, oseqs].astype(np.float64),
                                  ctx[oseqs].astype(np.int64).copy())
            tc = time.perf_counter()
            O.inject(d, weights, cache, [feats[s] for s in oseqs])
            dr = O.draft_forward(d, weights, cache, last[oseqs])
            t_draft = time.perf_counter() - tc
            oracle_tokens, oracle_gaps = dr["tokens"], dr["gaps"]
            all_tok = I.stream(seed, 99, 0).integers(0, d.vocab - 1, size=(b, B))
            all_tok[oseqs] = oracle_tokens
            t_plant, hid = I.planted_targets(d, seed, 0, weights.lm_head, all_tok, L_plant)
            tc = time.perf_counter()
            g, _ = O.verify(d, weights.lm_head, hid[oseqs])
            O.accept(oracle_tokens, g)
            secs.append(t_draft + time.perf_counter() - tc)
            del cache
        osec = float(np.mean(secs))
        cpu = {"value": len(oseqs) / osec, "unit": "block-steps/s",
               "cores": int(max(blas_threads(), 1)),
               "affinity_cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "seconds_per_step": osec,
               "sample": (f"{len(secs)} full steps of the same workload ({name}: inject "
                          f"{int(np.sum(rows))} rows, draft, verify, accept)"
                          if cpu_leg == "full" else
                          f"{len(secs)} steps of sequence 0 of the {b}-sequence workload ({name}: "
                          f"inject {int(rows[0])} rows, draft, verify, accept); block-steps/s of that one sequence")
                         + f", fp64 numpy, {sum(secs):.1f} s in all, mean per step"}
        log(f"[bench] oracle steps: {len(secs)} x {osec:.2f}s")
    else:
        all_tok = I.stream(seed, 99, 0).integers(0, d.vocab - 1, size=(b, B))
        t_plant, hid = I.planted_targets(d, seed, 0, weights.lm_head, all_tok, L_plant)

    dev = torch.device("cuda:0")
    t0 = time.time()
    n4 = getattr(args, "anchor_steps", 0) > 0 and name in ANCHOR_WORKLOADS and not block
    dr_gpu = Drafter(d, weights, b, cap, int(max(17 * b, np.sum(rows))), device=dev,
                     max_blocks=max(ANCHOR_BLOCKS) if n4 else 0)
    dr_gpu.kv_import(upload(k_plain.reshape(-1, d.head_dim), dr_gpu.dt, dev).reshape(shape),
                     upload(v_plain.reshape(-1, d.head_dim), dr_gpu.dt, dev).reshape(shape))
    del k_plain, v_plain
    log(f"[bench] device setup in {time.time() - t0:.1f}s")
    ctx0 = torch.as_tensor(ctx).to(dev)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)).to(dev)
    R = int(np.sum(rows))
    feats_t = upload(np.concatenate(feats, axis=0), dr_gpu.dt, dev)
    last_t = torch.as_tensor(last).to(dev)
    th = upload(hid.reshape(b * (B + 1), d.hidden), dr_gpu.dt, dev).reshape(b, B + 1, d.hidden)
    draft_out = torch.empty((b, B), dtype=torch.int32, device=dev)
    tgt = torch.empty((b, B + 1), dtype=torch.int32, device=dev)
    acc = torch.empty(b, dtype=torch.int32, device=dev)
    bonus = torch.empty(b, dtype=torch.int32, device=dev)
    # Every step must start from the configured context lengths, so the
    # workload stays fixed.  Each timed step gets its own copy of the lengths,
    # made before the timed region (the injection appends at the same
    # positions every step, and only the lengths it commits differ), so the
    # timed region holds the step's launches only.  Warm-up steps and graph
    # replays roll the drafter's own lengths back instead (a uniform length is
    # one fill, a ragged one a copy).
    ctx_uniform = int(ctx[0]) if bool(np.all(ctx == ctx[0])) else None
    # The verify head is bracketed by a pair of events on every EV_EVERY-th
    # timed step: an event record is a barrier packet on the stream (about
    # 6 us here), so bracketing every step would add ~12 us of instrumentation
    # to each.  The sampled steps stay inside the timed region.
    ev_idx = list(range(0, steps, EV_EVERY))
    ev_v0 = {i: torch.cuda.Event(enable_timing=True) for i in ev_idx}
    ev_v1 = {i: torch.cuda.Event(enable_timing=True) for i in ev_idx}

    def rewind():
        if ctx_uniform is not None:
            dr_gpu.ctx_len[:b].fill_(ctx_uniform)
        else:
            torch.add(ctx0, 0, out=dr_gpu.ctx_len[:b])

    ctx_fresh = torch.zeros((steps, dr_gpu.ckv.max_batch), dtype=torch.int32, device=dev)
    ctx_fresh[:, :b] = ctx0.to(torch.int32)

    def step(i=None):
        if i is None:
            rewind()
        else:
            dr_gpu.bind_ctx_len(ctx_fresh[i])
        dr_gpu.inject(feats_t, cu, b, R)
        dr_gpu.draft(last_t, draft_out, b)
        timed = i is not None and i in ev_v0
        if timed:
            ev_v0[i].record()
        dr_gpu.verify(th, draft_out, tgt, acc, bonus, b)
        if timed:
            ev_v1[i].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    dr_gpu.bind_ctx_len(None)
    ms_total = e0.elapsed_time(e1)
    graph_res = None
    if args.graph:
        graph_res = time_graph(args, torch, b, rewind, lambda: (dr_gpu.inject(feats_t, cu, b, R),
                                                               dr_gpu.draft(last_t, draft_out, b),
                                                               dr_gpu.verify(th, draft_out, tgt, acc, bonus, b)),
                               [draft_out, tgt, acc, bonus])
    ms_step = ms_total / steps
    verify_in_region = [ev_v0[i].elapsed_time(ev_v1[i]) for i in ev_idx]
    # More samples of the same launch (same inputs, same stream), right after
    # the timed region, so the in-region brackets stay few.
    pv0 = [torch.cuda.Event(enable_timing=True) for _ in range(VERIFY_PROBES)]
    pv1 = [torch.cuda.Event(enable_timing=True) for _ in range(VERIFY_PROBES)]
    for i in range(VERIFY_PROBES):
        pv0[i].record()
        dr_gpu.verify(th, draft_out, tgt, acc, bonus, b)
        pv1[i].record()
    torch.cuda.synchronize()
    verify_samples = verify_in_region + [a.elapsed_time(e) for a, e in zip(pv0, pv1)]
    verify_ms = float(np.mean(verify_samples))

    measured_cost = None
    if getattr(args, "target_steps", 0) > 0 and name in TARGET_WORKLOADS:
        e_l_target = I.geometric_mean_accept(I.workload_geom_p(w), B)
        measured_cost = time_target(torch, dr_gpu, d, b, ctx, B, None, ms_step, e_l_target, args.target_steps)
    sampled = None
    if getattr(args, "sampling_steps", 0) > 0 and name in SAMPLING_WORKLOADS:
        sampled = time_sampling(torch, dr_gpu, b, B, d.vocab, feats_t, cu, R, last_t, th, rewind,
                                args.sampling_steps, ms_step)
    anchors = policy = None
    if n4:
        anchors = time_anchors(torch, dr_gpu, d, b, ctx, last, args.anchor_steps)
        policy = time_block_policy(torch, dr_gpu, d, b, rows, feats_t, last_t, th, rewind, p_acc, seed,
                                   args.anchor_steps)
    status = dr_gpu.read_status()
    got_draft = draft_out.cpu().numpy()
    got_acc = acc.cpu().numpy()
    parity = None
    if oseqs:
        want, gaps, got = oracle_tokens.reshape(-1), oracle_gaps.reshape(-1), got_draft[oseqs].reshape(-1)
        above = gaps > 1e-2
        parity = {"sequences": len(oseqs), "compared": int(above.sum()), "below_gap": int((~above).sum()),
                  "mismatched_above_gap": int(np.sum(got[above] != want[above])),
                  "equal_below_gap": int(np.sum(got[~above] == want[~above])),
                  "rule": "drafted tokens bit-exact where the oracle's top-1/top-2 gap exceeds 1e-2"}
    del dr_gpu
    torch.cuda.empty_cache()

    model = step_model(d, b, ctx, rows)
    es = 2 if d.dtype == "bf16" else 4
    lm_bytes = d.vocab * d.hidden * es + b * (B + 1) * d.hidden * es + b * (B + 3) * 4
    lm_rows = b * (B + 1)
    lm_flops = 2 * lm_rows * d.vocab * d.hidden
    # The verify head's own bound: HBM when streaming W_lm takes longer than
    # its MFMA work at peak (few rows), MFMA otherwise.
    lm_t_hbm = lm_bytes / (HBM_PEAK_GBS * 1e9)
    lm_t_mfma = lm_flops / (BF16_PEAK_TFLOPS * 1e12)
    lm_kernel = head_kernel_label(lm_rows, d.hidden)
    traffic_key = name if not block or block == max(w.block_sizes) else f"{name}-B{block}"
    if lm_t_mfma > lm_t_hbm:
        ach = lm_flops / (verify_ms * 1e-3) / 1e12
        lm_roof = {"kernel": lm_kernel, "bound": "mfma", "achieved": round(ach, 1),
                   "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                   "traffic": measured_traffic(traffic_key),
                   "flops_per_launch": lm_flops, "bytes_per_launch": lm_bytes}
    else:
        ach = lm_bytes / (verify_ms * 1e-3) / 1e9
        lm_roof = {"kernel": lm_kernel, "bound": "hbm", "achieved": round(ach, 1),
                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(traffic_key),
                   "bytes_per_launch": lm_bytes, "flops_per_launch": lm_flops}
    lm_roof.update({"avg_launch_ms": round(verify_ms, 5), "launches_sampled": len(verify_samples),
                    "in_region_avg_ms": round(float(np.mean(verify_in_region)), 5),
                    "in_region_samples": len(verify_in_region),
                    "min_launch_ms": round(min(verify_samples), 5),
                    "timing": f"HIP event pairs on the launch stream around every {EV_EVERY}th timed "
                              f"step's verify call and around {VERIFY_PROBES} verify calls right after "
                              "the timed region"})
    step_gbs = model["bytes"] / (ms_step * 1e-3) / 1e9
    t_hbm = model["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = model["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    t_roof = max(t_hbm, t_mfma)
    value = b * 1000.0 / ms_step
    # S = C_AR * E / C_DF: C_AR is one autoregressive target step, C_DF one
    # draft-and-verify step (this step plus the target's verify pass over the
    # block), E the tokens a step commits on average: E[L] of the planted
    # acceptance, and E[L] + 1 with the fallback token.
    t_target_ms = TARGET_PARAMS * 2 / (lm_bytes / (verify_ms * 1e-3)) * 1e3
    e_l = I.geometric_mean_accept(p_acc, B)
    c_df = ms_step + t_target_ms
    cost = {"source": "S = C_AR * E / C_DF with C_AR = t_target, C_DF = t_step + t_target",
            "t_step_ms": round(ms_step, 4),
            "t_target_ms_modeled": round(t_target_ms, 4),
            "target": f"{TARGET_PARAMS:.0e} bf16 parameters streamed at the verify head's measured rate",
            "E_L_planted": round(e_l, 4),
            "S_with_E_L": round(t_target_ms * e_l / c_df, 3),
            "S_with_E_L_plus_bonus": round(t_target_ms * (e_l + 1) / c_df, 3)}
    return {
        "metric": f"draft+verify block-steps/s (B={B})",
        "value": round(value, 2),
        "unit": "block-steps/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "dtype": d.dtype,
        "config": {"workload": name, "batch": b, "ctx": [int(c) for c in ctx] if b <= 4 else
                   {"min": int(ctx.min()), "max": int(ctx.max()), "mean": float(ctx.mean())},
                   "block": B, "injected_rows": int(R), "hidden": d.hidden, "layers": d.n_layers,
                   "vocab": d.vocab},
        "drafted_tokens_per_s": round(value * B, 1),
        "step_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                          "algorithmic_bytes": model["bytes"], "flops": model["flops"],
                          "t_roofline_ms": round(t_roof * 1e3, 4),
                          "frac": round(t_roof * 1e3 / ms_step, 4),
                          "achieved_GBs": round(step_gbs, 1),
                          "achieved_TFLOPs": round(model["flops"] / (ms_step * 1e-3) / 1e12, 1)},
        "roofline": lm_roof,
        "cpu_baseline": cpu,
        "cost_model": cost,
        "cost_model_measured": measured_cost,
        "graph": graph_res,
        "wall_s_timed": round(wall, 4),
        # Targets are planted against the oracle's drafted tokens; without the
        # oracle leg they are planted against random tokens (accept ~ 0), which
        # leaves the verify head's work unchanged.
        "accept": {"mean_len": float(np.mean(got_acc)), "planted_mean": float(np.mean(L_plant)),
                   "planted_against": "oracle draft" if cpu_leg == "full" else
                   ("oracle draft (sequence 0), random tokens elsewhere" if cpu_leg == "one" else "random tokens")},
        "draft_parity": parity,
        "sampling_T1": sampled,
        "multi_anchor": anchors,
        "block_policy": policy,
        "status": status,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3-8b-b1")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--block-size", type=int, default=0, metavar="B",
                    help="block size B of the step (one of the workload's sweep sizes; default its largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (reported under 'graph')")
    ap.add_argument("--calibrate-copy", type=int, default=1024, metavar="MIB",
                    help="size of the timed plain device copy (a measured HBM ceiling; the reference "
                         "dispatch for HBM byte counters); 0 skips it")
    ap.add_argument("--sampling-steps", type=int, default=10,
                    help="timed temperature-1 steps on the batch-1 and batch-32 workloads (0: none)")
    ap.add_argument("--target-steps", type=int, default=10,
                    help="timed passes of the 36-layer target on the batch-1 and batch-32 workloads (0: none)")
    ap.add_argument("--anchor-steps", type=int, default=10,
                    help="timed multi-anchor drafting passes and block-size policy steps per size on the "
                         "batch-1 workload (0: none)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline workload only")
    ap.add_argument("--extras", default="",
                    help="comma-separated NAME[:B] workloads to time after the headline one "
                         "(default: batch 32, long context and the hidden-5120 B sweep)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the draft-and-verify step of a batch runs on one "
              "device, and this build has no multi-GPU path (sequences shard across GPUs with "
              "no exchange; see the design notes).  Run with --gpus 1.", file=sys.stderr)
        return 2

    from block_diffusion_speculative_amd import configs as C
    w = C.get(args.workload)
    if args.block_size and args.block_size not in w.block_sizes:
        log(f"block size {args.block_size} is not swept on {args.workload} (sizes {w.block_sizes})")
        return 2
    if args.no_extras:
        extras = []
    elif args.extras:
        extras = []
        for item in args.extras.split(","):
            nm, _, bs = item.partition(":")
            extras.append((nm, int(bs) if bs else 0))
    else:
        extras = [e for e in EXTRAS if not (e[0] == args.workload and e[1] in (args.block_size, 0))]

    import torch
    from block_diffusion_speculative_amd import _lib

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    _lib.load()
    fresh = _lib.is_fresh()
    if not fresh:
        log("[bench] WARNING: libdflash.so was built from other sources than the ones in the tree")
    dev = torch.device("cuda:0")
    ceiling = copy_ceiling(torch, dev, args.calibrate_copy) if args.calibrate_copy > 0 else None
    head = run_workload(args, torch, args.workload, args.block_size, args.steps, args.warmup,
                        "" if args.no_cpu_baseline else "full")
    out = {
        "metric": head["metric"],
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded random weights of the drafter's shapes; seeded context K/V, features and planted targets)",
    }
    out.update({k: v for k, v in head.items() if k not in out})
    out["hbm_copy_ceiling"] = ceiling
    out["library_fresh"] = fresh
    res = {}
    for nm, bs in extras:
        key = nm if not bs or bs == max(C.get(nm).block_sizes) else f"{nm}-B{bs}"
        # the batch-32 line carries an oracle leg of one sequence
        leg = "one" if (nm == "qwen3-8b-b32" and not args.no_cpu_baseline) else ""
        r = run_workload(args, torch, nm, bs, EXTRA_STEPS, EXTRA_WARMUP, leg)
        for k in ("graph", "steps", "warmup", "dtype", "unit"):
            r.pop(k, None)
        res[key] = r
        log(f"[bench] {key}: {r['ms_per_step']} ms/step, {r['value']} block-steps/s, "
            f"step roofline {r['step_roofline']['frac']}")
    if res:
        out["workloads"] = res
        out["workloads_timing"] = f"{EXTRA_WARMUP} warm-up and {EXTRA_STEPS} timed steps each"
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
