"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: hidden states, attention outputs, fused context rows and cache rows
within a per-row relative error of 2e-2; token ids, accept lengths and
fallback tokens bit-exact wherever the oracle's top-1/top-2 logit gap exceeds
1e-2 (positions under the gap are counted and reported).
"""
import numpy as np
import pytest

import oracle.dflash_oracle as O
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I
import harness as Hn

pytestmark = pytest.mark.gpu

SMALL_BF16 = C.Dims(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
                    intermediate=1024, vocab=4096, n_feat_layers=3, dtype="bf16")
# Few output tiles over long k ranges: at 80-85 rows every many-row GEMM but
# the heads splits its k-tiles over workgroups (down projection 8 parts,
# fc 6, the rest 2).
SPLIT_BF16 = C.Dims(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
                    intermediate=4096, vocab=4096, n_feat_layers=3, dtype="bf16")


def _compare_step(case, step, new_rows, seqs=None, accept_p=0.12, check_cache=True):
    """Run inject + draft + verify on both sides and assert parity.  Returns a
    report dict.  check_cache: True compares every cached position of the
    followed sequences, "new" only the rows this step injected (full-size
    caches)."""
    d = case.dims
    seqs = list(range(case.batch)) if seqs is None else list(seqs)
    gpu = Hn.GpuRunner(case)
    ref = Hn.oracle_step(case, step, new_rows, seqs, accept_p)
    # GPU inject + draft
    gpu.inject(ref["feats"])
    fused = gpu.fused_view(int(np.sum(new_rows)))   # inject and draft share workspace
    got_draft = gpu.draft(ref["last"])
    views = gpu.views()
    views["fused"] = fused
    rep = {"errors": {}}
    # injected cache rows and ctx_len
    ctx_after = case.ctx + np.asarray(new_rows, dtype=np.int32)
    assert np.array_equal(gpu.ctx_len()[:case.batch], ctx_after)
    cu = np.concatenate([[0], np.cumsum(new_rows)])
    # the fused features before their RMSNorm, normalised here in fp64 and
    # compared with the oracle's fused context rows
    for i, s in enumerate(seqs):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        if rows.stop > rows.start:
            c = O.rms_norm(views["fused"][rows].astype(np.float64), case.weights.fc_norm, d.rms_eps)
            rep["errors"]["fused"] = max(rep["errors"].get("fused", 0.0), Hn.rel_err_rows(c, ref["fused"][i]))
            rep["errors"]["fused_head"] = max(rep["errors"].get("fused_head", 0.0),
                                              Hn.rel_err_heads(c, ref["fused"][i]))
    if check_cache == "new":
        # the rows this step appended, [ctx, ctx + n), of every layer and head
        # (cache rows are one head's head_dim channels each)
        for i, s in enumerate(seqs):
            lo, hi = int(case.ctx[s]), int(ctx_after[s])
            if hi == lo:
                continue
            kg, vg = gpu.kv_rows(s, lo, hi)
            ek = Hn.rel_err_rows(kg, ref["cache"].k[:, i, :, lo:hi])
            ev = Hn.rel_err_rows(vg, ref["cache"].v[:, i, :, lo:hi])
            rep["errors"]["cache_new"] = max(rep["errors"].get("cache_new", 0.0), ek, ev)
    elif check_cache:
        kg, vg = gpu.kv_plain()
        for i, s in enumerate(seqs):
            n = int(ctx_after[s])
            if n == 0:
                continue
            ek = Hn.rel_err_rows(kg[:, s, :, :n], ref["cache"].k[:, i, :, :n])
            ev = Hn.rel_err_rows(vg[:, s, :, :n], ref["cache"].v[:, i, :, :n])
            rep["errors"]["cache"] = max(rep["errors"].get("cache", 0.0), ek, ev)
    # per-layer intermediates of the chosen sequences
    B = d.block_size
    rows = np.concatenate([np.arange(s * B, (s + 1) * B) for s in seqs])
    dr = ref["draft"]
    for l in range(d.n_layers):
        pairs = {f"attn{l}": (views["attn"][l][rows], dr["attn_out"][l]),
                 f"mid{l}": (views["mid"][l][rows], dr["mid"][l]),
                 f"hidden{l}": (views["hidden"][l + 1][rows], dr["hidden"][l + 1])}
        for k, (g_, r_) in pairs.items():
            rep["errors"][k] = Hn.rel_err_rows(g_, r_)
            # per 128-channel segment (one head of the attention output)
            rep["errors"][k + "_head"] = Hn.rel_err_heads(g_, r_)
    rep["errors"]["embed"] = Hn.rel_err_rows(views["hidden"][0][rows], dr["hidden"][0])
    print({k: f"{v:.2e}" for k, v in rep["errors"].items()}, flush=True)
    for k, v in rep["errors"].items():
        assert v <= Hn.REL_TOL, (k, v, rep)
    tr = Hn.TokenReport()
    tr.add(got_draft[seqs], dr["tokens"], dr["gaps"], "draft")
    # verify on targets planted from the oracle's tokens (random stand-ins for
    # sequences the oracle did not run)
    all_tok = I.stream(case.seed, 99, step).integers(0, d.vocab - 1, size=(case.batch, B))
    all_tok[seqs] = dr["tokens"]
    t, hid = Hn.planted_verify_inputs(case, step, all_tok, ref["planted_L"])
    g_ref, vgaps = O.verify(d, case.weights.lm_head, hid[seqs])
    L_ref, bonus_ref = O.accept(dr["tokens"], g_ref)
    ta, al, bo = gpu.verify(hid, all_tok.astype(np.int32))
    tr.add(ta[seqs], g_ref, vgaps, "verify")
    # accept length and fallback token: compared where every position that
    # decides them is above the gap
    for i, s in enumerate(seqs):
        upto = min(int(L_ref[i]), B)
        decided = np.all(vgaps[i, :upto + 1] > Hn.GAP)
        if decided:
            assert al[s] == L_ref[i], (s, al[s], L_ref[i])
            assert bo[s] == bonus_ref[i], (s, bo[s], bonus_ref[i])
        assert 0 <= al[s] <= B
    assert np.array_equal(L_ref, ref["planted_L"][seqs]), "planted accept length not recovered by the oracle"
    assert not tr.mismatched, tr.mismatched
    rep["tokens"] = tr
    rep["status"] = gpu.drafter.read_status()
    assert rep["status"] == 0
    print({k: f"{v:.2e}" for k, v in rep["errors"].items() if not k.endswith("_head")},
          "worst per-head", f"{max(v for k, v in rep['errors'].items() if k.endswith('_head')):.2e}",
          "compared", tr.compared, "below_gap", tr.below_gap)
    return rep


def test_tiny_f32_step():
    w = C.get("tiny-f32")
    case = Hn.build_case(w.dims, 1, [128], seed=0)
    _compare_step(case, 0, [9], accept_p=w.geom_p)


def test_tiny_f32_ragged_batch():
    d = C.TINY_DRAFT
    case = Hn.build_case(d, 3, [1, 45, 130], seed=1)
    _compare_step(case, 0, [1, 17, 5])


def test_tiny_f32_empty_context_and_block_sizes():
    for B in (1, 4, 8):
        d = C.TINY_DRAFT.with_block(B)
        case = Hn.build_case(d, 2, [0, 33], seed=2)
        _compare_step(case, 0, [0, 3])


def test_small_bf16_step():
    case = Hn.build_case(SMALL_BF16, 2, [77, 300], seed=3)
    _compare_step(case, 0, [5, 17])


def test_batch1_inject_17_rows():
    """One sequence injecting 17 rows (a fully accepted 16-slot block plus
    its fallback token): the fc and KV-injection launches take the skinny
    kernel's 17-row variant (row 16 through LDS), as does the verify head."""
    case = Hn.build_case(SMALL_BF16, 1, [90], seed=5)
    _compare_step(case, 0, [17])


@pytest.mark.parametrize("rows", [[15, 17], [16, 17]])
def test_routing_boundaries(rows):
    """Launch sizes on both sides of the skinny/tiled switch: injections of
    32 rows (the largest on the skinny kernel) and 33 rows (tiled), at batch 2
    with 32 draft and 34 verify rows (tiled) beside the batch-1 step's 16 and
    17 (skinny) in the other tests."""
    case = Hn.build_case(SMALL_BF16, 2, [40, 9], seed=25)
    _compare_step(case, 0, rows)


def test_small_bf16_gains_and_no_rope():
    d = C.Dims(**{**SMALL_BF16.__dict__, "rope_theta": 0.0})
    case = Hn.build_case(d, 1, [64], seed=4, gain_std=0.05)
    _compare_step(case, 0, [2])


def test_small_bf16_batch5_tiled():
    """80 draft rows, 85 verify rows and 85 injected rows: every GEMM of the
    step takes the tiled (many-row) kernel, the RMSNorm scales come from
    rstd_kernel and the argmax finish runs as its own kernel."""
    case = Hn.build_case(SMALL_BF16, 5, [3, 70, 129, 200, 31], seed=9)
    _compare_step(case, 0, [17, 17, 17, 17, 17])


def test_large_vocab_batch16_big_tiles():
    """A 65536-token vocabulary: the draft head (256 rows) and the verify head
    (272 rows, a ragged last token block) run the 128 x 256 tile over many
    items per workgroup."""
    d = C.Dims(**{**SMALL_BF16.__dict__, "vocab": 65536})
    ctx = [(37 * s) % 150 for s in range(16)]
    case = Hn.build_case(d, 16, ctx, seed=12)
    _compare_step(case, 0, [(5 * s) % 17 for s in range(16)], seqs=[0, 7, 15])


@pytest.mark.parametrize("batch,vocab", [(4, 98304), (12, 4608)])
def test_head_rounds_wide_and_even(batch, vocab):
    """Head item dealing.  Batch 4 over a 98304-token vocabulary: the draft
    head (64 rows) and the verify head (68 rows) run tiles 24 fragments wide
    (256 items, one round, where 16 wide would take 384 items and two).  Batch
    12 over 4608 tokens: the verify head's 204 rows run 128 x 384 tiles, 24
    items on a 24-workgroup grid whose first four XCDs hold four items each
    for three workgroups, so one item of each goes to a workgroup of another
    XCD.  Tokens and acceptance against the oracle."""
    d = C.Dims(**{**SMALL_BF16.__dict__, "vocab": vocab})
    ctx = [(41 * s) % 120 for s in range(batch)]
    case = Hn.build_case(d, batch, ctx, seed=31)
    rep = _compare_step(case, 0, [1 + (3 * s) % 17 for s in range(batch)], seqs=[0, batch - 1])
    assert rep["tokens"].compared >= 1


def test_split_k_batch5():
    case = Hn.build_case(SPLIT_BF16, 5, [3, 70, 129, 200, 31], seed=13)
    _compare_step(case, 0, [17, 17, 17, 17, 17])


def test_max_batch64():
    """The largest batch the library takes (64 sequences: 1024 draft rows and
    1088 verify rows, every argmax key slot row in use), ragged contexts and
    injections; the oracle follows three sequences."""
    ctx = [(7 * s) % 100 for s in range(64)]
    case = Hn.build_case(SMALL_BF16, 64, ctx, seed=23)
    rep = _compare_step(case, 0, [1 + s % 17 for s in range(64)], seqs=[0, 33, 63])
    assert rep["tokens"].compared >= 1


def test_ragged_batch_longest_first():
    """A batch whose (sequence, KV head) pairs fill the compute units on their
    own (32 sequences x 8 KV heads): the block attention splits every context
    in two, and with twice as many workgroups as compute units the workgroups
    take the sequences longest context first, ties by index.  Ragged contexts
    with a tie; the oracle follows the longest, the shortest, the tied pair
    and a middle one."""
    dims = C.Dims(hidden=512, n_q_heads=16, n_kv_heads=8, head_dim=64, n_layers=2,
                  intermediate=1024, vocab=4096, n_feat_layers=3, dtype="bf16")
    ctx = [(53 * s) % 257 for s in range(32)]
    ctx[19] = ctx[7]
    order = sorted(range(32), key=lambda s: (-ctx[s], s))
    seqs = sorted({order[0], order[-1], 7, 19, order[16]})
    case = Hn.build_case(dims, 32, ctx, seed=29)
    rep = _compare_step(case, 0, [1 + s % 17 for s in range(32)], seqs=seqs)
    assert rep["tokens"].compared >= 1


def test_inject_exactly_to_capacity():
    """An injection that fills the cache to its last position is accepted
    (no status bit) and the draft reads every cached position."""
    case = Hn.build_case(SMALL_BF16, 1, [20], seed=24, capacity=32)
    _compare_step(case, 0, [12])


def test_tiny_f32_batch6_tiled():
    d = C.TINY_DRAFT
    case = Hn.build_case(d, 6, [0, 16, 17, 50, 96, 128], seed=10)
    _compare_step(case, 0, [12, 1, 17, 9, 16, 15])


@pytest.mark.parametrize("dims", ["small", "tiny"])
def test_decode_loop_four_steps(dims):
    """Four draft-and-verify steps in a row, as a decoder runs them: each
    step injects the L + 1 rows the previous one committed (the first step
    one row), drafts from the previous fallback token at the grown context,
    and verifies targets planted on the oracle's drafted tokens.  Context
    lengths follow the oracle exactly, accept lengths and fallback tokens
    wherever the positions deciding them are above the 1e-2 gap, drafted
    tokens wherever the oracle's gap exceeds 1e-2."""
    d = {"small": SMALL_BF16, "tiny": C.TINY_DRAFT}[dims]
    b, B, seed, p_acc = 2, d.block_size, 30, 0.12
    ctx0 = [40, 70]
    case = Hn.build_case(d, b, ctx0, seed=seed, capacity=C.kv_capacity(max(ctx0) + 4 * 17))
    gpu = Hn.GpuRunner(case)
    cache = Hn.oracle_prefill(case, list(range(b)))
    rows = np.ones(b, dtype=np.int64)
    last = I.last_tokens(d, seed, 0, b)
    tr = Hn.TokenReport()
    for step in range(4):
        feats = [I.features(d, seed, step + 1, s, int(rows[s])) for s in range(b)]
        gpu.inject(feats)
        O.inject(d, case.weights, cache, feats)
        assert np.array_equal(gpu.ctx_len()[:b], cache.length), (step, gpu.ctx_len()[:b], cache.length)
        got = gpu.draft(last)
        ref = O.draft_forward(d, case.weights, cache, last)
        tr.add(got, ref["tokens"], ref["gaps"], f"draft{step}")
        L_plant = I.planted_accept(seed, step, b, p_acc, B)
        _, hid = I.planted_targets(d, seed, step, case.weights.lm_head, ref["tokens"], L_plant)
        ta, al, bo = gpu.verify(hid, ref["tokens"].astype(np.int32))
        g_ref, vgaps = O.verify(d, case.weights.lm_head, hid)
        L_ref, bonus_ref = O.accept(ref["tokens"], g_ref)
        tr.add(ta, g_ref, vgaps, f"verify{step}")
        assert np.array_equal(L_ref, L_plant)
        for s_ in range(b):
            if np.all(vgaps[s_, :min(int(L_ref[s_]), B) + 1] > Hn.GAP):   # decided above the gap
                assert al[s_] == L_ref[s_] and bo[s_] == bonus_ref[s_], (step, s_, al, L_ref, bo, bonus_ref)
        # both sides go on from the oracle's commit
        rows = L_ref + 1
        last = bonus_ref.astype(np.int32)
    assert gpu.drafter.read_status() == 0
    assert not tr.mismatched, tr.mismatched
    assert tr.compared > 0
    print("compared", tr.compared, "below_gap", tr.below_gap, "ctx", cache.length)


@pytest.mark.parametrize("rows,split", [(12, 5), (20, 7)])
def test_incremental_injection_matches_single(rows, split):
    """Injecting rows in two calls equals one call (positions and append
    offsets).  Launches of up to 32 rows share one summation order, so the
    cache is bit-identical; larger launches agree to rounding."""
    d = SMALL_BF16
    case = Hn.build_case(d, 2, [0, 0], seed=5, capacity=64)
    F = [I.features(d, 5, 0, s, rows) for s in range(2)]
    a = Hn.GpuRunner(case, max_rows=2 * rows)
    a.inject(F)
    b = Hn.GpuRunner(case, max_rows=2 * rows)
    b.inject([f[:split] for f in F])
    b.inject([f[split:] for f in F])
    ka, va = a.kv_plain()
    kb, vb = b.kv_plain()
    assert np.array_equal(a.ctx_len()[:2], [rows, rows]) and np.array_equal(b.ctx_len()[:2], [rows, rows])
    if 2 * rows <= 32:
        assert np.array_equal(ka[:, :, :, :rows], kb[:, :, :, :rows])
        assert np.array_equal(va[:, :, :, :rows], vb[:, :, :, :rows])
    else:
        assert Hn.rel_err_rows(kb[:, :, :, :rows], ka[:, :, :, :rows]) < 1e-2
        assert Hn.rel_err_rows(vb[:, :, :, :rows], va[:, :, :, :rows]) < 1e-2


def test_capacity_overflow_sets_status():
    d = C.TINY_DRAFT
    case = Hn.build_case(d, 2, [0, 0], seed=6, capacity=32)
    g = Hn.GpuRunner(case, max_rows=64)
    g.inject([I.features(d, 6, 0, 0, 30), I.features(d, 6, 0, 1, 3)])
    assert np.array_equal(g.ctx_len()[:2], [30, 3])
    g.inject([I.features(d, 6, 1, 0, 3), I.features(d, 6, 1, 1, 3)])   # seq 0 would reach 33 > 32
    assert np.array_equal(g.ctx_len()[:2], [30, 6])
    assert g.drafter.read_status() & 1


def test_bad_token_sets_status():
    d = C.TINY_DRAFT
    case = Hn.build_case(d, 1, [16], seed=7)
    g = Hn.GpuRunner(case)
    g.draft(np.array([d.vocab + 5], dtype=np.int32))
    assert g.drafter.read_status() & 2


@pytest.mark.parametrize("dims,batch", [("small", 1), ("small", 2), ("split", 5)])
def test_deterministic_repeat(dims, batch):
    """Same inputs, same bits, whatever the workspace held before (batch 1:
    skinny GEMMs whose consumers reduce the norm statistics themselves;
    batch 2: 32 draft rows on the tiled kernel with rstd_kernel's per-row
    scales; batch 5 of the split configuration: split-K partial tiles summed
    in part order whichever part finishes last)."""
    d = {"small": SMALL_BF16, "split": SPLIT_BF16}[dims]
    case = Hn.build_case(d, batch, [40, 90, 7, 130, 64][:batch], seed=8)
    g = Hn.GpuRunner(case)
    last = I.last_tokens(d, 8, 0, batch)
    t1 = g.draft(last)
    v1 = g.views()
    g.drafter.ws.fill_(0xFF)   # poison scratch except the counters below
    g.drafter.ws[: 1 << 20].zero_()
    t2 = g.draft(last)
    v2 = g.views()
    assert np.array_equal(t1, t2)
    for k in ("attn", "mid", "hidden"):
        for a, b in zip(v1[k], v2[k]):
            assert np.array_equal(a, b)


@pytest.mark.slow
def test_qwen3_8b_b1_full_shape():
    """The Qwen3-8B-shaped drafter at batch 1, context 2048 (cache imported),
    one step of 9 injected rows."""
    w = C.get("qwen3-8b-b1")
    case = Hn.build_case(w.dims, 1, [2048], seed=0, kv_mode="import")
    rep = _compare_step(case, 0, [9], accept_p=I.workload_geom_p(w), check_cache="new")
    assert rep["tokens"].compared >= 1


@pytest.mark.slow
def test_qwen3_8b_b32_ragged_sampled():
    """The batch-32 ragged workload at full shape (contexts U[512, 4096],
    injected rows U[1, 17], cache imported); the oracle follows sequences 0,
    13 and 31, the GPU runs the whole batch."""
    w = C.get("qwen3-8b-b32")
    ctx = I.context_lengths(w, 0)
    rows = I.new_row_counts(w, 0, 0)
    case = Hn.build_case(w.dims, w.batch, ctx, seed=0, kv_mode="import")
    rep = _compare_step(case, 0, rows, seqs=[0, 13, 31], accept_p=I.workload_geom_p(w), check_cache="new")
    assert rep["tokens"].compared >= 1


@pytest.mark.slow
def test_qwen3_8b_long_context_sampled():
    """The long-context workload at full shape: 4 sequences of 16384 cached
    positions (imported), one injected row each; the oracle follows sequences
    0 and 3."""
    w = C.get("qwen3-8b-long")
    ctx = I.context_lengths(w, 0)
    rows = I.new_row_counts(w, 0, 0)
    case = Hn.build_case(w.dims, w.batch, ctx, seed=0, kv_mode="import")
    rep = _compare_step(case, 0, rows, seqs=[0, 3], accept_p=I.workload_geom_p(w), check_cache="new")
    assert rep["tokens"].compared >= 1


@pytest.mark.slow
@pytest.mark.parametrize("block", [4, 8, 16])
def test_larger_b8_block_sweep_sampled(block):
    """The larger drafter (hidden 5120, 40/8 heads, 8 layers, intermediate
    17408) at batch 8 over 8192 cached positions, for block sizes 4, 8 and 16;
    the oracle follows sequences 0 and 7."""
    w = C.get("larger-b8")
    d = w.dims.with_block(block)
    ctx = I.context_lengths(w, 0)
    case = Hn.build_case(d, w.batch, ctx, seed=0, kv_mode="import")
    rows = [1 + (3 * s) % block for s in range(w.batch)]
    rep = _compare_step(case, 0, rows, seqs=[0, 7], accept_p=I.workload_geom_p(w), check_cache="new")
    assert rep["tokens"].compared >= 1


@pytest.mark.parametrize("batch", [1, 5])
def test_graph_replay_matches_eager(batch):
    """One inject + draft + verify step captured in a HIP graph and replayed
    three times, with eager steps and synchronisations between the replays:
    every replay's drafted tokens, target argmax, accept lengths, fallback
    tokens and ctx_len equal the eager step's (batch 1: skinny GEMMs with the
    fused argmax and commit tails; batch 5: tiled GEMMs, split-K, rstd and
    the argmax finish kernel)."""
    import torch
    d = SPLIT_BF16 if batch == 5 else SMALL_BF16
    case = Hn.build_case(d, batch, [40, 90, 7, 130, 64][:batch], seed=14)
    g = Hn.GpuRunner(case)
    dr, dev = g.drafter, g.drafter.device
    B, H = d.block_size, d.hidden
    rows = [17] * batch
    ft = g.upload(np.concatenate([I.features(d, 14, 0, s, 17) for s in range(batch)]), dr.dt, dev)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)).to(dev)
    last = torch.as_tensor(I.last_tokens(d, 14, 0, batch).astype(np.int32)).to(dev)
    hid = I.stream(14, 99, 1).standard_normal((batch * (B + 1), H)).astype(np.float32)
    th = g.upload(hid, dr.dt, dev).reshape(batch, B + 1, H)
    ctx0 = torch.as_tensor(np.asarray(case.ctx, dtype=np.int32)).to(dev)
    out = torch.empty((batch, B), dtype=torch.int32, device=dev)
    ta = torch.empty((batch, B + 1), dtype=torch.int32, device=dev)
    al = torch.empty(batch, dtype=torch.int32, device=dev)
    bo = torch.empty(batch, dtype=torch.int32, device=dev)

    def step():
        torch.add(ctx0, 0, out=dr.ctx_len[:batch])   # a kernel, not a copy node
        dr.inject(ft, cu, batch, int(np.sum(rows)))
        dr.draft(last, out, batch)
        dr.verify(th, out, ta, al, bo, batch)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, ta, al, bo, dr.ctx_len[:batch])]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        for x in (out, ta, al, bo):
            x.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, ta, al, bo, dr.ctx_len[:batch]), ref):
            assert torch.equal(got, want)
        step()
        torch.cuda.synchronize()
        for got, want in zip((out, ta, al, bo), ref[:4]):
            assert torch.equal(got, want)


TIE_DIMS = C.Dims(**{**SMALL_BF16.__dict__, "vocab": 65536})


def _far_index(tok: int, lower: bool, vocab: int, avoid) -> int:
    """An index far from ``tok`` (another workgroup and argmax slot of the
    head): about half way down to 0 when ``lower`` (and tok >= 64), else half
    way up to the last real token; never the mask id or a member of
    ``avoid``."""
    if lower and tok >= 64:
        t = tok // 2
        while t in avoid:
            t -= 1
        return t
    t = tok + (vocab - 1 - tok) // 2
    while t in avoid or t >= vocab - 1:
        t = t + 1 if t + 1 < vocab - 1 else tok + 1
    return t


@pytest.mark.parametrize("batch", [1, 5])
def test_argmax_exact_ties_lowest_index(batch):
    """Exact ties inside both heads' top-1, built by duplicating lm_head rows
    ("Term: DFlash speculative decoding", "DFlash: architecture and
    workflow": the drafted token and the target's token are each an argmax;
    ties go to the lowest index).  A duplicated row gives bit-identical
    logits on both sides, so the tied positions are compared bit-exactly with
    no gap exemption.  Batch 1 runs the skinny heads (fused finish), batch 5
    the tiled heads and argmax_finish_kernel; the 65536-token vocabulary puts
    the two rows of a pair in different workgroups and argmax slots, with the
    lower index first in some pairs and second in others."""
    d = TIE_DIMS
    seed = 40 + batch
    ctx = [31 + 29 * s for s in range(batch)]
    case = Hn.build_case(d, batch, ctx, seed=seed)
    W = case.weights
    feats, last = Hn.step_inputs(case, 0, [1] * batch)
    cache0 = Hn.oracle_prefill(case, list(range(batch)))
    O.inject(d, W, cache0, feats)
    toks0 = O.draft_forward(d, W, cache0, last)["tokens"]
    # draft ties: duplicate the rows of distinct drafted tokens, half of them
    # to a lower index (the argmax moves there) and half to a higher one
    lm = W.lm_head.copy()
    avoid = set(int(t) for t in toks0.reshape(-1)) | {d.mask_id}
    draft_pairs = {}
    vals, counts = np.unique(toks0.reshape(-1), return_counts=True)
    by_count = [int(v) for v in vals[np.argsort(-counts, kind="stable")] if int(v) != d.mask_id]
    for i, tok in enumerate(by_count[:6]):
        t2 = _far_index(tok, i % 2 == 0, d.vocab, avoid)
        lm[t2] = lm[tok]
        draft_pairs[tok] = t2
        avoid.add(t2)
    W.lm_head = lm
    cache1 = Hn.oracle_prefill(case, list(range(batch)))
    O.inject(d, W, cache1, feats)
    dr = O.draft_forward(d, W, cache1, last)
    # every constructed pair that is some slot's top-1 is an exact tie there
    tied_draft = np.zeros_like(dr["tokens"], dtype=bool)
    for tok, t2 in draft_pairs.items():
        hit = (toks0 == tok)
        assert np.all(dr["tokens"][hit] == min(tok, t2))
        assert np.all(dr["gaps"][hit] == 0.0)
        tied_draft |= hit
    assert tied_draft.sum() >= 2 and any(t2 < tok for tok, t2 in draft_pairs.items()
                                         if np.any(toks0 == tok))
    # verify ties: planted targets on the oracle's tokens; the rows of a few
    # targets past the accepted prefix get a duplicate too
    L_plant = I.planted_accept(seed, 0, batch, 0.15, d.block_size)
    t, _ = I.planted_targets(d, seed, 0, W.lm_head, dr["tokens"], L_plant)
    verify_pairs = {}
    for s in range(batch):
        for j in range(int(L_plant[s]) + 1, d.block_size + 1, 3):
            tok = int(t[s, j])
            if tok in avoid or tok in verify_pairs:
                continue
            t3 = _far_index(tok, (s + j) % 2 == 0, d.vocab, avoid | {tok})
            lm[t3] = lm[tok]
            verify_pairs[tok] = t3
            avoid |= {tok, t3}
    W.lm_head = lm
    # the draft does not see the new pairs (neither row is any slot's top-1)
    assert np.array_equal(O.draft_forward(d, W, cache1, last)["tokens"], dr["tokens"])
    t, hid = I.planted_targets(d, seed, 0, W.lm_head, dr["tokens"], L_plant)
    g_ref, vgaps = O.verify(d, W.lm_head, hid)
    L_ref, bonus_ref = O.accept(dr["tokens"], g_ref)
    tied_verify = np.isin(t, list(draft_pairs) + list(draft_pairs.values())
                          + list(verify_pairs) + list(verify_pairs.values()))
    assert np.all(vgaps[tied_verify] == 0.0) and tied_verify.sum() >= 2
    # GPU on the same (modified) weights
    gpu = Hn.GpuRunner(case)
    gpu.inject(feats)
    got = gpu.draft(last)
    ta, al, bo = gpu.verify(hid, dr["tokens"].astype(np.int32))
    assert np.array_equal(got[tied_draft], dr["tokens"][tied_draft]), (got, dr["tokens"])
    assert np.array_equal(ta[tied_verify], g_ref[tied_verify]), (ta, g_ref)
    tr = Hn.TokenReport()
    tr.add(got, dr["tokens"], dr["gaps"], "draft")
    tr.add(ta, g_ref, vgaps, "verify")
    assert not tr.mismatched, tr.mismatched
    # accept length and fallback token: decided by positions that are above
    # the gap or constructed ties
    for s in range(batch):
        upto = min(int(L_ref[s]), d.block_size)
        ok = (vgaps[s, :upto + 1] > Hn.GAP) | tied_verify[s, :upto + 1]
        if np.all(ok):
            assert al[s] == L_ref[s] and bo[s] == bonus_ref[s], (s, al, L_ref, bo, bonus_ref)
    print("tied draft slots", int(tied_draft.sum()), "tied verify rows", int(tied_verify.sum()),
          "compared", tr.compared, "below_gap", tr.below_gap)


def test_deterministic_injection_two_row_tiles():
    """A 24-row injection (two row tiles on the skinny kernel, whose
    consumer reduces the RMSNorm tile sums itself) writes the same cache bits
    again after the workspace outside its counter area is poisoned."""
    d = SMALL_BF16
    case = Hn.build_case(d, 2, [0, 0], seed=26, capacity=64)
    F = [I.features(d, 26, 0, s, 12) for s in range(2)]
    g = Hn.GpuRunner(case, max_rows=24)
    g.inject(F)
    k1, v1 = g.kv_plain()
    g.drafter.set_ctx_len([0, 0])
    g.drafter.ws.fill_(0xFF)
    g.drafter.ws[: 1 << 20].zero_()
    g.inject(F)
    k2, v2 = g.kv_plain()
    assert np.array_equal(g.ctx_len()[:2], [12, 12])
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def _compare_anchors(case, gpu, anchors, seed, check_views=True):
    """Anchored drafting (dflash_draft_anchors) against the oracle's
    draft_anchors on the case's cache: tokens under the gap rule, and the
    per-layer attention outputs and residuals of every block."""
    import torch
    d = case.dims
    seq = np.array([a[0] for a in anchors], dtype=np.int32)
    pos = np.array([a[1] for a in anchors], dtype=np.int32)
    tok = np.array([a[2] for a in anchors], dtype=np.int32)
    n = len(anchors)
    cache = Hn.oracle_prefill(case, list(range(case.batch)))
    ref = O.draft_anchors(d, case.weights, cache, seq, pos, tok)
    dev = gpu.drafter.device
    out = torch.full((n, d.block_size), -1, dtype=torch.int32, device=dev)
    t = lambda a: torch.as_tensor(a).to(dev)
    gpu.drafter.draft_anchors(t(seq), t(pos), t(tok), out, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tr = Hn.TokenReport()
    tr.add(got, ref["tokens"], ref["gaps"], "anchors")
    assert not tr.mismatched, tr.mismatched
    errs = {}
    if check_views:
        from block_diffusion_speculative_amd import _lib
        M = n * d.block_size
        for l in range(d.n_layers):
            ga = gpu.drafter.view(_lib.VIEW_ATTN, n, l).reshape(M, -1).cpu().numpy()
            gh = gpu.drafter.view(_lib.VIEW_HIDDEN, n, l).reshape(M, -1).cpu().numpy()
            ra = ref["attn_out"][l].reshape(M, -1)
            rh = ref["hidden"][l + 1].reshape(M, -1)
            errs[f"attn{l}"] = max(Hn.rel_err_rows(ga, ra), Hn.rel_err_heads(ga, ra))
            errs[f"hidden{l}"] = max(Hn.rel_err_rows(gh, rh), Hn.rel_err_heads(gh, rh))
        for k, v in errs.items():
            assert v <= Hn.REL_TOL, (k, v, errs)
    assert gpu.drafter.read_status() == 0
    print({k: f"{v:.2e}" for k, v in errs.items()}, "compared", tr.compared, "below_gap", tr.below_gap)
    return tr


def test_anchored_blocks_small():
    """Blocks with explicit anchors: the frontier of each sequence, two
    candidate anchor tokens at one frontier, earlier anchors (position 0,
    inside a key step, on a step boundary) and a block over an empty prefix;
    7 blocks over 2 cached sequences (112 draft rows: the tiled path)."""
    d = SMALL_BF16
    case = Hn.build_case(d, 2, [100, 301], seed=33)
    gpu = Hn.GpuRunner(case, max_blocks=7)
    anchors = [(0, 100, 17), (1, 301, 500), (1, 301, 2048), (1, 150, 9), (1, 64, 9), (0, 0, 77), (0, 37, 3000)]
    _compare_anchors(case, gpu, anchors, 33)


def test_anchored_single_block_skinny():
    """One anchored block (16 rows: the skinny path) at an earlier position
    equals the oracle's drafting over that prefix."""
    d = SMALL_BF16
    case = Hn.build_case(d, 1, [200], seed=34)
    gpu = Hn.GpuRunner(case)
    _compare_anchors(case, gpu, [(0, 123, 42)], 34)


def test_anchor_outside_cache_sets_status():
    import torch
    d = C.TINY_DRAFT
    case = Hn.build_case(d, 1, [20], seed=35)
    g = Hn.GpuRunner(case)
    dev = g.drafter.device
    out = torch.empty((1, d.block_size), dtype=torch.int32, device=dev)
    t = lambda a: torch.as_tensor(np.array(a, dtype=np.int32)).to(dev)
    g.drafter.draft_anchors(t([0]), t([25]), t([3]), out, 1)      # beyond the 20 cached positions
    torch.cuda.synchronize()
    assert g.drafter.read_status() & 4
    g.drafter.clear_status()
    g.drafter.draft_anchors(t([5]), t([10]), t([3]), out, 1)      # no such sequence
    torch.cuda.synchronize()
    assert g.drafter.read_status() & 4


@pytest.mark.slow
def test_anchored_blocks_qwen3_8b_full_shape():
    """The Qwen3-8B-shaped drafter over one 2048-position cache (imported):
    four blocks (64 rows) anchored at the frontier with two tokens, at 1000
    and at 2047."""
    w = C.get("qwen3-8b-b1")
    case = Hn.build_case(w.dims, 1, [2048], seed=36, kv_mode="import")
    gpu = Hn.GpuRunner(case, max_blocks=4)
    tr = _compare_anchors(case, gpu, [(0, 2048, 11), (0, 2048, 70000), (0, 1000, 11), (0, 2047, 5)], 36)
    assert tr.compared >= 16


def test_decode_loop_block_size_per_step():
    """Adaptive block size: a decode loop whose block size changes every
    step (16, 4, 8, 16, 1) on one drafter, cache and workspace, each step
    compared with the oracle at that step's block size (drafted tokens under
    the gap rule, accept lengths, fallback tokens and context lengths)."""
    d0 = SMALL_BF16
    b, seed = 2, 37
    ctx0 = [30, 61]
    case = Hn.build_case(d0, b, ctx0, seed=seed, capacity=C.kv_capacity(max(ctx0) + 5 * 17))
    gpu = Hn.GpuRunner(case)
    cache = Hn.oracle_prefill(case, list(range(b)))
    rows = np.ones(b, dtype=np.int64)
    last = I.last_tokens(d0, seed, 0, b)
    tr = Hn.TokenReport()
    for step, B in enumerate((16, 4, 8, 16, 1)):
        d = d0.with_block(B)
        feats = [I.features(d, seed, step + 1, s, int(rows[s])) for s in range(b)]
        gpu.inject(feats)
        O.inject(d, case.weights, cache, feats)
        assert np.array_equal(gpu.ctx_len()[:b], cache.length)
        import torch
        dev = gpu.drafter.device
        out = torch.full((b, B), -1, dtype=torch.int32, device=dev)
        gpu.drafter.draft(torch.as_tensor(last).to(dev), out, b, block_size=B)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = O.draft_forward(d, case.weights, cache, last)
        tr.add(got, ref["tokens"], ref["gaps"], f"draft{step}")
        L_plant = I.planted_accept(seed, step, b, 0.2, B)
        _, hid = I.planted_targets(d, seed, step, case.weights.lm_head, ref["tokens"], L_plant)
        th = gpu.upload(hid.reshape(b * (B + 1), d.hidden), gpu.drafter.dt, dev).reshape(b, B + 1, d.hidden)
        ta = torch.full((b, B + 1), -1, dtype=torch.int32, device=dev)
        al = torch.full((b,), -1, dtype=torch.int32, device=dev)
        bo = torch.full((b,), -1, dtype=torch.int32, device=dev)
        gpu.drafter.verify(th, torch.as_tensor(ref["tokens"].astype(np.int32)).to(dev), ta, al, bo, b,
                           block_size=B)
        torch.cuda.synchronize()
        g_ref, vgaps = O.verify(d, case.weights.lm_head, hid)
        L_ref, bonus_ref = O.accept(ref["tokens"], g_ref)
        assert np.array_equal(L_ref, L_plant)
        tr.add(ta.cpu().numpy(), g_ref, vgaps, f"verify{step}")
        al, bo = al.cpu().numpy(), bo.cpu().numpy()
        for s_ in range(b):
            if np.all(vgaps[s_, :min(int(L_ref[s_]), B) + 1] > Hn.GAP):   # decided above the gap
                assert al[s_] == L_ref[s_] and bo[s_] == bonus_ref[s_], (step, s_, al, L_ref, bo, bonus_ref)
        rows = L_ref + 1
        last = bonus_ref.astype(np.int32)
    assert gpu.drafter.read_status() == 0
    assert not tr.mismatched, tr.mismatched
    print("compared", tr.compared, "below_gap", tr.below_gap, "ctx", cache.length)


def _grid_uniforms(seed, tid, shape):
    """Uniforms in (0, 1) on the 2^-24 grid (exact in fp32), seeded."""
    g = I.stream(seed, 60 + tid)
    return ((g.integers(0, 1 << 24, size=shape) + 0.5) / float(1 << 24)).astype(np.float32)


def _sampling_step(dims, batch, ctx, T, seed, seqs=None, kv_mode="inject"):
    """Sampled drafting and speculative-sampling verification on both
    sides from the same uniforms.  Drafted tokens are compared where the
    oracle's top-1/top-2 gap of logit / T + g, in logit units (times T),
    exceeds 1e-2; the accepted length where every acceptance decision's
    margin |log(p/q) - log u| times T exceeds 1e-2; the emitted token where,
    in addition, the final draw's gap does."""
    import torch
    d = dims
    B, V, H = d.block_size, d.vocab, d.hidden
    case = Hn.build_case(d, batch, ctx, seed=seed, kv_mode=kv_mode)
    seqs = list(range(batch)) if seqs is None else list(seqs)
    gpu = Hn.GpuRunner(case)
    feats, last = Hn.step_inputs(case, 0, [3] * batch)
    gpu.inject(feats)
    cache = Hn.oracle_prefill(case, seqs)
    O.inject(d, case.weights, cache, [feats[s] for s in seqs])
    u_draft = _grid_uniforms(seed, 0, (batch, B, V))
    u_acc = _grid_uniforms(seed, 1, (batch, B))
    u_res = _grid_uniforms(seed, 2, (batch, V))
    ref = O.draft_sample(d, case.weights, cache, last[seqs], T, u_draft[seqs])
    dev = gpu.drafter.device
    t = lambda a: torch.as_tensor(np.ascontiguousarray(a)).to(dev)
    out = torch.full((batch, B), -1, dtype=torch.int32, device=dev)
    dlog = torch.empty((batch * B, V), dtype=torch.float32, device=dev)
    gpu.drafter.draft_sample(t(last), T, t(u_draft), out, dlog, batch)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tr = Hn.TokenReport()
    tr.add(got[seqs], ref["tokens"], ref["gaps"] * T, "draft")
    assert not tr.mismatched, tr.mismatched
    rows = np.concatenate([np.arange(s * B, (s + 1) * B) for s in seqs])
    e_logits = Hn.rel_err_rows(dlog.cpu().numpy()[rows], ref["logits"].reshape(-1, V))
    assert e_logits <= Hn.REL_TOL, e_logits
    # verification of the oracle's drafted tokens (random stand-ins for the
    # sequences the oracle does not follow) on planted target states
    all_tok = I.stream(seed, 99, 0).integers(0, V - 1, size=(batch, B))
    all_tok[seqs] = ref["tokens"]
    L_plant = I.planted_accept(seed, 0, batch, 0.12, B)
    _, hid = I.planted_targets(d, seed, 0, case.weights.lm_head, all_tok, L_plant)
    p_logits = O.linear(hid[seqs].astype(np.float64), case.weights.lm_head)
    L_ref, nxt_ref, margins, gaps = O.speculative_verify(all_tok[seqs], ref["logits"], p_logits, T,
                                                         u_acc[seqs], u_res[seqs])
    th = gpu.upload(hid.reshape(batch * (B + 1), H), gpu.drafter.dt, dev).reshape(batch, B + 1, H)
    tlog = torch.empty((batch * (B + 1), V), dtype=torch.float32, device=dev)
    al = torch.full((batch,), -1, dtype=torch.int32, device=dev)
    nx = torch.full((batch,), -1, dtype=torch.int32, device=dev)
    gpu.drafter.verify_sample(th, t(all_tok.astype(np.int32)), dlog, T, t(u_acc), t(u_res), tlog, al, nx, batch)
    torch.cuda.synchronize()
    al, nx = al.cpu().numpy(), nx.cpu().numpy()
    trows = np.concatenate([np.arange(s * (B + 1), (s + 1) * (B + 1)) for s in seqs])
    assert Hn.rel_err_rows(tlog.cpu().numpy()[trows], p_logits.reshape(-1, V)) <= Hn.REL_TOL
    decided = compared = 0
    for i, s in enumerate(seqs):
        assert 0 <= al[s] <= B and 0 <= nx[s] < V
        if margins[i] * T > Hn.GAP:
            decided += 1
            assert al[s] == L_ref[i], (s, al[s], L_ref[i], margins[i])
            if gaps[i] * T > Hn.GAP:
                compared += 1
                assert nx[s] == nxt_ref[i], (s, nx[s], nxt_ref[i], gaps[i])
    assert gpu.drafter.read_status() == 0
    print(f"T={T} draft compared {tr.compared} below_gap {tr.below_gap}; accept decided {decided}/{len(seqs)}, "
          f"next token compared {compared}; logits err {e_logits:.2e}; L {L_ref.tolist()}")
    return tr, decided, compared


@pytest.mark.parametrize("batch,T", [(1, 1.0), (1, 0.05), (3, 1.0), (3, 0.05)])
def test_sampling_small(batch, T):
    """Temperature 1 (near-uniform distributions: rejections and residual
    draws) and 0.05 (peaked: planted prefixes accepted); batch 1 runs the
    skinny heads, batch 3 (48 draft / 51 verify rows) the tiled ones."""
    tr, decided, _ = _sampling_step(SMALL_BF16, batch, [40, 77, 130][:batch], T, seed=70 + batch)
    assert tr.compared >= 8 and decided >= 1


def test_sampling_large_vocab():
    """A 65536-token vocabulary: 32 chunks per row in the sampling kernels."""
    d = C.Dims(**{**SMALL_BF16.__dict__, "vocab": 65536})
    _sampling_step(d, 2, [50, 90], 1.0, seed=74)


def test_sampling_repeatable():
    """Same uniforms, same draws; other uniforms, other draws."""
    import torch
    d = SMALL_BF16
    case = Hn.build_case(d, 1, [33], seed=75)
    gpu = Hn.GpuRunner(case)
    dev = gpu.drafter.device
    last = torch.as_tensor(I.last_tokens(d, 75, 0, 1)).to(dev)
    outs = []
    for tid in (0, 0, 5):
        u = torch.as_tensor(_grid_uniforms(75, tid, (1, d.block_size, d.vocab))).to(dev)
        out = torch.empty((1, d.block_size), dtype=torch.int32, device=dev)
        dlog = torch.empty((d.block_size, d.vocab), dtype=torch.float32, device=dev)
        gpu.drafter.draft_sample(last, 1.0, u, out, dlog, 1)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and not np.array_equal(outs[0], outs[2])


@pytest.mark.slow
def test_sampling_qwen3_8b_full_shape():
    """Temperature 1 on the Qwen3-8B-shaped drafter at batch 1 over a
    2048-position cache (imported)."""
    w = C.get("qwen3-8b-b1")
    tr, _, _ = _sampling_step(w.dims, 1, [2048], 1.0, seed=76, kv_mode="import")
    assert tr.compared >= 8
