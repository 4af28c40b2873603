"""GPU parity of draft trees (the DDTree paragraph of "LLMs hit ludicrous
speed: diffusion decoding and dMoE supercharge AI inference, shattering old
benchmarks"): the best-first tree build from the drafter's logits, the
target's tree pass under the ancestor-only mask, the greedy walk down the
tree and the commit of the accepted path, against the oracle."""
import numpy as np
import pytest

import oracle.dflash_oracle as O
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I
import harness as Hn
from test_gpu_parity import SMALL_BF16
from test_gpu_target import SMALL_TARGET, TargetCase, _check_pass

pytestmark = pytest.mark.gpu


def _continuations(tok, par):
    seq = {0: ()}
    for i in range(1, len(tok)):
        seq[i] = seq[int(par[i])] + (int(tok[i]),)
    return set(v for k, v in seq.items() if k > 0)


@pytest.mark.parametrize("batch,K,N", [(1, 4, 15), (3, 3, 31), (2, 1, 12)])
def test_draft_tree_build(batch, K, N):
    """The GPU tree (as its set of continuations) equals the oracle's where
    the choice is decided: the top-K boundary of every slot and the score
    gap between the N-th and the next continuation above 1e-2."""
    import torch
    d = SMALL_BF16
    case = Hn.build_case(d, batch, [50, 90, 13][:batch], seed=90 + K)
    gpu = Hn.GpuRunner(case)
    feats, last = Hn.step_inputs(case, 0, [2] * batch)
    gpu.inject(feats)
    cache = Hn.oracle_prefill(case, list(range(batch)))
    O.inject(d, case.weights, cache, feats)
    ref = O.draft_forward(d, case.weights, cache, last, keep_logits=True)
    dev = gpu.drafter.device
    B, V = d.block_size, d.vocab
    dlog = torch.empty((batch * B, V), dtype=torch.float32, device=dev)
    tt = torch.full((batch, N + 1), -1, dtype=torch.int32, device=dev)
    tp = torch.full((batch, N + 1), -2, dtype=torch.int32, device=dev)
    gpu.drafter.draft_tree(torch.as_tensor(last).to(dev), K, N, dlog, tt, tp, batch)
    torch.cuda.synchronize()
    tt, tp = tt.cpu().numpy(), tp.cpu().numpy()
    assert Hn.rel_err_rows(dlog.cpu().numpy(), ref["logits"].reshape(-1, V)) <= Hn.REL_TOL
    decided = 0
    for s in range(batch):
        assert tt[s, 0] == last[s] and tp[s, 0] == -1
        assert all(0 <= tp[s, i] < i for i in range(1, N + 1))
        lg = ref["logits"][s]
        tok, par, dep, score = O.build_tree(lg, int(last[s]), K, N + 1 if K > 1 else min(N + 1, B))
        lp = np.sort(O.log_softmax(lg), axis=-1)[:, ::-1]
        k_gap = float(np.min(lp[:, K - 1] - lp[:, K]))
        n_gap = float(score[N] - score[N + 1]) if len(score) > N + 1 else np.inf
        got = _continuations(tt[s], tp[s])
        if min(k_gap, n_gap) > Hn.GAP:
            decided += 1
            assert got == _continuations(tok[:N + 1], par[:N + 1]), s
        # every tree, decided or not: a valid top-N tree within the tolerance
        # (several are correct where scores lie within rounding of each other)
        _assert_valid_top_n(O.log_softmax(lg), got, K, N)
    print("trees decided", decided, "of", batch)


def _assert_valid_top_n(lp, got, K, N):
    """got (a set of continuations) holds N prefix-closed continuations,
    each of whose tokens is among the slot's top K up to 1e-2, and no member
    scores below the best continuation left out by more than 1e-2."""
    B = lp.shape[0]
    kth = np.sort(lp, axis=-1)[:, ::-1][:, K - 1]
    top = np.argsort(-lp, axis=-1, kind="stable")[:, :K]
    assert len(got) == N
    score = lambda c: sum(lp[j, t] for j, t in enumerate(c))
    for c in got:
        assert len(c) == 1 or c[:-1] in got, c                       # prefix-closed
        assert all(lp[j, t] >= kth[j] - Hn.GAP for j, t in enumerate(c)), c
    frontier = [(int(t),) for t in top[0] if (int(t),) not in got]
    for c in got:
        if len(c) < B:
            frontier += [c + (int(t),) for t in top[len(c)] if c + (int(t),) not in got]
    best_out = max((score(c) for c in frontier), default=-np.inf)
    assert min(score(c) for c in got) >= best_out - Hn.GAP, (min(score(c) for c in got), best_out)


def _plant_path_hidden(d, lm_head, tok, par, path_end, seed):
    """Target hidden rows of a tree pass that make the walk follow the
    path from the root to node path_end and stop there: the row of each
    node on the path points (4 x its lm_head row, plus noise) at the next
    node's token, every other row at a token no child of its node has."""
    n = len(tok)
    g = np.random.default_rng(seed)
    chain = [path_end]
    while chain[-1] > 0:
        chain.append(int(par[chain[-1]]))
    chain = chain[::-1]
    want = np.zeros(n, dtype=np.int64)
    for i in range(n):
        kids = {int(tok[c]) for c in range(n) if par[c] == i}
        if i in chain and i != path_end:
            want[i] = tok[chain[chain.index(i) + 1]]
        else:
            t = int(g.integers(0, d.vocab - 1))
            while t in kids:
                t = int(g.integers(0, d.vocab - 1))
            want[i] = t
    hid = 4.0 * lm_head[want] + g.standard_normal((n, d.hidden)) * 0.1
    return I.round_bf16_(hid.astype(np.float32)), chain, want


def test_tree_pass_accept_and_commit():
    """The target's pass over a 16-node tree (oracle-built, the same input
    on both sides) against the oracle; the walk over planted target states
    recovers the planted path; the path commit leaves the cache a following
    causal pass agrees on."""
    import torch
    d = SMALL_TARGET
    B, K, N = 6, 3, 15
    tc = TargetCase(d, 2, [37, 70], seed=95)
    rng = np.random.default_rng(95)
    trees = [O.build_tree(rng.standard_normal((B, d.vocab)) * 2.0, int(rng.integers(0, d.vocab - 1)), K, N)
             for _ in range(2)]
    toks = np.stack([t[0] for t in trees]).astype(np.int32)
    pars = np.stack([t[1] for t in trees]).astype(np.int32)
    dev = tc.gpu.device
    hid_gpu = torch.empty((2, N + 1, d.hidden), dtype=tc.gpu.dt, device=dev)
    feats = torch.empty((2, N + 1, 2 * d.hidden), dtype=tc.gpu.dt, device=dev)
    tc.gpu.forward(torch.as_tensor(toks).to(dev), 2, N + 1, [0, 3], hid_gpu, feats,
                   parents=torch.as_tensor(pars).to(dev))
    torch.cuda.synchronize()
    ref = O.target_forward(d, tc.w, tc.cache, toks, [0, 3], parents=pars)
    errs = {"hidden": max(Hn.rel_err_rows(hid_gpu.float().cpu().numpy(), ref["hidden"]),
                          Hn.rel_err_heads(hid_gpu.float().cpu().numpy(), ref["hidden"])),
            "features": Hn.rel_err_rows(feats.float().cpu().numpy(), ref["features"])}
    for s in range(2):
        lo = int(tc.cache.length[s])
        kg, vg = tc.kv_rows(s, lo, lo + N + 1)
        errs["kv"] = max(errs.get("kv", 0.0), Hn.rel_err_rows(kg, tc.cache.k[:, s, :, lo:lo + N + 1]),
                         Hn.rel_err_rows(vg, tc.cache.v[:, s, :, lo:lo + N + 1]))
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= Hn.REL_TOL, (k, v)
    assert tc.gpu.read_status() == 0
    # the walk: a drafter (for its lm_head and workspace) over planted target states
    dcase = Hn.build_case(C.Dims(**{**SMALL_BF16.__dict__, "vocab": d.vocab}), 2, [0, 0], seed=96)
    drafter = Hn.GpuRunner(dcase).drafter
    lm = dcase.weights.lm_head
    ends = [int(np.argmax(trees[0][2])), 5]            # the deepest node, and node 5
    planted = [_plant_path_hidden(d, lm, toks[s], pars[s], ends[s], 97 + s) for s in range(2)]
    th = np.stack([p[0] for p in planted])
    ta = torch.full((2, N + 1), -1, dtype=torch.int32, device=dev)
    al = torch.full((2,), -1, dtype=torch.int32, device=dev)
    bo = torch.full((2,), -1, dtype=torch.int32, device=dev)
    pa = torch.full((2, N + 1), -9, dtype=torch.int32, device=dev)
    drafter.tree_accept(drafter_upload(drafter, th), torch.as_tensor(toks).to(dev), torch.as_tensor(pars).to(dev),
                        2, N + 1, ta, al, bo, pa)
    torch.cuda.synchronize()
    ta, al, bo, pa = ta.cpu().numpy(), al.cpu().numpy(), bo.cpu().numpy(), pa.cpu().numpy()
    for s in range(2):
        g_ref, gaps = O.verify(d, lm, th[s][None])
        assert np.array_equal(ta[s][gaps[0] > Hn.GAP], g_ref[0][gaps[0] > Hn.GAP])
        L, bonus, path = O.tree_accept(toks[s], pars[s], g_ref[0])
        assert list(path) == planted[s][1], (path, planted[s][1])
        assert al[s] == L and bo[s] == bonus and list(pa[s][:L + 1]) == list(path) and np.all(pa[s][L + 1:] == -1)
    # commit the walked paths and check the cache with a following causal pass
    tc.gpu.commit_path(torch.as_tensor(pa).to(dev), torch.as_tensor(al).to(dev), 2, N + 1)
    torch.cuda.synchronize()
    for s in range(2):
        O.commit_path(tc.cache, s, pa[s][:al[s] + 1])
    assert np.array_equal(tc.gpu.ctx_len.cpu().numpy()[:2], tc.cache.length)
    _check_pass(tc, I.target_tokens(d, 95, 1, 2, 5), [2])


def drafter_upload(drafter, arr):
    import torch
    from block_diffusion_speculative_amd.engine import upload
    b, n, H = arr.shape
    return upload(arr.reshape(b * n, H), drafter.dt, drafter.device).reshape(b, n, H)


def test_tree_pass_32_nodes_two_query_tiles():
    """A 32-node tree (two query tiles, a full key step of new rows)."""
    d = SMALL_TARGET
    tc = TargetCase(d, 1, [100], seed=98)
    rng = np.random.default_rng(98)
    tok, par, _, _ = O.build_tree(rng.standard_normal((8, d.vocab)), 5, 4, 31)
    import torch
    dev = tc.gpu.device
    hid = torch.empty((1, 32, d.hidden), dtype=tc.gpu.dt, device=dev)
    tc.gpu.forward(torch.as_tensor(tok[None].astype(np.int32)).to(dev), 1, 32, [], hid, None,
                   parents=torch.as_tensor(par[None].astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    ref = O.target_forward(d, tc.w, tc.cache, tok[None], [], parents=par[None])
    e = max(Hn.rel_err_rows(hid.float().cpu().numpy(), ref["hidden"]),
            Hn.rel_err_heads(hid.float().cpu().numpy(), ref["hidden"]))
    assert e <= Hn.REL_TOL, e


def test_malformed_tree_sets_status():
    import torch
    d = SMALL_TARGET
    tc = TargetCase(d, 1, [10], seed=99)
    dev = tc.gpu.device
    par = torch.as_tensor(np.array([[-1, 0, 5, 1]], dtype=np.int32)).to(dev)   # node 2's parent after it
    hid = torch.empty((1, 4, d.hidden), dtype=tc.gpu.dt, device=dev)
    tc.gpu.forward(torch.as_tensor(np.array([[1, 2, 3, 4]], dtype=np.int32)).to(dev), 1, 4, [], hid, None,
                   parents=par)
    torch.cuda.synchronize()
    assert tc.gpu.read_status() & 8
