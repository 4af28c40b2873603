"""GPU parity of the target's causal verify pass (dflash_target_forward)
and its commit, against the oracle's target_forward / commit on the same
seeded inputs: final normalised hidden states, captured features and the
K/V rows the pass appends, within 2e-2 per row and per 128-channel segment."""
import numpy as np
import pytest

import oracle.dflash_oracle as O
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I
import harness as Hn

pytestmark = pytest.mark.gpu

SMALL_TARGET = C.Dims(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, n_layers=4,
                      intermediate=1024, vocab=4096, n_feat_layers=2, dtype="bf16")


def _errs(got, ref):
    return max(Hn.rel_err_rows(got, ref), Hn.rel_err_heads(got, ref))


class TargetCase:
    def __init__(self, dims, batch, ctx, seed, capacity=None):
        import torch
        from block_diffusion_speculative_amd.engine import Target, upload
        self.torch, self.dims, self.batch, self.seed = torch, dims, batch, seed
        self.ctx = np.asarray(ctx, dtype=np.int32)
        cap = capacity or C.kv_capacity(int(self.ctx.max()) + 40)
        self.w = I.make_target_weights(dims, seed)
        self.gpu = Target(dims, self.w, batch, cap, max_rows=32)
        shape = (dims.n_layers, batch, dims.n_kv_heads, cap, dims.head_dim)
        k = np.zeros(shape, dtype=np.float32)
        v = np.zeros(shape, dtype=np.float32)
        for l in range(dims.n_layers):
            for s in range(batch):
                ks, vs = I.kv_entries(dims, seed + 1000, l, s, int(self.ctx[s]))
                k[l, s, :, :self.ctx[s]] = ks
                v[l, s, :, :self.ctx[s]] = vs
        dev = self.gpu.device
        self.gpu.kv_import(upload(k.reshape(-1, dims.head_dim), self.gpu.dt, dev).reshape(shape),
                           upload(v.reshape(-1, dims.head_dim), self.gpu.dt, dev).reshape(shape))
        self.gpu.set_ctx_len(self.ctx)
        self.cache = O.OracleCache(k.astype(np.float64), v.astype(np.float64), self.ctx.astype(np.int64).copy())
        self.cap = cap
        torch.cuda.synchronize()

    def run(self, tokens, feat_layers):
        torch = self.torch
        d, dev = self.dims, self.gpu.device
        b, n = tokens.shape
        hid = torch.empty((b, n, d.hidden), dtype=self.gpu.dt, device=dev)
        feats = torch.empty((b, n, len(feat_layers) * d.hidden), dtype=self.gpu.dt, device=dev)
        self.gpu.forward(torch.as_tensor(tokens).to(dev), b, n, feat_layers, hid, feats if feat_layers else None)
        torch.cuda.synchronize()
        return hid.float().cpu().numpy(), feats.float().cpu().numpy()

    def kv_rows(self, s, lo, hi):
        torch = self.torch
        d = self.dims
        shape = (d.n_layers, self.batch, d.n_kv_heads, self.cap, d.head_dim)
        k = torch.empty(shape, dtype=self.gpu.dt, device=self.gpu.device)
        v = torch.empty(shape, dtype=self.gpu.dt, device=self.gpu.device)
        from block_diffusion_speculative_amd import _lib
        import ctypes
        _lib.call("dflash_kv_export", ctypes.byref(self.gpu.cd), ctypes.byref(self.gpu.ckv), k.data_ptr(),
                  v.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        return k[:, s, :, lo:hi].float().cpu().numpy(), v[:, s, :, lo:hi].float().cpu().numpy()


def _check_pass(tc, tokens, feat_layers, seqs=None, check_kv=True):
    seqs = list(range(tc.batch)) if seqs is None else seqs
    hid, feats = tc.run(tokens, feat_layers)
    sub = O.OracleCache(tc.cache.k[:, seqs], tc.cache.v[:, seqs], tc.cache.length[seqs].copy())
    ref = O.target_forward(tc.dims, tc.w, sub, tokens[seqs], feat_layers)
    tc.cache.k[:, seqs], tc.cache.v[:, seqs] = sub.k, sub.v
    errs = {"hidden": _errs(hid[seqs], ref["hidden"])}
    if feat_layers:
        errs["features"] = _errs(feats[seqs], ref["features"])
    n = tokens.shape[1]
    if check_kv:
        for i, s in enumerate(seqs):
            lo = int(tc.cache.length[s])
            kg, vg = tc.kv_rows(s, lo, lo + n)
            errs["kv"] = max(errs.get("kv", 0.0), Hn.rel_err_rows(kg, sub.k[:, i, :, lo:lo + n]),
                             Hn.rel_err_rows(vg, sub.v[:, i, :, lo:lo + n]))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= Hn.REL_TOL, (k, v, errs)
    assert tc.gpu.read_status() == 0
    return ref


def _commit(tc, accept_len, max_commit):
    torch = tc.torch
    tc.gpu.commit(torch.as_tensor(np.asarray(accept_len, dtype=np.int32)).to(tc.gpu.device), tc.batch, max_commit)
    O.commit(tc.cache, np.minimum(np.maximum(np.asarray(accept_len) + 1, 0), max_commit) - 1)
    torch.cuda.synchronize()
    assert np.array_equal(tc.gpu.ctx_len.cpu().numpy()[:tc.batch], tc.cache.length)


def test_target_pass_and_commit_small():
    """17 rows (two query tiles) over imported contexts of 40 and 75
    positions, features after layers 0 and 2; then commit 4 and 17 rows and
    a 5-row pass that must see the committed rows."""
    d = SMALL_TARGET
    tc = TargetCase(d, 2, [40, 75], seed=80)
    toks = I.target_tokens(d, 80, 0, 2, 17)
    _check_pass(tc, toks, [0, 2])
    _commit(tc, [3, 16], 17)
    _check_pass(tc, I.target_tokens(d, 80, 1, 2, 5), [1])


@pytest.mark.parametrize("rows", [1, 16, 17, 32])
def test_target_row_counts(rows):
    """One row (the autoregressive step), one full query tile, the verify
    pass of a 16-slot block (17 rows: a second row tile holding one row),
    and the largest pass (32 rows, a full key step of new rows)."""
    d = SMALL_TARGET
    tc = TargetCase(d, 1, [61], seed=81 + rows)
    _check_pass(tc, I.target_tokens(d, 81, rows, 1, rows), [3])


def test_target_batch4_tiled():
    """4 sequences x 17 rows = 68 rows: tiled GEMMs, per-row scales from
    rstd_kernel, ragged contexts including an empty one."""
    d = SMALL_TARGET
    tc = TargetCase(d, 4, [0, 33, 64, 150], seed=85)
    _check_pass(tc, I.target_tokens(d, 85, 0, 4, 17), [0, 1, 3])


def test_target_capacity_overflow_sets_status():
    import torch
    d = SMALL_TARGET
    tc = TargetCase(d, 1, [20], seed=86, capacity=32)
    tc.run(I.target_tokens(d, 86, 0, 1, 17), [])      # rows 20 .. 36 pass the 32 positions
    assert tc.gpu.read_status() & 1


@pytest.mark.slow
def test_target_full_width_qwen3_8b_layers():
    """The Qwen3-8B-shaped target's layer at full width (hidden 4096, 32/8
    heads, intermediate 12288; 6 of its 36 layers, each launched as in the
    full model) over a 2048-position context, 17 rows, features after
    layers 1 and 4."""
    d = C.Dims(**{**C.QWEN3_8B_TARGET.__dict__, "n_layers": 6})
    tc = TargetCase(d, 1, [2048], seed=87)
    _check_pass(tc, I.target_tokens(d, 87, 0, 1, 17), [1, 4])
