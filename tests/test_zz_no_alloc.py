"""The allocation-free verify call against dflash_verify_accept through the
C ABI: two calls in a row on one GPU (5 sequences on the tiled head, then a
smaller input of 1 sequence on the skinny head with its fused finish), each
compared bit-exactly (token ids, accept lengths, fallback tokens) with the
workspace call on the same inputs."""
import ctypes

import numpy as np
import pytest

from block_diffusion_speculative_amd import _lib
from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I
import harness as Hn

pytestmark = pytest.mark.gpu

DIMS = C.Dims(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, n_layers=1,
              intermediate=1024, vocab=8192, n_feat_layers=2, dtype="bf16")


def _verify_both(gpu, batch, seed):
    import torch
    d = DIMS
    B, H = d.block_size, d.hidden
    dr = gpu.drafter
    dev = dr.device
    draft = I.stream(seed, 99, 0).integers(0, d.vocab - 1, size=(batch, B))
    L = I.planted_accept(seed, 0, batch, 0.12, B)
    _, hid = I.planted_targets(d, seed, 0, gpu.case.weights.lm_head, draft, L)
    th = gpu.upload(hid.reshape(batch * (B + 1), H), dr.dt, dev).reshape(batch, B + 1, H)
    dt = torch.as_tensor(draft.astype(np.int32)).to(dev)
    outs = []
    for noalloc in (False, True):
        ta = torch.full((batch, B + 1), -1, dtype=torch.int32, device=dev)
        al = torch.full((batch,), -1, dtype=torch.int32, device=dev)
        bo = torch.full((batch,), -1, dtype=torch.int32, device=dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if noalloc:
            _lib.call("dflash_verify_accept_noalloc", ctypes.byref(dr.cd), dr.lm_head.data_ptr(), th.data_ptr(),
                      dt.data_ptr(), batch, ta.data_ptr(), al.data_ptr(), bo.data_ptr(), stream)
        else:
            _lib.call("dflash_verify_accept", ctypes.byref(dr.cd), dr.lm_head.data_ptr(), th.data_ptr(),
                      dt.data_ptr(), batch, ta.data_ptr(), al.data_ptr(), bo.data_ptr(),
                      dr.ws.data_ptr(), dr.ws_bytes, stream)
        torch.cuda.synchronize()
        outs.append((ta.cpu().numpy(), al.cpu().numpy(), bo.cpu().numpy()))
    (ta0, al0, bo0), (ta1, al1, bo1) = outs
    assert np.array_equal(ta0, ta1) and np.array_equal(al0, al1) and np.array_equal(bo0, bo1)
    assert np.all((al1 >= 0) & (al1 <= B))
    # the planted accept lengths come back (targets planted on these tokens)
    assert np.array_equal(al1, L)
    return outs[1]


def test_noalloc_verify_matches_workspace_call():
    case = Hn.build_case(DIMS, 5, [0] * 5, seed=50, capacity=64)
    gpu = Hn.GpuRunner(case)
    _verify_both(gpu, 5, seed=50)      # 85 rows: tiled head + argmax_finish_kernel
    _verify_both(gpu, 1, seed=51)      # 17 rows: skinny head, fused finish
    _verify_both(gpu, 5, seed=52)      # the scratch is left clear for the next call


def test_noalloc_rejects_batch_above_the_scratch():
    d = _lib.Dims()
    r = _lib.load().dflash_verify_accept_noalloc(ctypes.byref(d), 16, 16, 16, 65, 16, 16, 16, None)
    assert r == _lib.DFLASH_ERR_SHAPE
    assert b"static scratch" in _lib.load().dflash_last_error()
