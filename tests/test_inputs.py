"""The seeded input generator: determinism, bf16 rounding, planted acceptance."""
import math

import numpy as np

from block_diffusion_speculative_amd import configs as C
from block_diffusion_speculative_amd import inputs as I


def test_same_seed_same_bytes():
    a = I.normal(7, (1, 2), (1000, 37), 0.02, "bf16")
    b = I.normal(7, (1, 2), (1000, 37), 0.02, "bf16")
    c = I.normal(8, (1, 2), (1000, 37), 0.02, "bf16")
    assert a.tobytes() == b.tobytes()
    assert a.tobytes() != c.tobytes()


def test_chunked_generation_is_order_independent():
    n = (1 << 22) * 2 + 123          # three independent chunks, generated in parallel
    a = I.normal(3, (9,), (n,), 1.0, "f32")
    first = I.stream(3, 9, 0).standard_normal(1 << 22, dtype=np.float32)
    assert np.array_equal(a[: 1 << 22], first)
    last = I.stream(3, 9, 2).standard_normal(123, dtype=np.float32)
    assert np.array_equal(a[-123:], last)


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7 -> ties to even (1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8), 3.0], dtype=np.float32)
    I.round_bf16_(x)
    assert x.tolist() == [1.0, 1 + 2 ** -6, 1.0, -1.0, 3.0]
    bits = I.to_bf16_bits(np.array([1.0, -2.0], dtype=np.float32))
    assert bits.tolist() == [0x3F80, 0xC000]
    assert I.bf16_bits_to_f32(bits).tolist() == [1.0, -2.0]


def test_bf16_values_are_representable():
    a = I.normal(1, (1,), (4096,), 0.02, "bf16")
    assert np.all((a.view(np.uint32) & 0xFFFF) == 0)
    assert 0.018 < a.std() < 0.022


def test_geom_p_reaches_mean():
    p = I.geom_p_for_mean(7.8, 16)
    assert abs(p - 0.09133) < 5e-5
    assert abs(I.geometric_mean_accept(p, 16) - 7.8) < 1e-9
    assert abs(I.geometric_mean_accept(0.12, 16) - 6.385) < 1e-3


def test_planted_accept_distribution():
    p = 0.12
    L = np.concatenate([I.planted_accept(0, s, 1000, p, 16) for s in range(20)])
    assert L.min() >= 0 and L.max() <= 16
    want = I.geometric_mean_accept(p, 16)
    assert abs(L.mean() - want) < 5 * L.std() / math.sqrt(len(L))
    # P(L = 0) = p
    assert abs((L == 0).mean() - p) < 5 * math.sqrt(p * (1 - p) / len(L))


def test_planted_targets_structure():
    dims = C.Dims(hidden=64, n_q_heads=2, n_kv_heads=1, head_dim=32, n_layers=1,
                  intermediate=64, vocab=128, n_feat_layers=2, dtype="bf16")
    lm = I.normal(0, (5,), (128, 64), 0.02, "bf16")
    draft = np.arange(16 * 3).reshape(3, 16) % 127
    L = np.array([0, 5, 16], dtype=np.int32)
    t, hid = I.planted_targets(dims, 0, 0, lm, draft, L)
    for s in range(3):
        assert np.array_equal(t[s, :L[s]], draft[s, :L[s]])
        for j in range(L[s], 16):
            assert t[s, j] != draft[s, j]
    assert hid.shape == (3, 17, 64)
    assert np.all((hid.view(np.uint32) & 0xFFFF) == 0)


def test_last_tokens_never_mask():
    dims = C.TINY_DRAFT
    t = I.last_tokens(dims, 0, 0, 5000)
    assert t.min() >= 0 and t.max() < dims.mask_id


def test_workloads_consistent():
    for w in C.WORKLOADS.values():
        d = w.dims
        assert d.n_q_heads % d.n_kv_heads == 0
        assert d.head_dim % 32 == 0 and d.hidden % 32 == 0
    assert C.get("qwen3-8b-b1").dims.qkv_rows == 6144
    pc = C.QWEN3_8B_DRAFT.param_count()
    assert pc["fc"] == 4096 * 20480 and pc["lm_head"] == 151936 * 4096
