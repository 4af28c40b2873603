"""The adaptive block-size policy on the CPU: the censored geometric
estimate, the expected accepted length against brute force, and the choice
against an exhaustive search."""
import math

import numpy as np
import pytest

from block_diffusion_speculative_amd import inputs as I
from block_diffusion_speculative_amd.policy import (BlockSizePolicy, expected_accept,
                                                    mle_geometric)


def test_expected_accept_matches_brute_force():
    for p in (0.05, 0.0913, 0.3, 0.9):
        for B in (1, 4, 8, 16):
            q = 1 - p
            brute = sum(min(k, B) * q ** k * p for k in range(4000))
            assert abs(expected_accept(p, B) - brute) < 1e-9
    assert expected_accept(0.0, 8) == 8.0 and expected_accept(1.0, 8) == 0.0
    # the planted-acceptance generator's closed form is the same quantity
    assert abs(expected_accept(0.0913, 16) - I.geometric_mean_accept(0.0913, 16)) < 1e-12


def test_censored_estimate_recovers_p():
    rng = np.random.default_rng(3)
    for p in (0.05, 0.12, 0.4):
        obs = []
        for B in (4, 8, 16):
            G = rng.geometric(p, size=20000) - 1
            obs += [(int(min(g, B)), B) for g in G]
        p_hat = mle_geometric(obs)
        se = math.sqrt(p * p * (1 - p) / (len(obs) * 0.5))
        assert abs(p_hat - p) < 6 * se + 2e-3, (p, p_hat)


def test_censored_estimate_is_the_likelihood_maximum():
    obs = [(3, 16), (16, 16), (0, 4), (4, 4), (7, 8)]
    p_hat = mle_geometric(obs)

    def loglik(p):
        q = 1 - p
        return sum(L * math.log(q) + (math.log(p) if L < B else 0.0) for L, B in obs)

    grid = np.linspace(1e-4, 1 - 1e-4, 20001)
    best = grid[np.argmax([loglik(p) for p in grid])]
    assert abs(p_hat - best) < 1e-3


def test_estimate_edge_cases():
    assert mle_geometric([]) is None
    assert mle_geometric([(16, 16), (8, 8)]) == 0.0          # nothing stopped short
    assert mle_geometric([(0, 16), (0, 4)]) == 1.0           # nothing accepted
    with pytest.raises(ValueError):
        mle_geometric([(5, 4)])


def test_choice_is_the_exhaustive_argmax():
    times = {4: 3.42, 8: 3.60, 16: 4.28}                      # measured step times (ms)
    pol = BlockSizePolicy(times, prior_steps=0)
    assert pol.choose() == 16                                 # no history: the default
    rng = np.random.default_rng(5)
    for p in (0.02, 0.1, 0.25, 0.6):
        pol = BlockSizePolicy(times, window=4096, prior_steps=0)
        for B in (4, 8, 16):
            pol.observe_many([int(min(g, B)) for g in rng.geometric(p, 1000) - 1], B)
        ph = pol.p_hat()
        best = max(times, key=lambda B: ((1 - ph) * (1 - (1 - ph) ** B) / ph + 1) / times[B])
        assert pol.choose() == best
    # long acceptances favour the large block, short ones the small block
    pol = BlockSizePolicy(times, prior_steps=0)
    pol.observe_many([16] * 20 + [12], 16)
    assert pol.choose() == 16
    pol = BlockSizePolicy(times, prior_steps=0)
    pol.observe_many([0, 1, 0, 2, 1, 0], 16)
    assert pol.choose() == 4


def test_window_forgets_old_steps():
    pol = BlockSizePolicy({4: 1.0, 16: 1.2}, window=8, prior_steps=0)
    pol.observe_many([16] * 8, 16)
    assert pol.choose() == 16
    pol.observe_many([0] * 8, 16)
    assert pol.choose() == 4


def test_bad_tables_rejected():
    with pytest.raises(ValueError):
        BlockSizePolicy({})
    with pytest.raises(ValueError):
        BlockSizePolicy({4: 0.0})
    with pytest.raises(ValueError):
        BlockSizePolicy({32: 1.0})
