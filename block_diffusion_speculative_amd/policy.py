"""Adaptive block size: the block size of the next draft-and-verify step,
chosen from the accept lengths seen so far ("DFlash, Diffusion LLMs, dLLM,
MTP and Speculative Decoding: A Deep Research Report", "Discussion and open
problems": adaptive block sizes).

Host logic only; the kernels take any block size B <= 16 per call.

Model.  The accepted length of a step with block size B is L = min(G, B)
with G geometric on {0, 1, ...}, P(G = k) = (1 - p)^k p: drafted tokens are
accepted one after another until the first mismatch.  With q = 1 - p,
E[min(G, B)] = q (1 - q^B) / p, and a step commits E[min(G, B)] + 1 tokens
(the accepted ones and the target's own next token).  The pages' speedup
model S ~ C_AR E[L] / C_DF ("Term: DFlash speculative decoding",
"Mathematical view of acceptance and speedup") makes the tokens committed
per unit of step time the quantity to maximise, so the policy picks

    B* = argmax_B (E[min(G, B)] + 1) / t(B)

over the candidate sizes, with t(B) the caller's measured step time at B.

Estimate.  p is the maximum-likelihood estimate over the observed (L, B)
pairs.  A step with L < B saw G = L (probability q^L p); a step with L = B
only saw G >= B (probability q^B, censored).  The log-likelihood
(sum L) log q + n_short log p, with n_short the number of steps that stopped
short of their block, peaks at p = n_short / (n_short + sum L).  Optional
pseudo-observations (a prior of `prior_steps` steps with mean accepted
length `prior_mean`) keep the estimate finite before any step stopped short.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, Optional, Sequence, Tuple


def expected_accept(p: float, B: int) -> float:
    """E[min(G, B)] for G geometric on {0, 1, ...} with parameter p."""
    if p <= 0.0:
        return float(B)
    if p >= 1.0:
        return 0.0
    q = 1.0 - p
    return q * (1.0 - q ** B) / p


def mle_geometric(observations: Iterable[Tuple[int, int]], prior_steps: float = 0.0,
                  prior_mean: float = 7.8) -> Optional[float]:
    """Maximum-likelihood p from (accepted length L, block size B) pairs,
    L = B counted as censored; None when nothing has been observed.  A prior
    of `prior_steps` uncensored steps with mean `prior_mean` may be added."""
    total, short, n = 0.0, 0.0, 0
    for L, B in observations:
        if not 0 <= L <= B:
            raise ValueError(f"accepted length {L} outside [0, {B}]")
        total += L
        short += 1.0 if L < B else 0.0
        n += 1
    total += prior_steps * prior_mean
    short += prior_steps
    if n == 0 and prior_steps == 0:
        return None
    if short == 0:
        return 0.0
    return short / (short + total)


class BlockSizePolicy:
    """Chooses B per step.  step_time maps each candidate block size to the
    measured time of one step at that size (any unit); window bounds the
    history used (the most recent steps)."""

    def __init__(self, step_time: Dict[int, float], window: int = 64, prior_steps: float = 1.0,
                 prior_mean: float = 7.8, default: Optional[int] = None):
        if not step_time or any(t <= 0 for t in step_time.values()):
            raise ValueError("step_time needs a positive time per candidate block size")
        if any(not 1 <= B <= 16 for B in step_time):
            raise ValueError("block sizes must lie in [1, 16]")
        self.step_time = dict(step_time)
        self.history = deque(maxlen=window)
        self.prior_steps = prior_steps
        self.prior_mean = prior_mean
        self.default = default if default is not None else max(step_time)

    def observe(self, accepted: int, block_size: int) -> None:
        self.history.append((int(accepted), int(block_size)))

    def observe_many(self, accepted: Sequence[int], block_size: int) -> None:
        for L in accepted:
            self.observe(L, block_size)

    def p_hat(self) -> Optional[float]:
        return mle_geometric(self.history, self.prior_steps, self.prior_mean)

    def rate(self, B: int, p: float) -> float:
        """Committed tokens per unit time at block size B."""
        return (expected_accept(p, B) + 1.0) / self.step_time[B]

    def choose(self) -> int:
        p = self.p_hat()
        if p is None:
            return self.default
        # ties go to the smaller block (less verify work for the same rate)
        return max(sorted(self.step_time), key=lambda B: (self.rate(B, p), -B))
