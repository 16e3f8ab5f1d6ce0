"""Closed-form quantities of speculative decoding, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (see the ``oracle`` package docstring).

Sources:
  [FI] "Fast Inference from Transformers via Speculative Decoding" (paper
       summary page): "Expected Number of Generated Tokens" (Equation 1),
       "Computing alpha from p and q: The DLK Divergence" (Definition 3.2,
       Lemma 3.3, Theorem 3.5), "Walltime Improvement Analysis" (Theorem
       3.8), "Number of Arithmetic Operations" (Theorem 3.11).
  [TM] "Speculative Decoding: Two Models, One Output": "What the speedup
       depends on".
"""
from __future__ import annotations

import numpy as np


def expected_tokens(alpha: float, gamma: int) -> float:
    """E[# tokens per step] under i.i.d. acceptance with rate alpha:
    the truncated geometric series 1 + a + ... + a^gamma
    = (1 - a^(gamma+1)) / (1 - a)  ([FI] Equation 1, [TM])."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def walltime_improvement(alpha: float, gamma: int, c: float) -> float:
    """Expected tokens per step divided by the step cost gamma*c + 1
    ([FI] Theorem 3.8)."""
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def operations_factor(alpha: float, gamma: int, c_hat: float) -> float:
    """Arithmetic per emitted token relative to plain decoding:
    (gamma*c_hat + gamma + 1) target-equivalent runs per step divided by the
    expected tokens per step ([FI] Theorem 3.11)."""
    return (gamma * c_hat + gamma + 1.0) / expected_tokens(alpha, gamma)


def dlk(p: np.ndarray, q: np.ndarray) -> float:
    """DLK(p, q) = sum_x |p(x) - M(x)| with M the pointwise mean
    ([FI] Definition 3.2)."""
    m = 0.5 * (p + q)
    return float(np.abs(p - m).sum())


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """beta = sum_x min(p(x), q(x)) ([FI] Theorem 3.5)."""
    return float(np.minimum(p, q).sum())
