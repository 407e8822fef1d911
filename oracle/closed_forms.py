"""Closed forms the speculative-decoding blog states (test infrastructure).

[SD] "Speculative Decoding: small model guesses, large model verifies"
(feifeigd.github.io, 2026-08-24):
* section 3: the per-position acceptance probability is sum_x min(q(x), p(x));
* section 4: with per-position acceptance rate alpha, gamma candidates and a
  draft/target cost ratio c, the expected tokens per round is
  E[N] = (1 - alpha^(gamma+1)) / (1 - alpha), the round costs gamma*c + 1 and
  the speedup is E[N] / (gamma*c + 1).
"""
from __future__ import annotations

import numpy as np


def acceptance_probability(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """sum_x min(p(x), q(x)) over the last axis ([SD] section 3)."""
    return np.minimum(np.asarray(p, dtype=np.float64), np.asarray(q, dtype=np.float64)).sum(-1)


def expected_tokens(alpha, gamma: int):
    """E[N] = (1 - alpha^(gamma+1)) / (1 - alpha); gamma + 1 at alpha = 1 ([SD] section 4)."""
    alpha = np.asarray(alpha, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
    return np.where(alpha == 1.0, gamma + 1.0, e)


def speedup(alpha, c, gamma: int):
    """E[N] / (gamma * c + 1) ([SD] section 4)."""
    return expected_tokens(alpha, gamma) / (gamma * np.asarray(c, dtype=np.float64) + 1.0)
