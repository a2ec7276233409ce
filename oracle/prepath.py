"""fp64 CPU oracle for the steps just before the KDA recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` imports this module.  It shares no
code with the HIP library.

The recurrence takes q and k L2-normalised per token and head, a log-gate
g <= 0 and a write strength beta in (0, 1).  From raw projections these are
obtained as written out below ("Kimi Linear architecture" (ttj.ttj.kr),
section "KDA: a memo that erases and rewrites": one forget rate per channel in
(0, 1); "From GPT-2 to Kimi K3", section "Gated DeltaNet: now it can forget":
alpha in [0, 1]).  The pages do not print the parametrisation; this is the
one the benchmark inputs are drawn with: g = -softplus(x), so that
alpha = exp(g) = 1 / (1 + e^x) lies in (0, 1), and beta = sigmoid(x).
"""
from __future__ import annotations

import numpy as np

from . import widen


def l2_normalize(x):
    """x / ||x|| over the last axis in fp64; an all-zero vector stays zero."""
    x = widen(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    out = np.zeros_like(x)
    np.divide(x, n, out=out, where=n > 0)
    return out


def neg_softplus(x):
    """-log(1 + e^x) in fp64, without overflow for large |x|."""
    x = widen(x)
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def sigmoid(x):
    """1 / (1 + e^-x) in fp64, without overflow for large |x|."""
    x = widen(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def prepare(q_raw, k_raw, g_raw, beta_raw):
    """(q, k, g, beta) for the recurrence from raw projections, fp64."""
    return l2_normalize(q_raw), l2_normalize(k_raw), neg_softplus(g_raw), sigmoid(beta_raw)
