"""Parameter-free KDA input transforms in fp64, applied before the recurrence.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

KDA normalises queries and keys to unit L2 norm and drives its per-channel
forgetting factor through a gate (Kimi K3 report, English and Chinese
editions, "Methodology notes", Kimi Delta Attention bullet; SemiAnalysis
digest, section 1 on KDA). The weighted parts named there (short
convolution, low-rank gate projection, output gate) need trained weights and
are not part of this core. The pages give no formula for the parameter-free
parts; the readings taken here:

    l2norm(x) = x / sqrt(sum_c x_c^2 + EPS)   per (token, head), EPS = 1e-6
                (a zero row stays zero)
    gate(u)   = -exp(u)                        the log-decay g, so the decay
                                               alpha = exp(-exp(u)) lies in (0, 1)
    beta(b)   = 1 / (1 + exp(-b))              write strength in (0, 1)

The gate is the map the benchmark workloads use to draw g from u, and the
sigmoid the one they use for beta.
"""

from __future__ import annotations

import numpy as np

FRONT_L2NORM_QK = 1
FRONT_GATE = 2
FRONT_BETA_SIGMOID = 4
FRONT_ALL = FRONT_L2NORM_QK | FRONT_GATE | FRONT_BETA_SIGMOID
EPS = 1e-6


def to_f64(x: np.ndarray) -> np.ndarray:
    """fp64 copy of an fp32/fp64 array or of bf16 bit patterns (uint16)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def l2norm(x: np.ndarray) -> np.ndarray:
    """Rows of the last axis scaled to unit L2 norm (EPS inside the root)."""
    x = to_f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def gate(u: np.ndarray) -> np.ndarray:
    """Log-decay from the gate pre-activation: g = -exp(u)."""
    return -np.exp(to_f64(u))


def sigmoid(b: np.ndarray) -> np.ndarray:
    """Write strength from its logit, evaluated without overflow for either sign."""
    b = to_f64(b)
    e = np.exp(-np.abs(b))
    return np.where(b >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def apply(q, k, v, g, beta, flags: int):
    """The transforms selected by `flags` on raw inputs; all five results in fp64
    (the oracle's recurrence takes fp64 q, k, v, g and beta together)."""
    q, k, v, g, beta = (to_f64(a) for a in (q, k, v, g, beta))
    if flags & FRONT_L2NORM_QK:
        q, k = l2norm(q), l2norm(k)
    if flags & FRONT_GATE:
        g = gate(g)
    if flags & FRONT_BETA_SIGMOID:
        beta = sigmoid(beta)
    return q, k, v, g, beta
