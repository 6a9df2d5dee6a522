"""Pins of the fp64 oracle: facts fixed by the pages or by mathematics that do
not depend on the oracle's own code.

Each pin takes the module (or any object) exposing the oracle's `prefill`
function and a `lib` handle, and raises AssertionError when the pinned fact
does not hold. tests/test_oracle.py runs them on the oracle; the mutant test
runs them on deliberately broken copies of the oracle to show that each
plausible mistake is caught by at least one pin.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import brute


def dyadic(rng, shape, denom=8, lim=4):
    """Random values j / denom in [-lim, lim]: exact in fp32 and bf16."""
    n = int(round(lim * denom))
    return (rng.integers(-n, n + 1, size=shape) / denom).astype(np.float32)


def unit_keys(rng, T, H, D, nnz=4):
    """Keys with exactly unit norm in fp32: nnz entries of +-1/sqrt(nnz)."""
    assert int(math.isqrt(nnz)) ** 2 == nnz
    k = np.zeros((T, H, D), np.float32)
    val = 1.0 / math.isqrt(nnz)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(D, size=nnz, replace=False)
            k[t, h, idx] = val * rng.choice([-1.0, 1.0], size=nnz)
    return k


def decay(rng, shape):
    return (-np.exp(rng.normal(-2.0, 0.7, size=shape))).astype(np.float32)


def _run(recur, lib, q, k, v, g, beta, cu, **kw):
    return recur.prefill(q, k, v, g, beta, cu, lib=lib, **kw)


# --- P1: alpha = 1 (g = 0) and beta = 0 leave the state unchanged ---------------
def pin_identity(recur, lib=None):
    rng = np.random.default_rng(11)
    T, H, Dk, Dv = 9, 2, 8, 5
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    g = np.zeros((T, H, Dk), np.float32)
    beta = np.zeros((T, H), np.float32)
    s0 = rng.standard_normal((1, H, Dk, Dv)).astype(np.float32)
    r = _run(recur, lib, q, k, v, g, beta, [0, T], initial_state=s0, col_block=3)
    assert np.array_equal(r["final"], s0.astype(np.float64)), "state changed with g=0, beta=0"
    ref = np.einsum("hij,thi->thj", s0[0].astype(np.float64), q.astype(np.float64))
    assert np.allclose(r["o"], ref, rtol=0, atol=1e-13), "o != S0^T q with g=0, beta=0"


# --- P2: beta = 0 gives pure per-channel decay: S_t = diag(exp(G_t)) S_0 --------
def pin_pure_decay(recur, lib=None):
    rng = np.random.default_rng(12)
    T, H, Dk, Dv = 23, 2, 8, 6
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    g = decay(rng, (T, H, Dk))
    beta = np.zeros((T, H), np.float32)
    s0 = rng.standard_normal((1, H, Dk, Dv)).astype(np.float32)
    r = _run(recur, lib, q, k, v, g, beta, [0, T], initial_state=s0, col_block=4)
    G = np.cumsum(g.astype(np.float64), axis=0)                      # [T, H, Dk]
    S0 = s0[0].astype(np.float64)
    fin = np.exp(G[-1])[:, :, None] * S0
    assert np.allclose(r["final"][0], fin, rtol=1e-12, atol=1e-300), "pure decay final state"
    ref_o = np.einsum("hij,thi->thj", S0, np.exp(G) * q.astype(np.float64))
    assert np.allclose(r["o"], ref_o, rtol=1e-11, atol=1e-13), "pure decay outputs"


# --- P3: delta rule, beta = 1 and ||k|| = 1: S_t^T k_t = v_t exactly ----------------
def pin_delta_retrieval(recur, lib=None):
    """The delta rule removes the association stored under k_t and writes v_t
    in its place, so reading the updated state with the same unit key returns
    v_t (Kimi K3 report, "Methodology notes", DeltaNet and Delta Rule)."""
    rng = np.random.default_rng(13)
    T, H, Dk, Dv = 17, 2, 16, 7
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = unit_keys(rng, T, H, Dk)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    g = decay(rng, (T, H, Dk))
    beta = np.ones((T, H), np.float32)
    s0 = rng.standard_normal((1, H, Dk, Dv)).astype(np.float32)
    r = _run(recur, lib, q, k, v, g, beta, [0, T], initial_state=s0, ckpt_interval=1)
    St = r["ckpt"]                                                 # [T, H, Dk, Dv]
    got = np.einsum("thij,thi->thj", St, k.astype(np.float64))
    assert np.allclose(got, v.astype(np.float64), rtol=0, atol=1e-12), "S_t^T k_t != v_t"
    assert np.array_equal(St[-1], r["final"][0]), "last per-token state != final state"


# --- P4: one-hot keys: closed-form row update ----------------------------------
def pin_one_hot(recur, lib=None):
    """With k_t = e_j, every row decays by alpha_t and then row j moves a
    fraction beta_t of the way to v_t: forget-then-write order."""
    rng = np.random.default_rng(14)
    T, H, Dk, Dv = 19, 2, 6, 5
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    js = rng.integers(0, Dk, size=(T, H))
    k = np.zeros((T, H, Dk), np.float32)
    for t in range(T):
        for h in range(H):
            k[t, h, js[t, h]] = 1.0
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    g = decay(rng, (T, H, Dk))
    beta = rng.uniform(0.05, 0.95, size=(T, H)).astype(np.float32)
    s0 = rng.standard_normal((1, H, Dk, Dv)).astype(np.float32)
    r = _run(recur, lib, q, k, v, g, beta, [0, T], initial_state=s0, ckpt_interval=1)
    for h in range(H):
        S = s0[0, h].astype(np.float64)
        for t in range(T):
            S = np.exp(g[t, h].astype(np.float64))[:, None] * S
            j = js[t, h]
            b = float(beta[t, h])
            S[j] = (1.0 - b) * S[j] + b * v[t, h].astype(np.float64)
            assert np.allclose(r["ckpt"][t, h], S, rtol=1e-13, atol=1e-14), "one-hot state"
            o = S.T @ q[t, h].astype(np.float64)
            assert np.allclose(r["o"][t, h], o, rtol=1e-12, atol=1e-13), "one-hot output"


# --- P5: exact rational brute force on tiny inputs --------------------------------
def pin_exact_rationals(recur, lib=None):
    rng = np.random.default_rng(15)
    for trial in range(3):
        T, Dk, Dv = 4, 3, 2
        q = dyadic(rng, (T, 1, Dk))
        k = dyadic(rng, (T, 1, Dk), denom=4, lim=1)
        v = dyadic(rng, (T, 1, Dv))
        g = decay(rng, (T, 1, Dk))
        beta = (rng.integers(1, 8, size=(T, 1)) / 8).astype(np.float32)
        s0 = dyadic(rng, (1, 1, Dk, Dv))
        r = _run(recur, lib, q, k, v, g, beta, [0, T], initial_state=s0, ckpt_interval=1,
                 col_block=1)
        F = lambda x: Fraction(float(x))
        alpha = [[Fraction(math.exp(float(g[t, 0, i]))) for i in range(Dk)] for t in range(T)]
        outs, states = brute.run(
            [[F(x) for x in q[t, 0]] for t in range(T)],
            [[F(x) for x in k[t, 0]] for t in range(T)],
            [[F(x) for x in v[t, 0]] for t in range(T)],
            alpha, [F(beta[t, 0]) for t in range(T)],
            [[F(x) for x in row] for row in s0[0, 0]])
        for t in range(T):
            exact_o = np.array([float(x) for x in outs[t]])
            exact_s = np.array([[float(x) for x in row] for row in states[t]])
            assert np.allclose(r["o"][t, 0], exact_o, rtol=1e-13, atol=1e-14), "rational o"
            assert np.allclose(r["ckpt"][t, 0], exact_s, rtol=1e-13, atol=1e-14), "rational S"


# --- P6: (V, S_0) -> (O, S_T) is jointly linear; O is linear in Q ---------------------
def pin_linearity(recur, lib=None):
    rng = np.random.default_rng(16)
    T, H, Dk, Dv = 21, 2, 8, 6
    q1, q2 = dyadic(rng, (T, H, Dk)), dyadic(rng, (T, H, Dk))
    k = rng.standard_normal((T, H, Dk)).astype(np.float32) * 0.3
    v1, v2 = dyadic(rng, (T, H, Dv)), dyadic(rng, (T, H, Dv))
    g = decay(rng, (T, H, Dk))
    beta = rng.uniform(0, 1, size=(T, H)).astype(np.float32)
    s1, s2 = dyadic(rng, (1, H, Dk, Dv)), dyadic(rng, (1, H, Dk, Dv))
    a = _run(recur, lib, q1, k, v1, g, beta, [0, T], initial_state=s1)
    b = _run(recur, lib, q1, k, v2, g, beta, [0, T], initial_state=s2)
    c = _run(recur, lib, q1, k, v1 + v2, g, beta, [0, T], initial_state=s1 + s2)
    scale = np.abs(c["o"]).max() + 1.0
    assert np.allclose(c["o"], a["o"] + b["o"], rtol=0, atol=1e-12 * scale), "o not linear in (V, S0)"
    assert np.allclose(c["final"], a["final"] + b["final"], rtol=0, atol=1e-12 * scale), \
        "S_T not linear in (V, S0)"
    d = _run(recur, lib, q2, k, v1, g, beta, [0, T], initial_state=s1)
    e = _run(recur, lib, q1 + q2, k, v1, g, beta, [0, T], initial_state=s1)
    assert np.allclose(e["o"], a["o"] + d["o"], rtol=0, atol=1e-12 * scale), "o not linear in Q"
    assert np.array_equal(e["final"], a["final"]), "state depends on Q"


ALL_PINS = [pin_identity, pin_pure_decay, pin_delta_retrieval, pin_one_hot,
            pin_exact_rationals, pin_linearity]
