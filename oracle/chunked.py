"""Chunked (blockwise) formulation of the KDA recurrence in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages describe FlashKDA's prefill as unrolling the token recurrence by
chunks so that most of the work becomes matrix products: a preparation step
builds decayed queries and keys, an inverse transform and causal matrices
(called a UT transform on the SemiAnalysis digest, section 1 on KDA), and a
blockwise recurrence produces pseudo-values, outputs and the updated state
(Kimi K3 report, "Methodology notes", FlashKDA bullet). The pages give no
formulas; the algebra below is derived from the token recurrence

    S_r = Diag(a_r) S_{r-1} + k_r u_r^T,  u_r = beta_r (v_r - (Diag(a_r) S_{r-1})^T k_r),
    o_r = S_r^T q_r,

by unrolling it over the rows r = 1..C of one chunk that starts from state S:

    G   = inclusive cumulative sum of g over the chunk's rows, Gamma = exp(G)
    Kd  = K * Gamma,   Ki = K * exp(-G),   Qd = Q * Gamma,
    Kc  = K * exp(G_last - G)
    A   = strictly-lower part of diag(beta) Kd Ki^T
    (I + A) U = diag(beta) (V - Kd S)          (unit lower-triangular solve)
      => U = U0 - W S with W = (I + A)^-1 diag(beta) Kd,  U0 = (I + A)^-1 diag(beta) V
    P   = lower part (with diagonal) of Qd Ki^T
    O   = Qd S + P U
    S'  = diag(Gamma_last) S + Kc^T U

A chunk is shorter at the end of a sequence; chunks also end at every
checkpoint position so that the checkpointed state is a chunk-end state.
The triangular solve is scipy's (a library routine used as one step).
"""

from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def chunk_step(S, Q, K, V, g, beta):
    """Advance state S (Dk x Dv) over one chunk; returns (O, S_new)."""
    C = K.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Kd = K * Gam
    Ki = K * np.exp(-G)
    Qd = Q * Gam
    Kc = K * np.exp(G[-1][None, :] - G)
    A = np.tril(beta[:, None] * (Kd @ Ki.T), -1)
    T = np.eye(C) + A
    W = solve_triangular(T, beta[:, None] * Kd, lower=True, unit_diagonal=True)
    U0 = solve_triangular(T, beta[:, None] * V, lower=True, unit_diagonal=True)
    U = U0 - W @ S
    P = np.tril(Qd @ Ki.T)
    O = Qd @ S + P @ U
    S_new = Gam[-1][:, None] * S + Kc.T @ U
    return O, S_new


def prefill(q, k, v, g, beta, cu_seqlens, *, chunk=64, initial_state=None, ckpt_interval=0):
    """Same contract as oracle.recurrence.prefill (all outputs fp64)."""
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    gf = np.asarray(g, np.float64)
    bf = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N, H, Dk = qf.shape
    Dv = vf.shape[2]
    nseq = len(cu) - 1
    o = np.zeros((N, H, Dv))
    final = np.zeros((nseq, H, Dk, Dv))
    ckpts = []
    for s in range(nseq):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        seq_ck = []
        for h in range(H):
            S = np.zeros((Dk, Dv)) if initial_state is None else \
                np.asarray(initial_state[s, h], np.float64).copy()
            c0 = t0
            head_ck = []
            while c0 < t1:
                c1 = min(c0 + chunk, t1)
                if ckpt_interval > 0:
                    nxt = t0 + ((c0 - t0) // ckpt_interval + 1) * ckpt_interval
                    c1 = min(c1, nxt)
                O, S = chunk_step(S, qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, h],
                                  gf[c0:c1, h], bf[c0:c1, h])
                o[c0:c1, h] = O
                if ckpt_interval > 0 and (c1 - t0) % ckpt_interval == 0:
                    head_ck.append(S.copy())
                c0 = c1
            final[s, h] = S
            seq_ck.append(head_ck)
        if ckpt_interval > 0:
            for m in range(len(seq_ck[0]) if seq_ck else 0):
                ckpts.append(np.stack([seq_ck[h][m] for h in range(H)]))
    ck = np.stack(ckpts) if ckpts else (np.zeros((0, H, Dk, Dv)) if ckpt_interval > 0 else None)
    return dict(o=o, final=final, ckpt=ck)
