"""ctypes wrapper of the fp64 C oracle (kda_oracle.c): the token-by-token KDA
recurrence S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
o_t = S_t^T q_t.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py)."""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
F32, BF16, F64 = 0, 1, 2


def load(path):
    """Load an oracle shared library built from kda_oracle.c (any path)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.kda_oracle_prefill.argtypes = [
        P, P, P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, P, P, ctypes.c_int64, P, P, P, ctypes.c_int64, ctypes.c_int,
        ctypes.c_int]
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [
        P, P, P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_num_threads.argtypes = [ctypes.c_int]
    lib.kda_oracle_num_threads.restype = ctypes.c_int
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _LIB = load(path)
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(arr):
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.float64:
        return F64
    raise TypeError(f"q/k/v must be float32, float64 or uint16 bf16 bits, got {arr.dtype}")


def _gb(x, dt):
    """g and beta travel as fp64 with fp64 q/k/v, as fp32 otherwise."""
    return np.ascontiguousarray(x, dtype=np.float64 if dt == F64 else np.float32)


def num_threads(n: int = 0) -> int:
    """Thread count the oracle runs with (n > 0 sets it)."""
    return _lib().kda_oracle_num_threads(int(n))


def prefill(q, k, v, g, beta, cu_seqlens, *, initial_state=None, ckpt_interval=0,
            units=None, col_block=16, n_threads=0, want_final=True, out=None,
            lib=None):
    """Run the recurrence over packed sequences.

    q, k: [N, H, Dk]; v: [N, H, Dv] (float32, uint16 bf16 bits or float64, one dtype);
    g: [N, H, Dk]; beta: [N, H] (float32; float64 when q/k/v are float64);
    cu_seqlens: [num_seqs + 1].
    initial_state: [num_seqs, H, Dk, Dv] float32 or None (zeros).
    units: optional int array [n, 3] of (seq, head, column block) to compute;
    outputs of other units stay NaN.
    Returns dict(o=[N,H,Dv] f64, final=[S,H,Dk,Dv] f64 | None, ckpt=[n,H,Dk,Dv] f64 | None).
    """
    q = np.ascontiguousarray(q); k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    g = _gb(g, dt)
    beta = _gb(beta, dt)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N, H, Dk = q.shape
    Dv = v.shape[2]
    S = len(cu) - 1
    if k.shape != (N, H, Dk) or v.shape[:2] != (N, H) or g.shape != (N, H, Dk) \
            or beta.shape != (N, H) or cu[-1] != N:
        raise ValueError("inconsistent shapes")
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float32)
        if s0.shape != (S, H, Dk, Dv):
            raise ValueError("initial_state shape")
    lengths = np.diff(cu)
    n_ck = int(np.sum(lengths // ckpt_interval)) if ckpt_interval > 0 else 0
    o = out if out is not None else np.full((N, H, Dv), np.nan)
    final = np.full((S, H, Dk, Dv), np.nan) if want_final else None
    ck = np.full((max(n_ck, 1), H, Dk, Dv), np.nan) if ckpt_interval > 0 else None
    u = None
    nu = 0
    if units is not None:
        u = np.ascontiguousarray(units, dtype=np.int32).reshape(-1, 3)
        nu = u.shape[0]
    rc = (lib or _lib()).kda_oracle_prefill(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(g), _ptr(beta), _ptr(cu), S, H, Dk, Dv,
        _ptr(s0), _ptr(final), int(ckpt_interval), _ptr(ck), _ptr(o), _ptr(u), nu,
        int(col_block), int(n_threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill failed")
    if ck is not None:
        ck = ck[:n_ck]
    return dict(o=o, final=final, ckpt=ck)


def decode(q, k, v, g, beta, state, *, units=None, col_block=16, n_threads=0, lib=None):
    """One decode step; state [B, H, Dk, Dv] float64 is updated in place.
    Returns o [B, H, Dv] float64 (NaN outside the listed units)."""
    q = np.ascontiguousarray(q); k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    g = _gb(g, dt)
    beta = _gb(beta, dt)
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array")
    B, H, Dk = q.shape
    Dv = v.shape[2]
    if state.shape != (B, H, Dk, Dv):
        raise ValueError("state shape")
    o = np.full((B, H, Dv), np.nan)
    u = None
    nu = 0
    if units is not None:
        u = np.ascontiguousarray(units, dtype=np.int32).reshape(-1, 3)
        nu = u.shape[0]
    rc = (lib or _lib()).kda_oracle_decode(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(g), _ptr(beta), B, H, Dk, Dv, _ptr(state),
        _ptr(o), _ptr(u), nu, int(col_block), int(n_threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode failed")
    return o
