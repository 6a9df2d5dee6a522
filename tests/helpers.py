"""Shared test helpers: host<->device marshalling and the parity metric."""

from __future__ import annotations

import numpy as np

# Tolerances per output tensor: max |gpu - oracle| and ||gpu - oracle||_F / ||oracle||_F.
TOL = {"bf16": (2e-3, 1e-3), "f32": (1e-5, 1e-5)}


def dev_tensor(arr: np.ndarray, device="cuda"):
    """numpy storage array -> torch tensor on the GPU (uint16 arrays are bf16 bits)."""
    import torch
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values in GPU output"
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel_f = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel_f


def assert_parity(got, ref, dtype, what=""):
    max_abs, rel_f = errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    assert max_abs <= tol_abs and rel_f <= tol_rel, \
        f"{what}: max_abs {max_abs:.3e} (tol {tol_abs:g}), rel_F {rel_f:.3e} (tol {tol_rel:g})"
    return max_abs, rel_f


def assert_parity_blocked(got, ref, dtype, what="", axis=1, block=4):
    """assert_parity over the whole tensors, computed slice by slice along
    `axis` (bounded temporaries for multi-GB outputs): the same max |diff| and
    ||diff||_F / ||ref||_F as one pass would give."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n = got.shape[axis]
    max_abs, dd, rr = 0.0, 0.0, 0.0
    for a in range(0, n, block):
        idx = [slice(None)] * got.ndim
        idx[axis] = slice(a, min(a + block, n))
        g = np.asarray(got[tuple(idx)], dtype=np.float64)
        r = np.asarray(ref[tuple(idx)], dtype=np.float64)
        assert np.isfinite(g).all(), f"{what}: non-finite values in GPU output"
        d = g - r
        if d.size:
            max_abs = max(max_abs, float(np.abs(d).max()))
        dd += float(np.sum(d * d))
        rr += float(np.sum(r * r))
    rel_f = float(np.sqrt(dd / rr)) if rr > 0 else float(np.sqrt(dd))
    tol_abs, tol_rel = TOL[dtype]
    assert max_abs <= tol_abs and rel_f <= tol_rel, \
        f"{what}: max_abs {max_abs:.3e} (tol {tol_abs:g}), rel_F {rel_f:.3e} (tol {tol_rel:g})"
    return max_abs, rel_f
