"""Seeded synthetic inputs for the KDA core (prefill and decode).

This module only draws and casts random numbers. It contains none of the
recurrence's arithmetic, and both the GPU library's tests/benchmark and the
CPU oracle consume exactly the arrays it returns.

Distributions (one recipe for every workload):
  * q, k ~ N(0, 1) per element, then L2-normalised over the key channels of
    each (token, head) in fp64 (the pages list L2 normalisation of queries and
    keys as part of KDA: Kimi K3 report, "Methodology notes", Kimi Delta
    Attention bullet), then cast to the storage dtype.
  * v ~ N(0, 1).
  * log-decay g = -exp(u), u ~ N(-4, 0.5)  (so alpha = exp(g) in (0, 1)).
  * beta = sigmoid(x), x ~ N(0, 1).
  * initial recurrent states ~ N(0, 0.02) (standard deviation 0.02), fp32.
  * N(mu, s) always names the standard deviation s.

Raw variant (raw=True, for the library's in-kernel front-end): the same
streams with the last step of each recipe left out -- q, k ~ N(0, 1) cast
to the storage dtype without normalisation, g holds u itself (fp32) and beta
holds x itself (fp32).

Casting: fp64 -> fp32 with round-to-nearest-even (numpy astype); bf16 tensors
are then rounded fp32 -> bf16 with round-to-nearest-even and are returned as
raw uint16 bit patterns.

Random streams: every (tensor, token block) pair owns an independent PCG64
stream seeded with [seed, tensor_tag, block_index], so the draw does not
depend on how many threads generate it. Token blocks are BLOCK_TOKENS long.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_TOKENS = 1024

# tensor tags of the random streams
TAG_LEN, TAG_Q, TAG_K, TAG_V, TAG_U, TAG_B, TAG_S0 = 1, 2, 3, 4, 5, 6, 7

DECAY_MU, DECAY_SIGMA = -4.0, 0.5
STATE_SIGMA = 0.02


def _pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- casting ---

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> storage dtype ('f32' -> float32, 'bf16' -> uint16 bits)."""
    f32 = x64.astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact fp32 view of its values."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


# --------------------------------------------------------- block drawing ---

def _fill_blocked(shape_tail, n_tok, seed, tag, make_block, out_dtype):
    """Fill an [n_tok, *shape_tail] array block by block in a thread pool.

    make_block(rng, nb) returns the block's values already cast."""
    out = np.empty((n_tok,) + tuple(shape_tail), dtype=out_dtype)
    nblk = (n_tok + BLOCK_TOKENS - 1) // BLOCK_TOKENS

    def work(b):
        t0 = b * BLOCK_TOKENS
        nb = min(BLOCK_TOKENS, n_tok - t0)
        rng = np.random.default_rng([seed, tag, b])
        out[t0:t0 + nb] = make_block(rng, nb)

    if nblk <= 1:
        for b in range(nblk):
            work(b)
    else:
        with ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def _unit_rows(rng, nb, H, D):
    x = rng.standard_normal((nb, H, D))
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x


def draw_qk(n_tok, H, D, seed, tag, dtype):
    st = np.uint16 if dtype == "bf16" else np.float32
    return _fill_blocked((H, D), n_tok, seed, tag,
                         lambda r, nb: to_storage(_unit_rows(r, nb, H, D), dtype), st)


def draw_qk_raw(n_tok, H, D, seed, tag, dtype):
    st = np.uint16 if dtype == "bf16" else np.float32
    return _fill_blocked((H, D), n_tok, seed, tag,
                         lambda r, nb: to_storage(r.standard_normal((nb, H, D)), dtype), st)


def draw_u(n_tok, H, D, seed, tag=TAG_U):
    return _fill_blocked((H, D), n_tok, seed, tag,
                         lambda r, nb: r.normal(DECAY_MU, DECAY_SIGMA, size=(nb, H, D)).astype(np.float32),
                         np.float32)


def draw_beta_logits(n_tok, H, seed, tag=TAG_B):
    return _fill_blocked((H,), n_tok, seed, tag,
                         lambda r, nb: r.standard_normal((nb, H)).astype(np.float32), np.float32)


def draw_v(n_tok, H, D, seed, dtype, tag=TAG_V):
    st = np.uint16 if dtype == "bf16" else np.float32
    return _fill_blocked((H, D), n_tok, seed, tag,
                         lambda r, nb: to_storage(r.standard_normal((nb, H, D)), dtype), st)


def draw_g(n_tok, H, D, seed, tag=TAG_U):
    def blk(r, nb):
        u = r.normal(DECAY_MU, DECAY_SIGMA, size=(nb, H, D))
        return (-np.exp(u)).astype(np.float32)
    return _fill_blocked((H, D), n_tok, seed, tag, blk, np.float32)


def draw_beta(n_tok, H, seed, tag=TAG_B):
    def blk(r, nb):
        x = r.standard_normal((nb, H))
        return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
    return _fill_blocked((H,), n_tok, seed, tag, blk, np.float32)


def draw_states(n, H, Dk, Dv, seed, tag=TAG_S0):
    """[n, H, Dk, Dv] fp32 ~ N(0, STATE_SIGMA); stream per leading index."""
    out = np.empty((n, H, Dk, Dv), dtype=np.float32)

    def work(i):
        rng = np.random.default_rng([seed, tag, i])
        out[i] = rng.normal(0.0, STATE_SIGMA, size=(H, Dk, Dv)).astype(np.float32)

    if n > 1:
        with ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(work, range(n)))
    elif n == 1:
        work(0)
    return out


# ------------------------------------------------------------ workloads ---

@dataclass
class PrefillInputs:
    """One prefill problem. q/k/v are uint16 bf16 bits or float32.

    lengths: per-sequence token counts, packed back to back along tokens.
    cu_seqlens: int32 [num_seqs + 1] prefix sums of lengths."""
    dtype: str
    H: int
    Dk: int
    Dv: int
    lengths: list
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    initial_state: np.ndarray | None
    ckpt_interval: int = 0
    chunk_size: int = 64
    seed: int = 0
    name: str = ""
    cu_seqlens: np.ndarray = field(init=False)

    def __post_init__(self):
        self.cu_seqlens = np.zeros(len(self.lengths) + 1, dtype=np.int32)
        acc = 0
        for i, L in enumerate(self.lengths):
            acc += int(L)
            self.cu_seqlens[i + 1] = acc

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    def num_checkpoints(self) -> int:
        if self.ckpt_interval <= 0:
            return 0
        return int(sum(L // self.ckpt_interval for L in self.lengths))


def make_prefill(lengths, H, Dk, Dv, dtype, seed, *, init_state=True,
                 ckpt_interval=0, chunk_size=64, name="", raw=False) -> PrefillInputs:
    """raw=True: q, k un-normalised, g = u and beta = x (see the module notes)."""
    lengths = [int(L) for L in lengths]
    n_tok = sum(lengths)
    if raw:
        q = draw_qk_raw(n_tok, H, Dk, seed, TAG_Q, dtype)
        k = draw_qk_raw(n_tok, H, Dk, seed, TAG_K, dtype)
        g = draw_u(n_tok, H, Dk, seed)
        beta = draw_beta_logits(n_tok, H, seed)
    else:
        q = draw_qk(n_tok, H, Dk, seed, TAG_Q, dtype)
        k = draw_qk(n_tok, H, Dk, seed, TAG_K, dtype)
        g = draw_g(n_tok, H, Dk, seed)
        beta = draw_beta(n_tok, H, seed)
    v = draw_v(n_tok, H, Dv, seed, dtype)
    s0 = draw_states(len(lengths), H, Dk, Dv, seed) if init_state else None
    return PrefillInputs(dtype, H, Dk, Dv, lengths, q, k, v, g, beta, s0,
                         ckpt_interval=ckpt_interval, chunk_size=chunk_size,
                         seed=seed, name=name)


def varlen_lengths(n, lo, hi, seed):
    """Log-uniform integer lengths in [lo, hi]: rint(exp(U(ln lo, ln hi)))."""
    rng = np.random.default_rng([seed, TAG_LEN])
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return [int(v) for v in np.clip(np.rint(x), lo, hi).astype(np.int64)]


# The five benchmark workloads of the KDA core; seed = 1000 + index.
WORKLOADS = {
    0: dict(kind="prefill", name="tiny fp32 prefill B=1 H=2 T=256 D=64",
            lengths=[256], H=2, D=64, dtype="f32", init_state=False, ckpt=0),
    1: dict(kind="prefill", name="prefill B=1 H=32 T=8192 D=128 bf16",
            lengths=[8192], H=32, D=128, dtype="bf16", init_state=True, ckpt=0),
    2: dict(kind="prefill", name="long prefill B=1 H=32 T=147456 D=128 bf16 ckpt/32768",
            lengths=[147456], H=32, D=128, dtype="bf16", init_state=False, ckpt=32768),
    3: dict(kind="prefill", name="varlen prefill 64 seqs log-uniform 128..16384 H=32 D=128 bf16",
            lengths=None, H=32, D=128, dtype="bf16", init_state=True, ckpt=0),
    4: dict(kind="decode", name="decode B=512 H=32 D=128 bf16, 64 steps",
            B=512, H=32, D=128, dtype="bf16", steps=64),
}


def workload_seed(i: int) -> int:
    return 1000 + i


def workload_lengths(i: int):
    w = WORKLOADS[i]
    if w["lengths"] is not None:
        return list(w["lengths"])
    return varlen_lengths(64, 128, 16384, workload_seed(i))


def make_workload(i: int) -> PrefillInputs:
    w = WORKLOADS[i]
    assert w["kind"] == "prefill"
    return make_prefill(workload_lengths(i), w["H"], w["D"], w["D"], w["dtype"],
                        workload_seed(i), init_state=w["init_state"],
                        ckpt_interval=w["ckpt"], name=w["name"])


# ---------------------------------------------------------------- decode ---

@dataclass
class DecodeStep:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray


def decode_state(B, H, Dk, Dv, seed) -> np.ndarray:
    return draw_states(B, H, Dk, Dv, seed)


def decode_step_inputs(B, H, Dk, Dv, dtype, seed, step, raw=False) -> DecodeStep:
    """Inputs of one decode step: [B, H, D] tensors; the step index selects
    the stream block, so steps are independent draws. raw=True as in
    make_prefill."""
    def one(tag, fn):
        rng = np.random.default_rng([seed, tag, 1_000_000 + step])
        return fn(rng)
    if raw:
        q = one(TAG_Q, lambda r: to_storage(r.standard_normal((B, H, Dk)), dtype))
        k = one(TAG_K, lambda r: to_storage(r.standard_normal((B, H, Dk)), dtype))
        g = one(TAG_U, lambda r: r.normal(DECAY_MU, DECAY_SIGMA, size=(B, H, Dk)).astype(np.float32))
        beta = one(TAG_B, lambda r: r.standard_normal((B, H)).astype(np.float32))
    else:
        q = one(TAG_Q, lambda r: to_storage(_unit_rows(r, B, H, Dk), dtype))
        k = one(TAG_K, lambda r: to_storage(_unit_rows(r, B, H, Dk), dtype))
        g = one(TAG_U, lambda r: (-np.exp(r.normal(DECAY_MU, DECAY_SIGMA, size=(B, H, Dk)))).astype(np.float32))
        beta = one(TAG_B, lambda r: (1.0 / (1.0 + np.exp(-r.standard_normal((B, H))))).astype(np.float32))
    v = one(TAG_V, lambda r: to_storage(r.standard_normal((B, H, Dv)), dtype))
    return DecodeStep(q, k, v, g, beta)
