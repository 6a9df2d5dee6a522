"""GPU parity over KDA's full per-channel decay range (Kimi K3 report,
"Methodology notes", Kimi Delta Attention: the forget gate is a diagonal,
per-channel matrix, so single channels may forget almost everything in one
token). The decays here reach alpha = e^-30 per token on whole channels,
alpha = e^-1e4 (zero in fp64) on isolated tokens and channels, alpha = 0
(g = -inf) on whole tokens, and stretches where every channel forgets: each
case against the fp64 oracle, element by element, through every scan design,
positions inside chunks, the chunk-parallel scan, the decode step and the
in-kernel front-end."""

import numpy as np
import pytest

from helpers import assert_parity, dev_tensor
from oracle import frontend as fe
from oracle import recurrence
from synth import make_prefill, decode_state, decode_step_inputs
from synth.inputs import PrefillInputs

pytestmark = pytest.mark.gpu

PATTERNS = ["mixed", "isolated", "stretch", "threshold", "few"]


def strong_g(x, pattern, seed):
    """A copy of x.g with strong decay written in (values only; no arithmetic
    of the method). mixed: half the channels draw g = -U(0.5, 30) per token.
    isolated: 1% of (token, head, channel) entries and 2% of whole tokens get
    g = -1e4. stretch: in every sequence longer than 60 tokens, all channels
    of 40 tokens get g = -1e4 and one token after them g = -inf. threshold:
    every channel a constant g per token, in [-0.55, -0.40] on even heads and
    [-0.70, -0.56] on odd heads: just below and just above the 16-token decay
    (2^12) at which a diagonal block changes its product form. few: on head h,
    FEW[h % 6] channels draw g = -U(0.8, 20) per token (a block with at most
    16 such channels sums their pairs apart from the others; 17 is the first
    count past that)."""
    rng = np.random.default_rng(seed)
    g = x.g.copy()
    N, H, D = g.shape
    if pattern == "mixed":
        ch = rng.random(D) < 0.5
        g[:, :, ch] = -rng.uniform(0.5, 30.0, size=(N, H, int(ch.sum()))).astype(np.float32)
    elif pattern == "isolated":
        g[rng.random((N, H, D)) < 0.01] = -1e4
        if N:
            g[rng.choice(N, size=max(1, N // 50), replace=False)] = -1e4
    elif pattern == "stretch":
        cu = x.cu_seqlens
        for s in range(x.num_seqs):
            a, L = int(cu[s]), int(cu[s + 1] - cu[s])
            if L > 60:
                t = a + L // 3 - 20 if L > 120 else a + 10
                g[t:t + 40] = -1e4
                g[t + 45] = -np.inf
    elif pattern == "threshold":
        for h in range(H):  # even heads just below the change, odd heads just above
            lo, hi = (0.40, 0.55) if h % 2 == 0 else (0.56, 0.70)
            g[:, h, :] = -rng.uniform(lo, hi, size=(1, D)).astype(np.float32)
    elif pattern == "few":
        for h in range(H):
            ch = rng.choice(D, size=FEW[h % len(FEW)], replace=False)
            g[:, h, ch] = -rng.uniform(0.8, 20.0, size=(N, len(ch))).astype(np.float32)
    else:
        raise ValueError(pattern)
    return g


FEW = [3, 17, 16, 1, 33, 8]


def with_g(x, g):
    return PrefillInputs(x.dtype, x.H, x.Dk, x.Dv, x.lengths, x.q, x.k, x.v, g, x.beta,
                         x.initial_state, ckpt_interval=x.ckpt_interval)


def gpu_prefill(x):
    import torch
    import linear_attention_05_amd as K
    s0 = dev_tensor(x.initial_state) if x.initial_state is not None else None
    o, fs, ck = K.kda_prefill_chunked(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        cu_seqlens=dev_tensor(x.cu_seqlens), initial_state=s0, ckpt_interval=x.ckpt_interval,
        num_checkpoints=x.num_checkpoints())
    torch.cuda.synchronize()
    return o.cpu().numpy(), fs.cpu().numpy(), None if ck is None else ck.cpu().numpy()


def check(x, what):
    print(f"decay range {what}: seqs={x.num_seqs} tokens={x.total_tokens} H={x.H} "
          f"Dk={x.Dk} Dv={x.Dv} {x.dtype}", flush=True)
    o, fs, ck = gpu_prefill(x)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state, ckpt_interval=x.ckpt_interval)
    assert_parity(o, r["o"], x.dtype, f"{what} o")
    assert_parity(fs, r["final"], x.dtype, f"{what} final")
    if x.ckpt_interval and r["ckpt"].size:
        assert_parity(ck, r["ckpt"], x.dtype, f"{what} checkpoints")


# (lengths, H, Dk, Dv, dtype): on a 256-CU device these sizes select the
# three-wave scan (few pairs), the five-wave scan (64 pairs), the 64-column
# four-wave scan (600 pairs) and, for fp32 inputs, the fp32 scan.
def _many(n, seed):
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.integers(0, 141, size=n)]


DESIGNS = {
    "trio": ([300, 129], 2, 128, 128, "bf16"),
    "trio-d64": ([300, 129], 2, 64, 64, "bf16"),
    "quad": ([700, 333], 32, 128, 128, "bf16"),
    "nt4": (_many(300, 5), 2, 128, 128, "bf16"),
    "fp32": ([300, 129], 2, 128, 128, "f32"),
    "fp32-d64": ([300, 129], 2, 64, 64, "f32"),
}


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("design", list(DESIGNS))
def test_decay_range_every_scan(design, pattern):
    lengths, H, Dk, Dv, dtype = DESIGNS[design]
    x = make_prefill(lengths, H, Dk, Dv, dtype, 900 + len(design), init_state=True,
                     ckpt_interval=128)
    check(with_g(x, strong_g(x, pattern, 17)), f"{design}/{pattern}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pattern", ["mixed", "stretch", "few"])
def test_decay_range_positions(dtype, pattern):
    from test_gpu_positions import gpu_at, oracle_states
    x = make_prefill([300, 129, 70], 2, 128, 128, dtype, 910, init_state=True)
    x = with_g(x, strong_g(x, pattern, 18))
    positions = [[0, 1, 63, 64, 65, 150, 299, 300], [100, 129], [7, 70]]
    print(f"decay range positions {dtype}/{pattern}", flush=True)
    o, fs, _, ps = gpu_at(x, positions)
    assert_parity(ps.cpu().numpy(), oracle_states(x, positions), dtype, "position states")
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    assert_parity(o.cpu().numpy(), r["o"], dtype, "o")
    assert_parity(fs.cpu().numpy(), r["final"], dtype, "final")


@pytest.mark.parametrize("H,Dk,Dv,dtype,T", [(1, 128, 128, "bf16", 4133), (2, 64, 64, "f32", 4000)])
@pytest.mark.parametrize("pattern", ["mixed", "stretch", "few"])
def test_decay_range_chunk_parallel_scan(H, Dk, Dv, dtype, T, pattern):
    from test_gpu_split import run, segments
    x = make_prefill([T], H, Dk, Dv, dtype, 920 + H, init_state=True)
    x = with_g(x, strong_g(x, pattern, 19))
    P = segments(x)
    print(f"decay range split {dtype}/{pattern}: T={T} H={H} P={P}", flush=True)
    assert P >= 6
    o, fs = run(x)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    assert_parity(o, r["o"], dtype, "split o")
    assert_parity(fs, r["final"], dtype, "split final")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decay_range_decode(dtype):
    import torch
    import linear_attention_05_amd as K
    B, H, D = 8, 2, 128
    s0 = decode_state(B, H, D, D, 930)
    st = dev_tensor(s0)
    ref = s0.astype(np.float64).copy()
    rng = np.random.default_rng(931)
    for t in range(12):
        d = decode_step_inputs(B, H, D, D, dtype, 930, t)
        g = d.g.copy()
        g[:, :, rng.random(D) < 0.5] = -rng.uniform(0.5, 30.0)
        g[rng.random(g.shape) < 0.05] = -1e4
        if t == 5:
            g[:] = -np.inf
        og = K.kda_decode_step(dev_tensor(d.q), dev_tensor(d.k), dev_tensor(d.v),
                               dev_tensor(g), dev_tensor(d.beta), st)
        orf = recurrence.decode(d.q, d.k, d.v, g, d.beta, ref)
        torch.cuda.synchronize()
        assert_parity(og.cpu().numpy(), orf, dtype, f"decode step {t} o")
    assert_parity(st.cpu().numpy(), ref, dtype, "decode state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_front_end_gate_strong(dtype):
    """Raw gate inputs u ~ N(0, 1) (g = -exp(u), often below -1 per token)
    with every front-end transform applied in-kernel."""
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import _binding as Bd
    x = make_prefill([300, 129], 2, 128, 128, dtype, 940, init_state=True, raw=True)
    u = np.random.default_rng(941).standard_normal(x.g.shape).astype(np.float32)
    x = with_g(x, u)
    front = Bd.FRONT_ALL
    print(f"front-end gate strong {dtype}", flush=True)
    o, fs, _ = K.kda_prefill_chunked(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        cu_seqlens=dev_tensor(x.cu_seqlens), initial_state=dev_tensor(x.initial_state),
        frontend=front)
    torch.cuda.synchronize()
    q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    r = recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state)
    assert_parity(o.cpu().numpy(), r["o"], dtype, "o")
    assert_parity(fs.cpu().numpy(), r["final"], dtype, "final")


def test_prefill_matches_decode_steps_strong_decay():
    """The two paths of the library agree under strong decay too."""
    import torch
    import linear_attention_05_amd as K
    x = make_prefill([150], 2, 128, 128, "bf16", 950, init_state=True)
    x = with_g(x, strong_g(x, "stretch", 20))
    o, f, _ = gpu_prefill(x)
    st = dev_tensor(x.initial_state)
    outs = []
    for t in range(x.total_tokens):
        sl = slice(t, t + 1)
        outs.append(K.kda_decode_step(dev_tensor(x.q[sl]), dev_tensor(x.k[sl]), dev_tensor(x.v[sl]),
                                      dev_tensor(x.g[sl]), dev_tensor(x.beta[sl]), st).cpu().numpy())
    torch.cuda.synchronize()
    assert_parity(o, np.concatenate(outs), "bf16", "prefill vs decode o")
    assert_parity(f, st.cpu().numpy(), "bf16", "prefill vs decode state")
