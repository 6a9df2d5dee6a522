"""GPU parity of the in-kernel parameter-free front-end (kda_prefill_chunked_ex,
kda_decode_step_ex: q/k L2 normalisation, gate g = -exp(u), sigmoid write
strength) against the oracle's fp64 front-end followed by its recurrence."""

import numpy as np
import pytest

from helpers import assert_parity, dev_tensor
from oracle import frontend as fe
from oracle import recurrence
from synth import decode_state, decode_step_inputs, make_prefill
from synth.inputs import PrefillInputs

pytestmark = pytest.mark.gpu

ALL = fe.FRONT_ALL


def gpu_prefill(x, front, *, phases=3, workspace=None, o=None, final_state=None):
    import torch
    import linear_attention_05_amd as K
    s0 = dev_tensor(x.initial_state) if x.initial_state is not None else None
    o, fs, ck = K.kda_prefill_chunked(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        cu_seqlens=dev_tensor(x.cu_seqlens), initial_state=s0, ckpt_interval=x.ckpt_interval,
        num_checkpoints=x.num_checkpoints(), workspace=workspace, o=o, final_state=final_state,
        phases=phases, frontend=front)
    torch.cuda.synchronize()
    return o, fs, ck


def oracle(x, front, units=None):
    q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    return recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state,
                              ckpt_interval=x.ckpt_interval, units=units)


def check(x, front, what):
    print(f"front-end prefill {what}: front={front} lengths={x.lengths[:8]} H={x.H} "
          f"Dk={x.Dk} Dv={x.Dv} {x.dtype}", flush=True)
    o, fs, ck = gpu_prefill(x, front)
    r = oracle(x, front)
    assert_parity(o.cpu().numpy(), r["o"], x.dtype, f"{what} o")
    assert_parity(fs.cpu().numpy(), r["final"], x.dtype, f"{what} final")
    if x.ckpt_interval and r["ckpt"].size:
        assert_parity(ck.cpu().numpy(), r["ckpt"], x.dtype, f"{what} checkpoints")


def mixed(lengths, H, Dk, Dv, dtype, seed, front, **kw):
    """Raw inputs where `front` transforms them, plain inputs elsewhere."""
    raw = make_prefill(lengths, H, Dk, Dv, dtype, seed, raw=True, **kw)
    plain = make_prefill(lengths, H, Dk, Dv, dtype, seed, **kw)
    pick = lambda bit, a, b: a if front & bit else b
    return PrefillInputs(dtype, H, Dk, Dv, list(lengths),
                         pick(fe.FRONT_L2NORM_QK, raw.q, plain.q),
                         pick(fe.FRONT_L2NORM_QK, raw.k, plain.k), plain.v,
                         pick(fe.FRONT_GATE, raw.g, plain.g),
                         pick(fe.FRONT_BETA_SIGMOID, raw.beta, plain.beta),
                         plain.initial_state, ckpt_interval=plain.ckpt_interval)


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_all_transforms_varlen_tails(Dk, Dv, dtype):
    x = make_prefill([100, 0, 64, 1, 257, 33], 3, Dk, Dv, dtype, 41, raw=True)
    check(x, ALL, "all")


@pytest.mark.parametrize("front", [fe.FRONT_L2NORM_QK, fe.FRONT_GATE, fe.FRONT_BETA_SIGMOID,
                                   fe.FRONT_GATE | fe.FRONT_BETA_SIGMOID])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_each_transform(front, dtype):
    check(mixed([200, 65], 2, 128, 128, dtype, 42, front), front, "one transform")


def test_prefill_checkpoints_several_chunks():
    x = make_prefill([600, 256], 4, 128, 128, "bf16", 43, raw=True, ckpt_interval=128)
    check(x, ALL, "checkpoints")


def test_prefill_zero_and_tiny_rows():
    """All-zero q/k rows stay zero; rows of very different scales normalise alike."""
    x = make_prefill([130, 70], 2, 128, 128, "f32", 44, raw=True)
    x.q[5] = 0.0
    x.k[17] = 0.0
    x.k[40] *= 1e-3
    x.q[41] *= 1e3
    check(x, ALL, "zero rows")


def test_prefill_split_phases_match_single_call_bitwise():
    """PREPARE applies the front-end; a following SCAN-only call ignores it."""
    import torch
    x = make_prefill([300, 90], 2, 128, 128, "bf16", 45, raw=True)
    o1, f1, _ = gpu_prefill(x, ALL)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    f2 = torch.empty_like(f1)
    gpu_prefill(x, ALL, phases=1, workspace=ws, o=o2, final_state=f2)
    gpu_prefill(x, 0, phases=2, workspace=ws, o=o2, final_state=f2)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_prefill_headline_shape_sampled():
    """T = 8192, H = 32, D = 128, bf16 raw inputs, in the launch configuration of
    the benchmark; 24 random (head, 16-column block) units checked on every token."""
    x = make_prefill([8192], 32, 128, 128, "bf16", 1001, raw=True)
    o, fs, _ = gpu_prefill(x, ALL)
    rng = np.random.default_rng(46)
    units = np.array([(0, h, cb) for h, cb in zip(rng.choice(32, 24), rng.choice(8, 24))])
    r = oracle(x, ALL, units=units)
    o = o.cpu().numpy()
    fs = fs.cpu().numpy()
    for _, h, cb in units:
        cols = slice(16 * cb, 16 * cb + 16)
        assert_parity(o[:, h, cols], r["o"][:, h, cols], "bf16", f"o head {h} cols {cb}")
        assert_parity(fs[0, h, :, cols], r["final"][0, h, :, cols], "bf16",
                      f"final head {h} cols {cb}")


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_all_transforms(Dk, Dv, dtype):
    import torch
    import linear_attention_05_amd as K
    B, H = 5, 3
    st = decode_state(B, H, Dk, Dv, 47)
    ref = st.astype(np.float64)
    dstate = dev_tensor(st)
    for step in range(3):
        x = decode_step_inputs(B, H, Dk, Dv, dtype, 47, step, raw=True)
        print(f"front-end decode Dk={Dk} Dv={Dv} {dtype} step {step}", flush=True)
        o = K.kda_decode_step(dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v),
                              dev_tensor(x.g), dev_tensor(x.beta), dstate, frontend=ALL)
        torch.cuda.synchronize()
        ro = recurrence.decode(*fe.apply(x.q, x.k, x.v, x.g, x.beta, ALL), ref)
        assert_parity(o.cpu().numpy(), ro, dtype, f"decode o step {step}")
    assert_parity(dstate.cpu().numpy(), ref, dtype, "decode state")


@pytest.mark.parametrize("front", [fe.FRONT_L2NORM_QK, fe.FRONT_GATE, fe.FRONT_BETA_SIGMOID])
def test_decode_each_transform(front):
    import torch
    import linear_attention_05_amd as K
    B, H, D = 4, 2, 128
    st = decode_state(B, H, D, D, 48)
    raw = decode_step_inputs(B, H, D, D, "bf16", 48, 0, raw=True)
    plain = decode_step_inputs(B, H, D, D, "bf16", 48, 0)
    pick = lambda bit, a, b: a if front & bit else b
    q = pick(fe.FRONT_L2NORM_QK, raw.q, plain.q)
    k = pick(fe.FRONT_L2NORM_QK, raw.k, plain.k)
    g = pick(fe.FRONT_GATE, raw.g, plain.g)
    beta = pick(fe.FRONT_BETA_SIGMOID, raw.beta, plain.beta)
    dstate = dev_tensor(st)
    o = K.kda_decode_step(dev_tensor(q), dev_tensor(k), dev_tensor(plain.v), dev_tensor(g),
                          dev_tensor(beta), dstate, frontend=front)
    torch.cuda.synchronize()
    ref = st.astype(np.float64)
    ro = recurrence.decode(*fe.apply(q, k, plain.v, g, beta, front), ref)
    assert_parity(o.cpu().numpy(), ro, "bf16", "decode o")
    assert_parity(dstate.cpu().numpy(), ref, "bf16", "decode state")
