"""GPU parity of kda_decode_step against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from helpers import assert_parity, assert_parity_blocked, dev_tensor
from oracle import recurrence
from synth import decode_state, decode_step_inputs, WORKLOADS, workload_seed

pytestmark = pytest.mark.gpu


def _run_steps(B, H, Dk, Dv, dtype, seed, steps, sample_pairs=None):
    import torch
    import linear_attention_05_amd as K
    s0 = decode_state(B, H, Dk, Dv, seed)
    state = dev_tensor(s0)
    if sample_pairs is None:
        sample_pairs = [(b, h) for b in range(B) for h in range(H)]
    bs = np.array([p[0] for p in sample_pairs])
    hs = np.array([p[1] for p in sample_pairs])
    ref_state = s0[bs, hs][:, None].astype(np.float64).copy()   # [n, 1, Dk, Dv]
    o_gpu, o_ref = [], []
    for t in range(steps):
        x = decode_step_inputs(B, H, Dk, Dv, dtype, seed, t)
        o = K.kda_decode_step(dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v),
                              dev_tensor(x.g), dev_tensor(x.beta), state)
        o_gpu.append(o.cpu().numpy()[bs, hs])
        sub = lambda a: np.ascontiguousarray(a[bs, hs][:, None])
        o_ref.append(recurrence.decode(sub(x.q), sub(x.k), sub(x.v), sub(x.g), sub(x.beta),
                                       ref_state)[:, 0])
    torch.cuda.synchronize()
    fin = state.cpu().numpy()[bs, hs]
    return np.stack(o_gpu), np.stack(o_ref), fin, ref_state[:, 0]


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(Dk, Dv, dtype):
    print(f"decode small Dk={Dk} Dv={Dv} {dtype}", flush=True)
    og, orf, fg, fr = _run_steps(3, 5, Dk, Dv, dtype, 77, 6)
    assert_parity(og, orf, dtype, "o")
    assert_parity(fg, fr, dtype, "final state")


def test_decode_full_workload():
    """Batched decode workload: B=512, H=32, D=128, bf16, 64 in-place steps over
    the full 1 GiB state; every (b, h) pair's outputs of all 64 steps and its
    final state against the oracle."""
    import torch
    import linear_attention_05_amd as K
    w = WORKLOADS[4]
    B, H, D, steps = w["B"], w["H"], w["D"], w["steps"]
    seed = workload_seed(4)
    s0 = decode_state(B, H, D, D, seed)
    state = dev_tensor(s0)
    ref = s0.astype(np.float64)
    print(f"decode full B={B} H={H} D={D} steps={steps}", flush=True)
    og, orf = [], []
    for t in range(steps):
        x = decode_step_inputs(B, H, D, D, w["dtype"], seed, t)
        o = K.kda_decode_step(dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v),
                              dev_tensor(x.g), dev_tensor(x.beta), state)
        og.append(o.cpu().numpy())
        orf.append(recurrence.decode(x.q, x.k, x.v, x.g, x.beta, ref))
        if t % 16 == 15:
            print(f"  step {t + 1}", flush=True)
    torch.cuda.synchronize()
    print(assert_parity(np.stack(og), np.stack(orf), "bf16", "o (64 steps)"), flush=True)
    print(assert_parity_blocked(state.cpu().numpy(), ref, "bf16", "final state", axis=0,
                                block=64), flush=True)


def test_decode_deterministic_and_in_place():
    import torch
    import linear_attention_05_amd as K
    B, H, D = 4, 3, 128
    s0 = dev_tensor(decode_state(B, H, D, D, 9))
    x = decode_step_inputs(B, H, D, D, "bf16", 9, 0)
    args = [dev_tensor(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    s1, s2 = s0.clone(), s0.clone()
    o1 = K.kda_decode_step(*args, s1)
    o2 = K.kda_decode_step(*args, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert not torch.equal(s1, s0)


@pytest.mark.parametrize("front", [0, 7])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_decode_batch_invariant(Dk, Dv, dtype, front):
    """With fewer (b, h) pairs than 8 per CU the step splits each state's
    value columns over 2 or 4 workgroups, keeping the order of every
    reduction: a batch row's output and new state are bitwise the same in
    batches of 1 to 16 rows (four and two slices) as in a batch of 136 rows
    (4352 pairs, one workgroup each)."""
    import torch
    import linear_attention_05_amd as K
    H, Bbig = 32, 136
    print(f"decode batch invariance Dk={Dk} Dv={Dv} {dtype} front={front}", flush=True)
    s0 = decode_state(Bbig, H, Dk, Dv, 61)
    x = decode_step_inputs(Bbig, H, Dk, Dv, dtype, 61, 0)
    big = [dev_tensor(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    sb = dev_tensor(s0)
    ob = K.kda_decode_step(*big, sb, frontend=front)
    for b in (1, 2, 4, 8, 16):
        ss = dev_tensor(np.ascontiguousarray(s0[:b]))
        small = [dev_tensor(np.ascontiguousarray(a[:b])) for a in (x.q, x.k, x.v, x.g, x.beta)]
        os_ = K.kda_decode_step(*small, ss, frontend=front)
        torch.cuda.synchronize()
        assert torch.equal(os_, ob[:b]), f"o differs at batch {b}"
        assert torch.equal(ss, sb[:b]), f"state differs at batch {b}"
