"""GPU parity of kda_prefill_chunked against the fp64 oracle (through the C ABI).

Every problem, the full-size workloads included, is compared element by
element on every output."""

import numpy as np
import pytest

from helpers import assert_parity, assert_parity_blocked, dev_tensor, errors
from oracle import recurrence
from synth import make_prefill, make_workload, WORKLOADS

pytestmark = pytest.mark.gpu


def gpu_prefill(x, *, final=True, ckpt=None, workspace=None, init=True):
    import torch
    import linear_attention_05_amd as K
    cu = dev_tensor(x.cu_seqlens)
    s0 = dev_tensor(x.initial_state) if (init and x.initial_state is not None) else None
    o, fs, ck = K.kda_prefill_chunked(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        cu_seqlens=cu, initial_state=s0, output_final_state=final,
        ckpt_interval=x.ckpt_interval, num_checkpoints=x.num_checkpoints(), workspace=workspace)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), None if fs is None else fs.cpu().numpy(),
            None if ck is None else ck.cpu().numpy())


def oracle_full(x):
    return recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                              initial_state=x.initial_state, ckpt_interval=x.ckpt_interval)


def check_full(x, what):
    print(f"prefill {what}: lengths={x.lengths[:8]} H={x.H} Dk={x.Dk} Dv={x.Dv} {x.dtype}",
          flush=True)
    o, fs, ck = gpu_prefill(x)
    r = oracle_full(x)
    res = {"o": assert_parity(o, r["o"], x.dtype, f"{what} o"),
           "final": assert_parity(fs, r["final"], x.dtype, f"{what} final")}
    if x.ckpt_interval:
        assert ck.shape == r["ckpt"].shape
        if ck.size:
            res["ckpt"] = assert_parity(ck, r["ckpt"], x.dtype, f"{what} checkpoints")
    return res


def test_tiny_fp32_workload():
    """fp32 inputs, B=1, H=2, T=256, D=64, zero initial state: 1e-5 bar."""
    check_full(make_workload(0), "tiny fp32")


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_tails_small(Dk, Dv, dtype):
    x = make_prefill([100, 0, 64, 1, 257, 33], 3, Dk, Dv, dtype, 31, init_state=True)
    check_full(x, "varlen tails")


def test_single_sequence_bf16_several_chunks():
    x = make_prefill([1000], 4, 128, 128, "bf16", 32, init_state=True)
    check_full(x, "single seq")


@pytest.mark.parametrize("interval", [64, 128])
def test_checkpoints_small(interval):
    x = make_prefill([256, 200, 64, 0, 130], 2, 128, 128, "bf16", 33, init_state=True,
                     ckpt_interval=interval)
    check_full(x, f"checkpoints/{interval}")


def test_no_initial_state_and_no_final():
    x = make_prefill([190, 70], 2, 128, 128, "bf16", 34, init_state=False)
    o, fs, _ = gpu_prefill(x, final=False)
    assert fs is None
    r = oracle_full(x)
    assert_parity(o, r["o"], "bf16", "o")


def test_zero_tokens_returns_initial_state():
    x = make_prefill([0, 0], 2, 64, 64, "f32", 35, init_state=True)
    o, fs, _ = gpu_prefill(x)
    assert o.shape == (0, 2, 64)
    assert np.array_equal(fs, x.initial_state)


def test_deterministic_and_packing_invariant():
    """Bitwise: run-to-run, and a packed batch == each sequence on its own."""
    x = make_prefill([150, 64, 77], 2, 128, 128, "bf16", 36, init_state=True)
    o1, f1, _ = gpu_prefill(x)
    o2, f2, _ = gpu_prefill(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    from synth.inputs import PrefillInputs
    cu = x.cu_seqlens
    for s in range(x.num_seqs):
        a, b = cu[s], cu[s + 1]
        one = PrefillInputs("bf16", 2, 128, 128, [int(b - a)], x.q[a:b], x.k[a:b], x.v[a:b],
                            x.g[a:b], x.beta[a:b], x.initial_state[s:s + 1])
        oo, ff, _ = gpu_prefill(one)
        assert np.array_equal(oo, o1[a:b])
        assert np.array_equal(ff[0], f1[s])


def test_resume_from_checkpoint_bitwise():
    """prefill(prefix) -> state -> prefill(rest, initial = state) == prefill(whole),
    when the prefix ends on a chunk boundary."""
    from synth.inputs import PrefillInputs
    x = make_prefill([320], 2, 128, 128, "bf16", 37, init_state=True)
    o, f, _ = gpu_prefill(x)
    sl = slice(0, 128), slice(128, 320)
    pre = PrefillInputs("bf16", 2, 128, 128, [128], *(a[sl[0]] for a in (x.q, x.k, x.v, x.g, x.beta)),
                        x.initial_state)
    o1, f1, _ = gpu_prefill(pre)
    rest = PrefillInputs("bf16", 2, 128, 128, [192], *(a[sl[1]] for a in (x.q, x.k, x.v, x.g, x.beta)),
                         f1)
    o2, f2, _ = gpu_prefill(rest)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(f2, f)


def test_prefill_matches_decode_steps():
    import torch
    import linear_attention_05_amd as K
    x = make_prefill([70], 2, 128, 128, "bf16", 38, init_state=True)
    o, f, _ = gpu_prefill(x)
    st = dev_tensor(x.initial_state)
    outs = []
    for t in range(70):
        sl = slice(t, t + 1)
        outs.append(K.kda_decode_step(dev_tensor(x.q[sl]), dev_tensor(x.k[sl]), dev_tensor(x.v[sl]),
                                      dev_tensor(x.g[sl]), dev_tensor(x.beta[sl]), st).cpu().numpy())
    torch.cuda.synchronize()
    od = np.concatenate(outs)
    ma, rf = errors(o, od)
    assert ma < 2e-3 and rf < 1e-3, (ma, rf)
    ma, rf = errors(f, st.cpu().numpy())
    assert ma < 2e-3 and rf < 1e-3, (ma, rf)


def check_workload(x):
    """Every output element of a full-size workload against the oracle (the
    oracle runs over all sequences, heads and columns; the comparison goes
    head block by head block to bound host memory)."""
    print(f"prefill full-size {x.name}: tokens={x.total_tokens} seqs={x.num_seqs}", flush=True)
    o, fs, ck = gpu_prefill(x)
    print("  gpu done; oracle over all outputs", flush=True)
    r = oracle_full(x)
    res = {"o": assert_parity_blocked(o, r["o"], x.dtype, "o", axis=1),
           "final": assert_parity_blocked(fs, r["final"], x.dtype, "final", axis=1)}
    if x.ckpt_interval:
        assert ck.shape == r["ckpt"].shape
        res["ckpt"] = assert_parity_blocked(ck, r["ckpt"], x.dtype, "checkpoints", axis=1)
    print(res, flush=True)
    return res


def test_workload_prefill_8k():
    check_workload(make_workload(1))


def test_workload_long_context_checkpoints():
    x = make_workload(2)
    assert x.num_checkpoints() == 4
    check_workload(x)


def test_workload_varlen_64_sequences():
    x = make_workload(3)
    assert x.num_seqs == 64 and min(x.lengths) >= 128 and max(x.lengths) <= 16384
    check_workload(x)


def _with(x, **arrays):
    from synth.inputs import PrefillInputs
    d = dict(dtype=x.dtype, H=x.H, Dk=x.Dk, Dv=x.Dv, lengths=x.lengths, q=x.q, k=x.k, v=x.v,
             g=x.g, beta=x.beta, initial_state=x.initial_state, ckpt_interval=x.ckpt_interval)
    d.update(arrays)
    return PrefillInputs(**d)


def test_strong_decay_within_precondition():
    """Per-channel decay up to ~0.5 nats per token (about 8 nats over 16
    tokens, inside the fp16 operand-range precondition), mixed with weak
    channels."""
    x = make_prefill([300, 129], 2, 128, 128, "bf16", 40, init_state=True)
    rng = np.random.default_rng(41)
    strong = -rng.uniform(0.05, 0.5, size=x.g.shape).astype(np.float32)
    mask = rng.random(size=(1, 1, x.Dk)) < 0.5
    g = np.where(mask, strong, x.g).astype(np.float32)
    check_full(_with(x, g=g), "strong decay")


def test_full_write_strength():
    x = make_prefill([256, 77], 2, 128, 128, "bf16", 42, init_state=True)
    check_full(_with(x, beta=np.ones_like(x.beta)), "beta=1")


def test_identity_keeps_state_exactly():
    """alpha = 1 (g = 0) and beta = 0: every chunk update adds exactly zero,
    so the final state equals the initial state bit for bit; o = S0^T q."""
    x = make_prefill([200, 64], 2, 128, 128, "bf16", 43, init_state=True)
    y = _with(x, g=np.zeros_like(x.g), beta=np.zeros_like(x.beta))
    o, fs, _ = gpu_prefill(y)
    assert np.array_equal(fs, y.initial_state)
    r = oracle_full(y)
    assert_parity(o, r["o"], "bf16", "identity o")


def test_many_short_sequences():
    """More sequences than one scan tile of the prep kernel (varlen tables
    built across several 256-wide passes), lengths 0..70."""
    rng = np.random.default_rng(44)
    lengths = [int(v) for v in rng.integers(0, 71, size=600)]
    x = make_prefill(lengths, 2, 64, 64, "bf16", 45, init_state=True, ckpt_interval=64)
    check_full(x, "600 sequences")


def test_twenty_thousand_short_sequences():
    """20,000 sequences of 0..100 tokens (three tiles of the varlen prep
    kernel's offset scans and length-class sort): every output against the
    oracle; a sequence left out of, or counted twice in, the scan order would
    leave its outputs and final state unwritten or wrong."""
    rng = np.random.default_rng(48)
    lengths = [int(v) for v in rng.integers(0, 101, size=20000)]
    x = make_prefill(lengths, 1, 64, 64, "bf16", 49, init_state=True, ckpt_interval=64)
    check_full(x, "20000 sequences")


def test_long_tail_with_checkpoints():
    x = make_prefill([64 * 37 + 19, 64 * 5], 2, 128, 128, "bf16", 46, init_state=True,
                     ckpt_interval=128)
    check_full(x, "long tail + checkpoints")


@pytest.mark.parametrize("Dk,Dv,nseq", [(128, 128, 2), (64, 64, 3), (128, 64, 3), (64, 128, 2)])
def test_pair_counts_between_designs(Dk, Dv, nseq):
    """32 heads and two or three sequences: on a 256-CU device these counts of
    (sequence, head) pairs select the scan whose two column blocks share one
    CU's operand stream; checked in full against the oracle."""
    lengths = [700, 333, 517][:nseq]
    x = make_prefill(lengths, 32, Dk, Dv, "bf16", 47, init_state=True, ckpt_interval=128)
    check_full(x, f"{nseq} seqs x 32 heads")
