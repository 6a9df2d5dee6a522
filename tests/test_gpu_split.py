"""GPU parity of the chunk-parallel scan (one sequence, few heads) against the
fp64 oracle, through the C ABI.

kda_prefill_chunked cuts such a sequence into segments of whole chunks,
scans them at once (values, and the identity for each segment's linear map),
chains the segment end states and corrects the outputs. The same inputs run
through the plain path (prepare and scan as two calls) must agree with the
oracle too."""

import numpy as np
import pytest

from helpers import assert_parity, dev_tensor
from oracle import recurrence
from synth import make_prefill

pytestmark = pytest.mark.gpu

CASES = [  # H, Dk, Dv, dtype, T, initial state
    (4, 128, 128, "bf16", 8192, True),
    (1, 128, 128, "bf16", 4133, True),
    (5, 128, 64, "bf16", 3072, True),
    (3, 64, 128, "bf16", 5000, False),
    (2, 64, 64, "f32", 4000, False),
    (2, 128, 128, "f32", 3300, True),
    # both scans in one launch (bf16, Dk == Dv) from three segments on
    (8, 128, 128, "bf16", 4096, True),
    (10, 128, 128, "bf16", 2048, True),
    (6, 64, 64, "bf16", 3000, False),
]


def run(x, *, phases=None, final=True):
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import _binding as B
    q, k, v, g, beta = (dev_tensor(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    s0 = dev_tensor(x.initial_state) if x.initial_state is not None else None
    if phases is None:
        o, fs, _ = K.kda_prefill_chunked(q, k, v, g, beta, initial_state=s0,
                                         output_final_state=final)
    else:  # prepare and scan as two calls: always the plain scan
        ws = torch.empty(K.kda_prefill_workspace_size(x.total_tokens, 1, x.H, x.Dk, x.Dv, q.dtype),
                         dtype=torch.uint8, device=q.device)
        o = torch.empty(x.total_tokens, x.H, x.Dv, device=q.device)
        fs = torch.empty(1, x.H, x.Dk, x.Dv, device=q.device)
        for p in (B.PHASE_PREPARE, B.PHASE_SCAN):
            K.kda_prefill_chunked(q, k, v, g, beta, initial_state=s0, final_state=fs, o=o,
                                  workspace=ws, phases=p)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (None if fs is None else fs.cpu().numpy())


def segments(x):
    import torch
    import linear_attention_05_amd as K
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    return K.kda_prefill_scan_segments(x.total_tokens, 1, x.H, x.Dk, x.Dv, dt)


@pytest.mark.parametrize("H,Dk,Dv,dtype,T,init", CASES)
def test_split_matches_oracle(H, Dk, Dv, dtype, T, init):
    x = make_prefill([T], H, Dk, Dv, dtype, 700 + T % 97 + H, init_state=init)
    P = segments(x)
    print(f"split prefill H={H} Dk={Dk} Dv={Dv} {dtype} T={T} init={init}: {P} segments",
          flush=True)
    assert P >= (3 if dtype == "bf16" and Dk == Dv else 6), \
        "these sizes should take the chunk-parallel scan"
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    o, fs = run(x)
    assert_parity(o, r["o"], dtype, "split o")
    assert_parity(fs, r["final"], dtype, "split final state")
    o2, fs2 = run(x, phases="split calls")
    assert_parity(o2, r["o"], dtype, "plain o")
    assert_parity(fs2, r["final"], dtype, "plain final state")


def test_split_without_final_state():
    x = make_prefill([3100], 2, 128, 128, "bf16", 771, init_state=True)
    assert segments(x) >= 6
    o, fs = run(x, final=False)
    assert fs is None
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    assert_parity(o, r["o"], "bf16", "split o, no final state")


def test_segment_rule():
    """The headline shape (32 heads) fills the device with the plain scan;
    short sequences and varlen batches never split; bf16 with Dk == Dv (both
    scans in one launch) splits from three segments, other inputs from six."""
    import torch
    import linear_attention_05_amd as K
    bf = torch.bfloat16
    assert K.kda_prefill_scan_segments(8192, 1, 32, 128, 128, bf) == 1
    assert K.kda_prefill_scan_segments(1024, 1, 1, 128, 128, bf) == 1
    assert K.kda_prefill_scan_segments(8192, 2, 1, 128, 128, bf) == 1
    assert K.kda_prefill_scan_segments(8192, 1, 4, 128, 128, bf) == 8
    assert K.kda_prefill_scan_segments(65536, 1, 8, 128, 128, bf) == 4
    assert K.kda_prefill_scan_segments(65536, 1, 10, 128, 128, bf) == 3
    assert K.kda_prefill_scan_segments(65536, 1, 16, 128, 128, bf) == 1
    assert K.kda_prefill_scan_segments(65536, 1, 8, 128, 128, torch.float32) == 1
    assert K.kda_prefill_scan_segments(65536, 1, 8, 128, 64, bf) == 1
    assert K.kda_prefill_scan_segments(65536, 1, 1, 128, 128, bf) == 16
    assert K.kda_prefill_scan_segments(8192, 1, 1, 128, 128, bf, chunk_size=32) == 0


def test_split_with_frontend():
    """Raw inputs with the in-kernel front-end (K1 applies it; the scans and the
    split path see the same handoff as for transformed inputs)."""
    import torch
    import linear_attention_05_amd as K
    from oracle import frontend as fe
    raw = make_prefill([4100], 2, 128, 128, "bf16", 781, raw=True)
    plain = make_prefill([4100], 2, 128, 128, "bf16", 781, init_state=True)
    assert segments(plain) >= 6
    q, k, v, g, beta = (dev_tensor(a) for a in (raw.q, raw.k, raw.v, raw.g, raw.beta))
    o, fs, _ = K.kda_prefill_chunked(q, k, v, g, beta, initial_state=dev_tensor(plain.initial_state),
                                     frontend=fe.FRONT_ALL)
    torch.cuda.synchronize()
    r = recurrence.prefill(*fe.apply(raw.q, raw.k, raw.v, raw.g, raw.beta, fe.FRONT_ALL),
                           raw.cu_seqlens, initial_state=plain.initial_state)
    assert_parity(o.cpu().numpy(), r["o"], "bf16", "split o, front-end")
    assert_parity(fs.cpu().numpy(), r["final"], "bf16", "split final state, front-end")


def test_split_large_states_f32():
    """fp32 inputs have no fp16 range limit: with v and S0 scaled by 2^18 the
    states reach ~1e5-1e6, beyond fp16, and the combine and the correction
    (split fp16 products) must still give 2^18 times the unscaled result
    (the recurrence is linear in (v, S0); scaling by a power of two is exact)."""
    c = 2.0 ** 18
    x = make_prefill([4096], 2, 128, 128, "f32", 4711, init_state=True)
    assert segments(x) >= 6
    big = make_prefill([4096], 2, 128, 128, "f32", 4711, init_state=True)
    big.v[...] = x.v * c
    big.initial_state[...] = x.initial_state * c
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    o, fs = run(big)
    assert np.abs(fs).max() > 65504.0, "the states should exceed the fp16 range"
    assert_parity(o / c, r["o"], "f32", "split o, states beyond fp16")
    assert_parity(fs / c, r["final"], "f32", "split final state, states beyond fp16")


@pytest.mark.parametrize("H,seed", [(4, 4242), (1, 4243)])
def test_split_full_size_sampled(H, seed):
    """The few-head workloads bench.py times (B=1, T=65536, D=128, bf16, S0),
    through the chunk-parallel scan, on (head, 16-column) units the oracle
    computes one by one over all 65536 tokens."""
    T, D = 65536, 128
    x = make_prefill([T], H, D, D, "bf16", seed, init_state=True)
    P = segments(x)
    print(f"split full-size H={H} T={T}: {P} segments", flush=True)
    assert P >= 8
    o, fs = run(x)
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    units = sorted({(0, 0, 0), (0, H - 1, D // 16 - 1), (0, H // 2, 3)})
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state,
                           units=np.array(units, dtype=np.int32), col_block=16)
    go, ro, gf, rf = [], [], [], []
    for _, h, cb in units:
        cols = slice(16 * cb, 16 * cb + 16)
        go.append(o[:, h, cols].ravel())
        ro.append(r["o"][:, h, cols].ravel())
        gf.append(fs[0, h, :, cols].ravel())
        rf.append(r["final"][0, h, :, cols].ravel())
    res = (assert_parity(np.concatenate(go), np.concatenate(ro), "bf16", "o (sampled)"),
           assert_parity(np.concatenate(gf), np.concatenate(rf), "bf16", "final (sampled)"))
    print(res, flush=True)


def _split_config(seed):
    rng = np.random.default_rng([910, seed])
    H = int(rng.integers(1, 6))
    Dk, Dv = (int(rng.choice([64, 128])), int(rng.choice([64, 128])))
    T = int(rng.integers(2048, 9000))
    dtype = str(rng.choice(["f32", "bf16"]))
    init = bool(rng.random() < 0.7)
    front = int(rng.integers(0, 8))
    return H, Dk, Dv, T, dtype, init, front


@pytest.mark.parametrize("seed", range(12))
def test_split_random_configuration(seed):
    """Seeded random one-sequence configurations (heads, head dimensions, length,
    dtype, initial state, front-end bits); the ones the rule sends to the
    chunk-parallel scan are compared with the oracle on every output."""
    import torch
    import linear_attention_05_amd as K
    from oracle import frontend as fe
    from synth.inputs import PrefillInputs
    H, Dk, Dv, T, dtype, init, front = _split_config(seed)
    plain = make_prefill([T], H, Dk, Dv, dtype, 3000 + seed, init_state=init)
    raw = make_prefill([T], H, Dk, Dv, dtype, 3000 + seed, raw=True, init_state=init)
    pick = lambda bit, name: getattr(raw if front & bit else plain, name)
    x = PrefillInputs(dtype, H, Dk, Dv, [T], pick(fe.FRONT_L2NORM_QK, "q"),
                      pick(fe.FRONT_L2NORM_QK, "k"), plain.v, pick(fe.FRONT_GATE, "g"),
                      pick(fe.FRONT_BETA_SIGMOID, "beta"), plain.initial_state)
    P = segments(x)
    print(f"split random seed {seed}: H={H} Dk={Dk} Dv={Dv} T={T} {dtype} init={init} "
          f"front={front}: {P} segments", flush=True)
    s0 = dev_tensor(x.initial_state) if init else None
    o, fs, _ = K.kda_prefill_chunked(dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v),
                                     dev_tensor(x.g), dev_tensor(x.beta), initial_state=s0,
                                     frontend=front)
    torch.cuda.synchronize()
    r = recurrence.prefill(*fe.apply(x.q, x.k, x.v, x.g, x.beta, front), x.cu_seqlens,
                           initial_state=x.initial_state if init else None)
    assert_parity(o.cpu().numpy(), r["o"], dtype, "o")
    assert_parity(fs.cpu().numpy(), r["final"], dtype, "final state")
