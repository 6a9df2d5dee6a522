"""Seeded random sweep of the prefill entry points: mixed sequence counts and
lengths (empty and ragged included), head counts, head dimensions, dtypes,
initial states, checkpoint intervals, front-end bits and requested
positions, each compared with the oracle on every output."""

import numpy as np
import pytest

from helpers import assert_parity, dev_tensor
from oracle import frontend as fe
from oracle import recurrence
from synth import make_prefill
from synth.inputs import PrefillInputs

pytestmark = pytest.mark.gpu


def _config(seed):
    rng = np.random.default_rng([900, seed])
    nseq = int(rng.integers(1, 7))
    lengths = [int(x) for x in rng.integers(0, 400, size=nseq)]
    if rng.random() < 0.3:
        lengths[int(rng.integers(nseq))] = 0
    H = int(rng.integers(1, 6))
    Dk, Dv = (int(rng.choice([64, 128])), int(rng.choice([64, 128])))
    dtype = str(rng.choice(["f32", "bf16"]))
    init = bool(rng.random() < 0.7)
    ckpt = int(rng.choice([0, 0, 64, 128]))
    front = int(rng.integers(0, 8))
    positions = [sorted(int(p) for p in rng.integers(0, L + 1, size=int(rng.integers(0, 4))))
                 for L in lengths]
    return lengths, H, Dk, Dv, dtype, init, ckpt, front, positions


@pytest.mark.parametrize("seed", range(48))
def test_random_prefill_configuration(seed):
    import torch
    import linear_attention_05_amd as K
    lengths, H, Dk, Dv, dtype, init, ckpt, front, positions = _config(seed)
    print(f"random prefill seed {seed}: lengths={lengths} H={H} Dk={Dk} Dv={Dv} {dtype} "
          f"init={init} ckpt={ckpt} front={front} positions={positions}", flush=True)
    # raw draws only where a front-end bit transforms them (untransformed raw
    # keys, decays or logits are outside the recurrence's preconditions)
    kw = dict(init_state=init, ckpt_interval=ckpt)
    plain = make_prefill(lengths, H, Dk, Dv, dtype, 2000 + seed, **kw)
    raw = make_prefill(lengths, H, Dk, Dv, dtype, 2000 + seed, raw=True, **kw)
    pick = lambda bit, name: getattr(raw if front & bit else plain, name)
    x = PrefillInputs(dtype, H, Dk, Dv, lengths, pick(fe.FRONT_L2NORM_QK, "q"),
                      pick(fe.FRONT_L2NORM_QK, "k"), plain.v, pick(fe.FRONT_GATE, "g"),
                      pick(fe.FRONT_BETA_SIGMOID, "beta"), plain.initial_state,
                      ckpt_interval=ckpt)
    offs = np.zeros(len(lengths) + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(p) for p in positions])
    vals = np.array([p for ps in positions for p in ps], dtype=np.int32)
    s0 = dev_tensor(x.initial_state) if init else None
    o, fs, ck, ps = K.kda_prefill_chunked_at(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        dev_tensor(offs), dev_tensor(vals), cu_seqlens=dev_tensor(x.cu_seqlens),
        initial_state=s0, ckpt_interval=ckpt, num_checkpoints=x.num_checkpoints(),
        frontend=front)
    torch.cuda.synchronize()

    q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    r = recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state,
                           ckpt_interval=ckpt)
    assert_parity(o.cpu().numpy(), r["o"], dtype, "o")
    assert_parity(fs.cpu().numpy(), r["final"], dtype, "final")
    if ckpt and r["ckpt"].size:
        assert_parity(ck.cpu().numpy(), r["ckpt"], dtype, "checkpoints")
    if vals.size:
        ref = []
        for s, plist in enumerate(positions):
            a = int(x.cu_seqlens[s])
            for P in plist:
                rp = recurrence.prefill(q[a:a + P], k[a:a + P], v[a:a + P], g[a:a + P],
                                        beta[a:a + P], np.array([0, P]),
                                        initial_state=x.initial_state[s:s + 1] if init else None)
                ref.append(rp["final"][0])
        assert_parity(ps.cpu().numpy(), np.stack(ref), dtype, "positions")


def _strong_g(x, seed):
    """A copy of x.g in which each head has a random number of channels (0 to
    all of them, a few small counts likelier) drawing g = -U(0.5, 20) per
    token: diagonal 16-token blocks then take every product form K1 has
    (shared reference row, slow channels apart, four levels)."""
    rng = np.random.default_rng([901, seed])
    g = x.g.copy()
    N, H, D = g.shape
    for h in range(H):
        n = int(rng.choice([0, 1, 2, 5, 16, 17, int(rng.integers(0, D + 1)), D]))
        ch = rng.choice(D, size=n, replace=False)
        g[:, h, ch] = -rng.uniform(0.5, 20.0, size=(N, n)).astype(np.float32)
    return g


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_strong_decay(seed):
    """The random configurations above (without the gate transform, whose raw
    input replaces g) with fast-decaying channels per head."""
    import torch
    import linear_attention_05_amd as K
    lengths, H, Dk, Dv, dtype, init, ckpt, front, _ = _config(seed)
    front &= ~fe.FRONT_GATE
    kw = dict(init_state=init, ckpt_interval=ckpt)
    plain = make_prefill(lengths, H, Dk, Dv, dtype, 3000 + seed, **kw)
    raw = make_prefill(lengths, H, Dk, Dv, dtype, 3000 + seed, raw=True, **kw)
    pick = lambda bit, name: getattr(raw if front & bit else plain, name)
    x = PrefillInputs(dtype, H, Dk, Dv, lengths, pick(fe.FRONT_L2NORM_QK, "q"),
                      pick(fe.FRONT_L2NORM_QK, "k"), plain.v, _strong_g(plain, seed),
                      pick(fe.FRONT_BETA_SIGMOID, "beta"), plain.initial_state,
                      ckpt_interval=ckpt)
    print(f"random strong-decay prefill seed {seed}: lengths={lengths} H={H} Dk={Dk} Dv={Dv} "
          f"{dtype} init={init} ckpt={ckpt} front={front}", flush=True)
    s0 = dev_tensor(x.initial_state) if init else None
    o, fs, ck = K.kda_prefill_chunked(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        cu_seqlens=dev_tensor(x.cu_seqlens), initial_state=s0, ckpt_interval=ckpt,
        num_checkpoints=x.num_checkpoints(), frontend=front)
    torch.cuda.synchronize()
    q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    r = recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state,
                           ckpt_interval=ckpt)
    assert_parity(o.cpu().numpy(), r["o"], dtype, "o")
    assert_parity(fs.cpu().numpy(), r["final"], dtype, "final")
    if ckpt and r["ckpt"].size:
        assert_parity(ck.cpu().numpy(), r["ckpt"], dtype, "checkpoints")
