"""CPU pins of the oracle's parameter-free front-end (oracle/frontend.py):
closed forms of each transform, and the composition with the recurrence
checked against the recurrence on inputs transformed by hand."""

import math

import numpy as np
import pytest

from oracle import frontend as fe
from oracle import recurrence
from synth import decode_state, decode_step_inputs, make_prefill


def test_l2norm_pythagorean_row():
    # (3, 4) has norm 5: unit row (0.6, 0.8); EPS moves it by ~EPS / 50
    got = fe.l2norm(np.array([[3.0, 4.0]]))
    assert np.abs(got - np.array([[0.6, 0.8]])).max() < 1e-7


def test_l2norm_unit_norm_scale_invariance_and_zero_row():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 3, 128))
    y = fe.l2norm(x)
    assert np.abs(np.linalg.norm(y, axis=-1) - 1.0).max() < 1e-7
    # EPS inside the root shifts a row by EPS / (2 |x|^2) relative; |x|^2 ~ 128
    bound = fe.EPS / (2 * np.min(np.sum(x * x, -1)))
    assert np.abs(fe.l2norm(9.5 * x) - y).max() < 1.5 * bound
    assert np.array_equal(fe.l2norm(np.zeros((2, 64))), np.zeros((2, 64)))


def test_l2norm_reads_bf16_bits():
    # bf16 0x4040 = 3.0, 0x4080 = 4.0
    got = fe.l2norm(np.array([[0x4040, 0x4080]], dtype=np.uint16))
    assert np.abs(got - np.array([[0.6, 0.8]])).max() < 1e-7


def test_gate_closed_forms():
    assert fe.gate(np.array([0.0]))[0] == -1.0
    assert abs(fe.gate(np.array([math.log(2.0)]))[0] + 2.0) < 1e-15
    u = np.linspace(-8, 3, 50)
    a = np.exp(fe.gate(u))
    assert np.all((a > 0) & (a < 1)) and np.all(np.diff(a) < 0)


def test_sigmoid_closed_forms():
    assert fe.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(fe.sigmoid(np.array([math.log(3.0)]))[0] - 0.75) < 1e-15
    x = np.linspace(-30, 30, 121)
    assert np.abs(fe.sigmoid(x) + fe.sigmoid(-x) - 1.0).max() < 1e-15
    ext = fe.sigmoid(np.array([-800.0, 800.0]))
    assert ext[0] == 0.0 and ext[1] == 1.0


def _hand_raw(x, scale=3.7):
    """Raw inputs whose front-end result is x's plain inputs: q, k scaled away
    from unit norm, u = log(-g), b = logit(beta)."""
    q = fe.to_f64(x.q) * scale
    k = fe.to_f64(x.k) / scale
    u = np.log(-x.g.astype(np.float64))
    b = np.log(x.beta.astype(np.float64) / (1.0 - x.beta.astype(np.float64)))
    return q, k, u, b


@pytest.mark.parametrize("flags", [fe.FRONT_ALL, fe.FRONT_L2NORM_QK, fe.FRONT_GATE,
                                   fe.FRONT_BETA_SIGMOID])
def test_front_end_then_recurrence_matches_plain(flags):
    # plain inputs are unit rows (to storage precision), g < 0, beta in (0, 1)
    x = make_prefill([90, 40], 2, 16, 8, "f32", 31, init_state=True)
    q_raw, k_raw, u, b = _hand_raw(x)
    q_in = q_raw if flags & fe.FRONT_L2NORM_QK else fe.to_f64(x.q)
    k_in = k_raw if flags & fe.FRONT_L2NORM_QK else fe.to_f64(x.k)
    g_in = u if flags & fe.FRONT_GATE else x.g.astype(np.float64)
    b_in = b if flags & fe.FRONT_BETA_SIGMOID else x.beta.astype(np.float64)
    q, k, v, g, beta = fe.apply(q_in, k_in, x.v, g_in, b_in, flags)
    got = recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state)
    # the plain path on the same (storage-rounded, hence not exactly unit) rows:
    # renormalise them by hand so both sides see the same vectors
    qp, kp = fe.to_f64(x.q), fe.to_f64(x.k)
    if flags & fe.FRONT_L2NORM_QK:
        qp = qp / np.sqrt(np.sum(qp * qp, -1, keepdims=True) + fe.EPS / 3.7 ** 2)
        kp = kp / np.sqrt(np.sum(kp * kp, -1, keepdims=True) + fe.EPS * 3.7 ** 2)
    ref = recurrence.prefill(qp, kp, fe.to_f64(x.v), x.g.astype(np.float64),
                             x.beta.astype(np.float64), x.cu_seqlens,
                             initial_state=x.initial_state)
    scale = np.abs(ref["o"]).max()
    assert np.abs(got["o"] - ref["o"]).max() < 1e-12 * scale
    assert np.abs(got["final"] - ref["final"]).max() < 1e-12 * np.abs(ref["final"]).max()


def test_front_end_is_not_interchangeable():
    """Each transform lands on its own input: swapping gate and sigmoid, or
    skipping the normalisation, changes the outputs well beyond rounding."""
    x = make_prefill([64], 1, 16, 8, "f32", 32, raw=True, init_state=False)
    ok = fe.apply(x.q, x.k, x.v, x.g, x.beta, fe.FRONT_ALL)
    r_ok = recurrence.prefill(*ok, x.cu_seqlens)["o"]
    q, k, v, g, beta = ok
    swapped = (q, k, v, np.log(fe.sigmoid(x.g)), np.exp(fe.gate(x.beta)))
    r_sw = recurrence.prefill(*swapped, x.cu_seqlens)["o"]
    no_norm = fe.apply(x.q, x.k, x.v, x.g, x.beta, fe.FRONT_GATE | fe.FRONT_BETA_SIGMOID)
    r_nn = recurrence.prefill(*no_norm, x.cu_seqlens)["o"]
    s = np.abs(r_ok).max()
    assert np.abs(r_sw - r_ok).max() > 1e-2 * s
    assert np.abs(r_nn - r_ok).max() > 1e-2 * s


def test_decode_front_end_matches_plain():
    B, H, D = 3, 2, 16
    st = decode_state(B, H, D, D, 33).astype(np.float64)
    x = decode_step_inputs(B, H, D, D, "f32", 33, 0)
    q_raw = fe.to_f64(x.q) * 2.5
    k_raw = fe.to_f64(x.k) * 0.4
    u = np.log(-x.g.astype(np.float64))
    b = np.log(x.beta.astype(np.float64) / (1.0 - x.beta.astype(np.float64)))
    s1 = st.copy()
    o1 = recurrence.decode(*fe.apply(q_raw, k_raw, x.v, u, b, fe.FRONT_ALL), s1)
    qp, kp = fe.to_f64(x.q), fe.to_f64(x.k)
    qp = qp / np.sqrt(np.sum(qp * qp, -1, keepdims=True) + fe.EPS / 2.5 ** 2)
    kp = kp / np.sqrt(np.sum(kp * kp, -1, keepdims=True) + fe.EPS / 0.4 ** 2)
    s2 = st.copy()
    o2 = recurrence.decode(qp, kp, fe.to_f64(x.v), x.g.astype(np.float64),
                           x.beta.astype(np.float64), s2)
    assert np.abs(o1 - o2).max() < 1e-12 * np.abs(o2).max()
    assert np.abs(s1 - s2).max() < 1e-12 * np.abs(s2).max()


def test_raw_recipe_reproduces_plain_recipe():
    """The raw draws are the plain recipe's draws before its last step: the
    front-end applied to them gives the plain inputs up to storage rounding."""
    a = make_prefill([70], 2, 32, 8, "f32", 34)
    b = make_prefill([70], 2, 32, 8, "f32", 34, raw=True)
    q, k, v, g, beta = fe.apply(b.q, b.k, b.v, b.g, b.beta, fe.FRONT_ALL)
    assert np.abs(q - a.q).max() < 1e-6 and np.abs(k - a.k).max() < 1e-6
    assert np.abs(g - a.g).max() < 1e-7 * np.abs(a.g).max() + 1e-9
    assert np.abs(beta - a.beta).max() < 1e-7
    assert np.array_equal(v, a.v.astype(np.float64))
