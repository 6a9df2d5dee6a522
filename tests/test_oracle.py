"""CPU tests of the oracle against its pins (facts independent of its code),
the chunked formulation, and structural invariances."""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import chunked, recurrence
from synth import make_prefill, decode_state, decode_step_inputs


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(recurrence)


def _max_rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-30)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 10_000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_matches_recurrence(chunk, dtype):
    # varlen with tails: lengths not multiples of any chunk, one empty sequence
    x = make_prefill([100, 37, 0, 64, 129], 2, 16, 8, dtype, 21, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state, col_block=4)
    c = chunked.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, chunk=chunk,
                        initial_state=x.initial_state)
    assert _max_rel(c["o"], r["o"]) < 1e-12
    assert _max_rel(c["final"], r["final"]) < 1e-12


def test_chunked_matches_recurrence_checkpoints():
    x = make_prefill([200, 64, 130], 2, 16, 16, "bf16", 22, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state, ckpt_interval=64)
    c = chunked.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, chunk=48,
                        initial_state=x.initial_state, ckpt_interval=64)
    assert r["ckpt"].shape == (3 + 1 + 2, 2, 16, 16)
    assert _max_rel(c["ckpt"], r["ckpt"]) < 1e-12
    assert _max_rel(c["o"], r["o"]) < 1e-12


def test_chunked_full_width_c0_shape():
    """The tiny fp32 workload's shape (H=2, T=256, D=64) at C=64."""
    x = make_prefill([256], 2, 64, 64, "f32", 1000, init_state=False)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    c = chunked.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, chunk=64)
    assert _max_rel(c["o"], r["o"]) < 1e-12
    assert _max_rel(c["final"], r["final"]) < 1e-12


def test_packing_invariance_bitwise():
    """A packed varlen batch equals running each sequence on its own."""
    x = make_prefill([50, 0, 77, 31], 2, 8, 8, "bf16", 23, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    cu = x.cu_seqlens
    for s in range(x.num_seqs):
        a, b = cu[s], cu[s + 1]
        one = recurrence.prefill(x.q[a:b], x.k[a:b], x.v[a:b], x.g[a:b], x.beta[a:b],
                                 [0, b - a], initial_state=x.initial_state[s:s + 1])
        assert np.array_equal(one["o"], r["o"][a:b])
        assert np.array_equal(one["final"][0], r["final"][s])


def test_empty_sequence_returns_initial_state():
    x = make_prefill([0, 5], 2, 8, 8, "f32", 24, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    assert np.array_equal(r["final"][0], x.initial_state[0].astype(np.float64))


def test_column_block_and_thread_invariance_bitwise():
    x = make_prefill([150, 70], 3, 16, 16, "bf16", 25, init_state=True)
    ref = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                             initial_state=x.initial_state, col_block=16, n_threads=1)
    for cb, nt in [(1, 8), (5, 3), (16, 8)]:
        r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                               initial_state=x.initial_state, col_block=cb, n_threads=nt)
        assert np.array_equal(r["o"], ref["o"])
        assert np.array_equal(r["final"], ref["final"])


def test_units_subset_bitwise():
    x = make_prefill([40, 90], 2, 8, 16, "bf16", 26, init_state=True)
    ref = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                             initial_state=x.initial_state, col_block=4)
    units = np.array([[1, 0, 2], [0, 1, 3]])
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state, col_block=4, units=units)
    a, b = x.cu_seqlens[1], x.cu_seqlens[2]
    assert np.array_equal(r["o"][a:b, 0, 8:12], ref["o"][a:b, 0, 8:12])
    assert np.array_equal(r["final"][1, 0, :, 8:12], ref["final"][1, 0, :, 8:12])
    assert np.array_equal(r["final"][0, 1, :, 12:16], ref["final"][0, 1, :, 12:16])
    assert np.isnan(r["o"][a:b, 1]).all()


def test_checkpoint_equals_prefix_final_and_resume():
    x = make_prefill([256], 2, 8, 8, "bf16", 27, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state, ckpt_interval=64)
    assert r["ckpt"].shape[0] == 4
    for m in range(1, 5):
        L = 64 * m
        p = recurrence.prefill(x.q[:L], x.k[:L], x.v[:L], x.g[:L], x.beta[:L], [0, L],
                               initial_state=x.initial_state)
        assert np.array_equal(p["final"], r["ckpt"][m - 1:m])
    assert np.array_equal(r["ckpt"][-1:], r["final"])
    # resume from the (fp32-rounded) checkpoint after 128 tokens
    s_mid = r["ckpt"][1:2].astype(np.float32)
    rest = recurrence.prefill(x.q[128:], x.k[128:], x.v[128:], x.g[128:], x.beta[128:],
                              [0, 128], initial_state=s_mid)
    assert _max_rel(rest["o"], r["o"][128:]) < 1e-6
    assert _max_rel(rest["final"], r["final"]) < 1e-6


def test_decode_steps_equal_prefill_bitwise():
    """T decode steps on one sequence perform the prefill's exact operations."""
    x = make_prefill([12], 2, 8, 8, "bf16", 28, init_state=True)
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                           initial_state=x.initial_state)
    state = x.initial_state.astype(np.float64).copy()                 # [1, H, Dk, Dv]
    for t in range(12):
        o = recurrence.decode(x.q[t:t + 1], x.k[t:t + 1], x.v[t:t + 1], x.g[t:t + 1],
                              x.beta[t:t + 1], state)
        assert np.array_equal(o[0], r["o"][t])
    assert np.array_equal(state, r["final"])


def test_decode_batch_rows_independent():
    B, H, D = 6, 2, 8
    s0 = decode_state(B, H, D, D, 29).astype(np.float64)
    st = decode_step_inputs(B, H, D, D, "bf16", 29, 0)
    full = s0.copy()
    o = recurrence.decode(st.q, st.k, st.v, st.g, st.beta, full)
    part = s0.copy()
    units = np.array([[4, 1, 0]])
    o2 = recurrence.decode(st.q, st.k, st.v, st.g, st.beta, part, units=units, col_block=8)
    assert np.array_equal(o2[4, 1], o[4, 1])
    assert np.array_equal(part[4, 1], full[4, 1])
    assert np.array_equal(part[0], s0[0])


@pytest.mark.parametrize("cut", [1, 40, 64, 129])
def test_segment_affine_decomposition(cut):
    """The chunk-parallel scan's decomposition, on the recurrence itself: a
    segment started from state X gives o = o(X = 0) + oI X and S_end = M X + F,
    where (oI, M) are the outputs and end state of the same segment run with
    zero values from the identity, and (o(X = 0), F) the run from zeros."""
    x = make_prefill([200], 2, 8, 6, "f32", 24, init_state=True)
    T, H, Dk, Dv = 200, 2, 8, 6
    full = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                              initial_state=x.initial_state)
    head = recurrence.prefill(x.q[:cut], x.k[:cut], x.v[:cut], x.g[:cut], x.beta[:cut],
                              np.array([0, cut]), initial_state=x.initial_state)
    X = head["final"][0]  # [H, Dk, Dv], the true start state of the tail segment
    tail = (x.q[cut:], x.k[cut:], x.v[cut:], x.g[cut:], x.beta[cut:])
    cu = np.array([0, T - cut])
    a = recurrence.prefill(*tail, cu)
    eye = np.broadcast_to(np.eye(Dk, dtype=np.float32), (1, H, Dk, Dk)).copy()
    zero_v = np.zeros((T - cut, H, Dk), dtype=np.float32)
    b = recurrence.prefill(tail[0], tail[1], zero_v, tail[3], tail[4], cu, initial_state=eye)
    o_rec = a["o"] + np.einsum("thk,hkv->thv", b["o"], X)
    s_rec = np.einsum("hij,hjv->hiv", b["final"][0], X) + a["final"][0]
    assert _max_rel(o_rec, full["o"][cut:]) < 1e-12
    assert _max_rel(s_rec, full["final"][0]) < 1e-12
    assert _max_rel(head["o"], full["o"][:cut]) == 0.0
