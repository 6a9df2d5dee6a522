"""GPU parity of kda_prefill_chunked_at: states after the first P tokens of a
sequence, for arbitrary P. The oracle's value is its final state on the
sequence's first P tokens from the same initial state."""

import numpy as np
import pytest

from helpers import assert_parity, dev_tensor
from oracle import frontend as fe
from oracle import recurrence
from synth import make_prefill, make_workload
from synth.inputs import PrefillInputs

pytestmark = pytest.mark.gpu


def gpu_at(x, positions, *, front=0, phases=3, workspace=None, o=None, final_state=None,
           ckpt_states=None, pos_states=None):
    """positions: one list of token counts per sequence."""
    import torch
    import linear_attention_05_amd as K
    offs = np.zeros(x.num_seqs + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(p) for p in positions])
    vals = np.array([P for p in positions for P in p], dtype=np.int32)
    s0 = dev_tensor(x.initial_state) if x.initial_state is not None else None
    res = K.kda_prefill_chunked_at(
        dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v), dev_tensor(x.g), dev_tensor(x.beta),
        dev_tensor(offs), dev_tensor(vals), cu_seqlens=dev_tensor(x.cu_seqlens),
        initial_state=s0, ckpt_interval=x.ckpt_interval, num_checkpoints=x.num_checkpoints(),
        workspace=workspace, o=o, final_state=final_state, ckpt_states=ckpt_states,
        pos_states=pos_states, phases=phases, frontend=front)
    torch.cuda.synchronize()
    return res


def oracle_states(x, positions, front=0, units=None):
    """State after the first P tokens of each listed position, [num_pos, H, Dk, Dv]."""
    if front:
        q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    else:  # storage dtypes straight to the oracle (no fp64 copies of large inputs)
        q, k, v, g, beta = x.q, x.k, x.v, x.g, x.beta
    out = []
    for s, plist in enumerate(positions):
        a = int(x.cu_seqlens[s])
        L = int(x.cu_seqlens[s + 1]) - a
        s0 = x.initial_state[s:s + 1] if x.initial_state is not None else None
        for P in plist:
            P = min(max(int(P), 0), L)
            r = recurrence.prefill(q[a:a + P], k[a:a + P], v[a:a + P], g[a:a + P],
                                   beta[a:a + P], np.array([0, P]), initial_state=s0, units=units)
            out.append(r["final"][0])
    return np.stack(out) if out else np.zeros((0, x.H, x.Dk, x.Dv))


def check(x, positions, what, front=0):
    print(f"positions {what}: lengths={x.lengths[:8]} H={x.H} Dk={x.Dk} Dv={x.Dv} {x.dtype} "
          f"front={front} positions={positions[:4]}", flush=True)
    o, fs, ck, ps = gpu_at(x, positions, front=front)
    ref = oracle_states(x, positions, front)
    assert_parity(ps.cpu().numpy(), ref, x.dtype, f"{what} position states")
    # the other outputs are those of the plain call
    q, k, v, g, beta = fe.apply(x.q, x.k, x.v, x.g, x.beta, front)
    r = recurrence.prefill(q, k, v, g, beta, x.cu_seqlens, initial_state=x.initial_state,
                           ckpt_interval=x.ckpt_interval)
    assert_parity(o.cpu().numpy(), r["o"], x.dtype, f"{what} o")
    assert_parity(fs.cpu().numpy(), r["final"], x.dtype, f"{what} final")
    if x.ckpt_interval and r["ckpt"].size:
        assert_parity(ck.cpu().numpy(), r["ckpt"], x.dtype, f"{what} checkpoints")


EDGE = [0, 1, 63, 64, 65, 100, 100, 127, 128, 129]


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_positions_varlen(Dk, Dv, dtype):
    lengths = [200, 0, 64, 1, 129, 70]
    x = make_prefill(lengths, 2, Dk, Dv, dtype, 51, init_state=True)
    positions = [EDGE + [200], [0], [0, 64], [1], [64, 128, 129], [5, 70]]
    check(x, positions, "edges")


def test_positions_with_interval_checkpoints():
    x = make_prefill([300, 190, 64], 2, 128, 128, "bf16", 52, init_state=True, ckpt_interval=64)
    check(x, [[63, 64, 128, 200, 256, 300], [], [64]], "with checkpoints")


def test_positions_with_front_end():
    x = make_prefill([250, 90], 3, 128, 128, "bf16", 53, init_state=True, raw=True)
    check(x, [[10, 64, 130, 250], [89, 90]], "front-end", front=fe.FRONT_ALL)


@pytest.mark.parametrize("Dk,Dv,seqs,H", [(128, 128, 2, 32), (64, 128, 2, 32)])
def test_positions_five_wave_scan(Dk, Dv, seqs, H):
    """Pair counts for which the five-wave scan is chosen (as in the prefill tests)."""
    x = make_prefill([300] * seqs, H, Dk, Dv, "bf16", 54, init_state=True)
    check(x, [[17, 128, 300]] + [[] for _ in range(seqs - 1)], "five-wave")


def test_positions_many_pairs_four_wave_scan():
    """Thousands of (sequence, head) pairs select the 64-column four-wave scan."""
    lengths = [100 + (7 * i) % 97 for i in range(600)]
    x = make_prefill(lengths, 4, 128, 128, "bf16", 55, init_state=True)
    positions = [[] for _ in lengths]
    for s in (0, 17, 311, 599):
        positions[s] = [1, lengths[s] // 2, lengths[s]]
    check(x, positions, "four-wave")


def test_positions_out_of_range_are_clamped():
    x = make_prefill([130, 40], 2, 64, 64, "f32", 56, init_state=True)
    o, fs, ck, ps = gpu_at(x, [[-5, 500], [41]])
    ref = oracle_states(x, [[0, 130], [40]])
    assert_parity(ps.cpu().numpy(), ref, "f32", "clamped positions")


def test_split_phases_match_single_call_bitwise():
    import torch
    x = make_prefill([300, 90], 2, 128, 128, "bf16", 57, init_state=True, raw=True)
    pos = [[10, 128, 299], [90]]
    o1, f1, _, p1 = gpu_at(x, pos, front=fe.FRONT_ALL)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    o2, f2, p2 = torch.empty_like(o1), torch.empty_like(f1), torch.empty_like(p1)
    gpu_at(x, pos, front=fe.FRONT_ALL, phases=1, workspace=ws, o=o2, final_state=f2,
           pos_states=p2)
    gpu_at(x, pos, front=fe.FRONT_ALL, phases=2, workspace=ws, o=o2, final_state=f2,
           pos_states=p2)
    assert torch.equal(o1, o2) and torch.equal(f1, f2) and torch.equal(p1, p2)


def test_headline_shape_positions_sampled():
    """T = 8192, H = 32, D = 128 bf16 (the benchmark's launch configuration) with
    prompt-boundary-like positions; 6 (head, 16-column block) units compared."""
    x = make_prefill([8192], 32, 128, 128, "bf16", 1001, init_state=True)
    positions = [[1000, 4096, 8191]]
    o, fs, ck, ps = gpu_at(x, positions)
    rng = np.random.default_rng(58)
    units = np.array([(0, h, cb) for h, cb in zip(rng.choice(32, 6), rng.choice(8, 6))])
    ref = oracle_states(x, positions, units=units)
    ps = ps.cpu().numpy()
    for _, h, cb in units:
        cols = slice(16 * cb, 16 * cb + 16)
        assert_parity(ps[:, h, :, cols], ref[:, h, :, cols], "bf16", f"head {h} cols {cb}")


def _sampled(x, positions, units, what):
    o, fs, ck, ps = gpu_at(x, positions)
    ref = oracle_states(x, positions, units=units)
    ps = ps.cpu().numpy()
    for _, h, cb in units:
        cols = slice(16 * cb, 16 * cb + 16)
        assert_parity(ps[:, h, :, cols], ref[:, h, :, cols], "bf16", f"{what} head {h} cols {cb}")
    return o, fs, ck


def test_long_context_positions_with_checkpoints_sampled():
    """T = 147,456 with checkpoints every 32,768 tokens (stops merged with the
    checkpoint segments), positions inside and on chunk boundaries."""
    x = make_workload(2)
    units = np.array([(0, 3, 1), (0, 30, 6)])
    _, _, ck = _sampled(x, [[5000, 32768, 70001, 147455]], units, "long context")
    # the checkpoints of the same call
    r = recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, ckpt_interval=x.ckpt_interval,
                           units=units)
    ck = ck.cpu().numpy()
    for _, h, cb in units:
        cols = slice(16 * cb, 16 * cb + 16)
        assert_parity(ck[:, h, :, cols], r["ckpt"][:, h, :, cols], "bf16", f"checkpoints head {h}")


def test_varlen_workload_positions_sampled():
    """64 packed sequences (the 64-column four-wave scan at this size), one
    position in every eighth sequence."""
    x = make_workload(3)
    positions = [[] for _ in range(x.num_seqs)]
    for s in range(0, x.num_seqs, 8):
        positions[s] = [x.lengths[s] // 3]
    units_by_seq = [(s, 5, 2) for s in range(0, x.num_seqs, 8)]
    o, fs, ck, ps = gpu_at(x, positions)
    ps = ps.cpu().numpy()
    for j, (s, h, cb) in enumerate(units_by_seq):
        one = PrefillInputs(x.dtype, x.H, x.Dk, x.Dv, [x.lengths[s]],
                            x.q[x.cu_seqlens[s]:x.cu_seqlens[s + 1]],
                            x.k[x.cu_seqlens[s]:x.cu_seqlens[s + 1]],
                            x.v[x.cu_seqlens[s]:x.cu_seqlens[s + 1]],
                            x.g[x.cu_seqlens[s]:x.cu_seqlens[s + 1]],
                            x.beta[x.cu_seqlens[s]:x.cu_seqlens[s + 1]],
                            x.initial_state[s:s + 1])
        ref = oracle_states(one, [positions[s]], units=np.array([(0, h, cb)]))
        cols = slice(16 * cb, 16 * cb + 16)
        assert_parity(ps[j, h, :, cols], ref[0, h, :, cols], "bf16", f"varlen seq {s}")
