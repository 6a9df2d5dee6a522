"""Graph capture. The library enqueues only kernels on the caller's stream (no
allocation, memset or copy), so decode steps and prefill calls can be
captured in a HIP graph and replayed. Each graph is replayed several times,
with eager work of the program and synchronisations between the replays, and
every replay is compared bitwise with the same calls run eagerly."""

import pytest

from helpers import dev_tensor
from synth import decode_state, decode_step_inputs, make_prefill

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capturing stream
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def test_decode_steps_in_a_graph():
    import torch
    import linear_attention_05_amd as K
    B, H, D, steps = 4, 8, 128, 4
    print(f"graph decode B={B} H={H} D={D} steps={steps}", flush=True)
    s0 = dev_tensor(decode_state(B, H, D, D, 81))
    xs = [[dev_tensor(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
          for x in (decode_step_inputs(B, H, D, D, "bf16", 81, t) for t in range(steps))]
    st_e = s0.clone()
    o_e = [K.kda_decode_step(*xs[t], st_e) for t in range(steps)]
    st_g = s0.clone()
    o_g = [torch.empty(B, H, D, device="cuda") for _ in range(steps)]

    def body():
        for t in range(steps):
            K.kda_decode_step(*xs[t], st_g, o_g[t])

    graph = _capture(body)
    scratch = s0.clone()
    for rep in range(3):
        st_g.copy_(s0)
        graph.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(o_g[t], o_e[t]), f"replay {rep}: o of step {t}"
        assert torch.equal(st_g, st_e), f"replay {rep}: state"
        K.kda_decode_step(*xs[rep % steps], scratch)  # eager work between replays
        torch.cuda.synchronize()


PREFILL = {  # lengths, H, Dk, Dv, dtype: plain varlen path, chunk-parallel path, fp32
    "varlen": ([300, 129, 700], 4, 128, 128, "bf16"),
    "split": ([8192], 4, 128, 128, "bf16"),
    "f32": ([500, 64], 2, 64, 64, "f32"),
}


@pytest.mark.parametrize("case", list(PREFILL))
def test_prefill_in_a_graph(case):
    import torch
    import linear_attention_05_amd as K
    lengths, H, Dk, Dv, dtype = PREFILL[case]
    print(f"graph prefill {case}: lengths={lengths} H={H} Dk={Dk} Dv={Dv} {dtype}", flush=True)
    x = make_prefill(lengths, H, Dk, Dv, dtype, 83, init_state=True)
    q, k, v, g, beta = (dev_tensor(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    cu = dev_tensor(x.cu_seqlens)
    s0 = dev_tensor(x.initial_state)
    N, S = x.total_tokens, x.num_seqs
    ws = torch.empty(K.kda_prefill_workspace_size(N, S, H, Dk, Dv, q.dtype), dtype=torch.uint8,
                     device="cuda")

    def call(o, fs):
        K.kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0, final_state=fs,
                              o=o, workspace=ws)

    o_e = torch.empty(N, H, Dv, device="cuda")
    fs_e = torch.empty(S, H, Dk, Dv, device="cuda")
    call(o_e, fs_e)
    o_g = torch.empty_like(o_e)
    fs_g = torch.empty_like(fs_e)
    graph = _capture(lambda: call(o_g, fs_g))
    for rep in range(3):
        o_g.zero_()
        fs_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: o"
        assert torch.equal(fs_g, fs_e), f"replay {rep}: final state"
        call(o_e, fs_e)  # eager work between replays (same results)
        torch.cuda.synchronize()
