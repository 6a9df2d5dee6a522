#!/usr/bin/env python3
"""Benchmark of the MI355X KDA core (one GPU).

One step = one chunked prefill (prepare + scan) of the 8192-token workload
(B=1, H=32, D_k=D_v=128, bf16 q/k/v, fp32 g/beta/state, random fp32 initial
state), inputs resident in HBM. The same run also times the batched decode
workload (B=512, H=32, D=128, 64 consecutive in-place steps over the 1 GiB
fp32 state) and the fp64 CPU oracle on a bounded sample of the prefill.

Prints ONE JSON line. Per-kernel durations come from HIP events recorded on
the stream the kernels run on (torch's current stream, which the binding
passes to the library)."""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PREFILL_WORKLOAD = 1
DECODE_WORKLOAD = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")


# Sources of the kernels whose counters profiles/ holds (K1, the scans, decode).
MEASURED_SOURCES = ("kda_internal.h", "kda_prefill.hip", "kda_decode.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_05_amd", "csrc")
    for f in MEASURED_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    or None when absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("fetch_bytes", 0) + k.get("write_bytes", 0)


def measured_mfma(kernel: str):
    """Matrix-core utilisation of a kernel from rocprofv3 counters
    (profiles/mfma.json): busy cycles over active cycles x SIMDs, and the MFMA
    FLOPs the counters saw per launch; None when absent or taken on different
    kernel sources."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("kernels", {}).get(kernel)


def dev(arr):
    import numpy as np
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def bench_prefill(steps, warmup):
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import _binding as B
    from linear_attention_05_amd import accounting as acc
    from synth import make_workload

    x = make_workload(PREFILL_WORKLOAD)
    N, H, D = x.total_tokens, x.H, x.Dk
    q, k, v, g, beta, s0 = (dev(a) for a in (x.q, x.k, x.v, x.g, x.beta, x.initial_state))
    o = torch.empty(N, H, D, device="cuda")
    fs = torch.empty(1, H, D, D, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_size(N, 1, H, D, D), dtype=torch.uint8, device="cuda")

    def phase(p):
        K.kda_prefill_chunked(q, k, v, g, beta, initial_state=s0, final_state=fs, o=o,
                              workspace=ws, phases=p)

    both = B.PHASE_PREPARE | B.PHASE_SCAN
    for _ in range(warmup):
        phase(both)
    # Timed steps: one whole library call per step (prep, K1 and K2 back to
    # back on the stream), events only around the region.
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for i in range(steps):
        phase(both)
    r1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = r0.elapsed_time(r1) / steps
    # Per-kernel durations: the same steps issued as two calls with an event
    # between the phases (the event adds a small gap, so these are timed in a
    # loop of their own, not in the headline steps).
    for _ in range(warmup):
        phase(B.PHASE_PREPARE)
        phase(B.PHASE_SCAN)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        phase(B.PHASE_PREPARE)
        ev[i][1].record()
        phase(B.PHASE_SCAN)
        ev[i][2].record()
    torch.cuda.synchronize()
    k1_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    k2_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    n_chunks = (N + 63) // 64
    flops = N * H * acc.prefill_flops_per_token_head(D, D)
    return dict(
        wall_ms=max(wall / steps * 1e3, event_ms), event_ms=event_ms, k1_ms=k1_ms,
        k2_ms=k2_ms, n_tok=N, H=H, D=D, flops=flops,
        compulsory_bytes=acc.prefill_compulsory_bytes(N, H, D, D, 2, 1, 1),
        k1_bytes=acc.k1_bytes(N, H, D, 2, 2, n_chunks),
        k2_bytes=acc.k2_bytes(N, H, D, D, 2, 2, n_chunks, 1, 1),
        inputs=x)


def bench_decode(steps, warmup):
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import accounting as acc
    from synth import WORKLOADS, decode_state, decode_step_inputs, workload_seed
    from concurrent.futures import ThreadPoolExecutor

    w = WORKLOADS[DECODE_WORKLOAD]
    Bsz, H, D = w["B"], w["H"], w["D"]
    seed = workload_seed(DECODE_WORKLOAD)
    state = dev(decode_state(Bsz, H, D, D, seed))
    with ThreadPoolExecutor(8) as ex:
        host = list(ex.map(lambda t: decode_step_inputs(Bsz, H, D, D, w["dtype"], seed, t),
                           range(steps)))
    inp = [tuple(dev(a) for a in (s.q, s.k, s.v, s.g, s.beta)) for s in host]
    o = torch.empty(Bsz, H, D, device="cuda")
    for i in range(warmup):
        K.kda_decode_step(*inp[i % steps], state, o)
    # wall clock of back-to-back steps (no events between them) ...
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        K.kda_decode_step(*inp[i], state, o)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # ... and each step's kernel alone, between events
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        K.kda_decode_step(*inp[i], state, o)
        ev[i][1].record()
    torch.cuda.synchronize()
    per = [e[0].elapsed_time(e[1]) for e in ev]
    kern_ms = float(np.median(per))
    byts = Bsz * H * acc.decode_bytes_per_head_token(D, D, 2)
    return dict(wall_ms=wall / steps * 1e3, kernel_ms=kern_ms, mean_ms=float(np.mean(per)),
                bytes=byts, flops=Bsz * H * acc.decode_flops_per_head_token(D, D))


def bench_strong_decay(counts=(0, 8, 128), steps=20, warmup=50):
    """The headline prefill with n channels per head (the same for every
    head) decaying by -U(0.6, 2) nats per token and the rest by the workload
    recipe: diagonal 16-token blocks then take the vector-unit form (up to 16
    such channels) or the four-level products (more)."""
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from synth import make_workload

    x = make_workload(PREFILL_WORKLOAD)
    N, H, D = x.total_tokens, x.H, x.Dk
    q, k, v, beta, s0 = (dev(a) for a in (x.q, x.k, x.v, x.beta, x.initial_state))
    o = torch.empty(N, H, D, device="cuda")
    fs = torch.empty(1, H, D, D, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_size(N, 1, H, D, D), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(77)
    rows = []
    for n in counts:
        g = x.g.copy()
        ch = rng.choice(D, size=n, replace=False)
        g[:, :, ch] = -rng.uniform(0.6, 2.0, size=(N, H, n)).astype(np.float32)
        gd = dev(np.ascontiguousarray(g))

        def call():
            K.kda_prefill_chunked(q, k, v, gd, beta, initial_state=s0, final_state=fs, o=o,
                                  workspace=ws)

        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        rows.append({"fast_channels_per_head": n, "ms": round(ms, 4),
                     "mtok_s": round(N / (ms * 1e-3) / 1e6, 3)})
    return {"workload": f"prefill B=1 T={N} H={H} D={D} bf16, n channels per head with "
                        "g = -U(0.6, 2) per token", "runs": rows}


def bench_decode_small(batches=(1, 8, 32), steps=32, replays=20):
    """Decode steps for small batches (H = 32, D = 128, bf16), launched from a
    captured graph of `steps` steps so that the host's per-call cost (about
    15 us from Python) does not hide the kernels: us per step over `replays`
    replays, each step on the state the previous one left."""
    import torch
    import linear_attention_05_amd as K
    from synth import decode_state, decode_step_inputs

    H, D = 32, 128
    rows = []
    for Bsz in batches:
        state = dev(decode_state(Bsz, H, D, D, 71))
        s = decode_step_inputs(Bsz, H, D, D, "bf16", 71, 0)
        inp = tuple(dev(a) for a in (s.q, s.k, s.v, s.g, s.beta))
        o = torch.empty(Bsz, H, D, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up off the default stream, as capture wants
            for _ in range(3):
                K.kda_decode_step(*inp, state, o)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                K.kda_decode_step(*inp, state, o)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (replays * steps)
        rows.append({"B": Bsz, "us_per_step": round(us, 2),
                     "state_gbps": round(Bsz * H * D * D * 8 / (us * 1e3), 1)})
    return {"workload": "KDA decode H=32 D=128 bf16, steps launched from a captured graph",
            "batches": rows}


def cpu_baseline(x, target_s=10.0):
    """fp64 oracle (all value columns of a growing set of heads, all tokens),
    timed until about target_s seconds of CPU work; reports the median
    per-head time scaled to the whole workload."""
    import numpy as np
    from oracle import recurrence

    cores = recurrence.num_threads(0)

    def run(heads):
        units = np.array([(0, h, cb) for h in heads for cb in range(x.Dv // 16)], np.int32)
        t = time.perf_counter()
        recurrence.prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state,
                           units=units, col_block=16)
        return time.perf_counter() - t

    t1 = run([0])
    n = int(max(1, min(x.H, round(target_s / max(t1, 1e-3)))))
    per_head, spent, reps = [], 0.0, 0
    while spent < target_s and reps < 100:
        tn = run(list(range(n)))
        per_head.append(tn / n)
        spent += tn
        reps += 1
    full = float(np.median(per_head)) * x.H
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    # the recurrence's own work: 7 Dk Dv FLOPs per token-head (decay, retrieval,
    # write, readout)
    gflops = x.total_tokens * x.H * 7 * x.Dk * x.Dv / full / 1e9
    return dict(value=x.total_tokens / full / 1e6, unit="Mtok/s", cores=cores, kind="oracle",
                sample=f"all {x.total_tokens} tokens x {n} of {x.H} heads x all {x.Dv} value "
                       f"columns, fp64 token recurrence, repeated {reps}x ({spent:.1f} s); "
                       f"median scaled to {x.H} heads",
                seconds=spent, gflops=round(gflops, 2), cpu_model=cpu_model)


def bench_few_heads(H=4, T=65536, D=128, reps=5):
    """One sequence with few heads (a head-sharded layer's per-GPU share): the
    chunk-parallel scan (one call) against the plain scan (prepare and scan as
    two calls on the same inputs), medians over reps, inputs resident."""
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import _binding as B
    from linear_attention_05_amd import accounting as acc
    from synth import make_prefill

    x = make_prefill([T], H, D, D, "bf16", 4242, init_state=True)
    args = [dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    s0 = dev(x.initial_state)
    o = torch.empty(T, H, D, device="cuda")
    fs = torch.empty(1, H, D, D, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_size(T, 1, H, D, D), dtype=torch.uint8, device="cuda")

    def split():
        K.kda_prefill_chunked(*args, initial_state=s0, final_state=fs, o=o, workspace=ws)

    def plain():
        for p in (B.PHASE_PREPARE, B.PHASE_SCAN):
            K.kda_prefill_chunked(*args, initial_state=s0, final_state=fs, o=o, workspace=ws,
                                  phases=p)

    def timed(fn):
        fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    ms_split, ms_plain = timed(split), timed(plain)
    byts = acc.prefill_compulsory_bytes(T, H, D, D, 2, 1, 1)
    return dict(workload=f"prefill B=1 H={H} T={T} D={D} bf16, S0 and final state",
                segments=K.kda_prefill_scan_segments(T, 1, H, D, D),
                split_ms=round(ms_split, 4), plain_ms=round(ms_plain, 4),
                split_mtok_s=round(T / (ms_split * 1e-3) / 1e6, 3),
                plain_mtok_s=round(T / (ms_plain * 1e-3) / 1e6, 3),
                speedup=round(ms_plain / ms_split, 3),
                split_path_roofline_frac=round(byts / (ms_split * 1e-3) / 8e12, 4))


def bench_prefill_workload(idx, reps=3):
    """Time one whole prefill call of another workload (long-context with
    checkpoints, or packed varlen): median over reps, inputs resident."""
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import accounting as acc
    from synth import make_workload

    x = make_workload(idx)
    N, H, D = x.total_tokens, x.H, x.Dk
    args = [dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    cu = dev(x.cu_seqlens)
    s0 = dev(x.initial_state) if x.initial_state is not None else None
    o = torch.empty(N, H, D, device="cuda")
    fs = torch.empty(x.num_seqs, H, D, D, device="cuda")
    nck = x.num_checkpoints()
    ck = torch.empty(max(nck, 0), H, D, D, device="cuda") if x.ckpt_interval else None
    ws = torch.empty(K.kda_prefill_workspace_size(N, x.num_seqs, H, D, D), dtype=torch.uint8,
                     device="cuda")

    def run():
        K.kda_prefill_chunked(*args, cu_seqlens=cu, initial_state=s0, final_state=fs,
                              ckpt_interval=x.ckpt_interval, ckpt_states=ck, o=o, workspace=ws)

    run()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    n_state = (x.num_seqs if x.initial_state is not None else 0) + x.num_seqs + nck
    byts = acc.prefill_compulsory_bytes(N, H, D, D, 2, 0, 0) + n_state * H * D * D * 4
    return dict(workload=x.name, tokens=N, seqs=x.num_seqs, ms=round(ms, 4),
                mtok_s=round(N / (ms * 1e-3) / 1e6, 3),
                tflops_algorithmic=round(N * H * acc.prefill_flops_per_token_head(D, D) / (ms * 1e-3) / 1e12, 2),
                path_roofline_frac=round(byts / (ms * 1e-3) / 8e12, 4))


def bench_frontend(steps=10, warmup=50, decode_steps=32):
    """The in-kernel parameter-free front-end (KDA_FRONT_*: q/k L2 normalisation,
    g = -exp(u), sigmoid write strength) on raw inputs of the headline prefill
    and decode shapes, beside what the same transforms cost as separate torch
    passes before the plain path."""
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from linear_attention_05_amd import _binding as B
    from synth import (WORKLOADS, decode_state, decode_step_inputs, make_prefill,
                       workload_lengths, workload_seed)

    w = WORKLOADS[PREFILL_WORKLOAD]
    x = make_prefill(workload_lengths(PREFILL_WORKLOAD), w["H"], w["D"], w["D"], w["dtype"],
                     workload_seed(PREFILL_WORKLOAD), raw=True)
    N, H, D = x.total_tokens, x.H, x.Dk
    q, k, v, u, b, s0 = (dev(a) for a in (x.q, x.k, x.v, x.g, x.beta, x.initial_state))
    o = torch.empty(N, H, D, device="cuda")
    fs = torch.empty(1, H, D, D, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_size(N, 1, H, D, D), dtype=torch.uint8, device="cuda")

    def phase(p):
        K.kda_prefill_chunked(q, k, v, u, b, initial_state=s0, final_state=fs, o=o,
                              workspace=ws, phases=p, frontend=B.FRONT_ALL)

    def prepass():  # the same transforms as separate passes (bf16 q/k written back)
        qn = (q.float() * torch.rsqrt(q.float().square().sum(-1, keepdim=True) + 1e-6)).bfloat16()
        kn = (k.float() * torch.rsqrt(k.float().square().sum(-1, keepdim=True) + 1e-6)).bfloat16()
        return qn, kn, -torch.exp(u), torch.sigmoid(b)

    for _ in range(warmup):
        phase(B.PHASE_PREPARE)
        phase(B.PHASE_SCAN)
        prepass()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        phase(B.PHASE_PREPARE)
        ev[i][1].record()
        phase(B.PHASE_SCAN)
        ev[i][2].record()
        prepass()
        ev[i][3].record()
    torch.cuda.synchronize()
    k1 = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    k2 = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    pre = float(np.median([e[2].elapsed_time(e[3]) for e in ev]))
    del q, k, v, u, b, o, ws

    # decode: plain and front-end steps interleaved on one state, so both see
    # the same memory
    wd = WORKLOADS[DECODE_WORKLOAD]
    Bsz, Hd, Dd = wd["B"], wd["H"], wd["D"]
    seed = workload_seed(DECODE_WORKLOAD)
    state = dev(decode_state(Bsz, Hd, Dd, Dd, seed))
    raw = [tuple(dev(a) for a in (s.q, s.k, s.v, s.g, s.beta))
           for s in (decode_step_inputs(Bsz, Hd, Dd, Dd, wd["dtype"], seed, t, raw=True)
                     for t in range(decode_steps))]
    plain = [tuple(dev(a) for a in (s.q, s.k, s.v, s.g, s.beta))
             for s in (decode_step_inputs(Bsz, Hd, Dd, Dd, wd["dtype"], seed, t)
                       for t in range(decode_steps))]
    od = torch.empty(Bsz, Hd, Dd, device="cuda")
    for i in range(2 * warmup):
        K.kda_decode_step(*plain[i % decode_steps], state, od)
        K.kda_decode_step(*raw[i % decode_steps], state, od, frontend=B.FRONT_ALL)
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(decode_steps)]
    torch.cuda.synchronize()
    for i in range(decode_steps):
        evd[i][0].record()
        K.kda_decode_step(*plain[i], state, od)
        evd[i][1].record()
        K.kda_decode_step(*raw[i], state, od, frontend=B.FRONT_ALL)
        evd[i][2].record()
    torch.cuda.synchronize()
    dec_plain = float(np.median([e[0].elapsed_time(e[1]) for e in evd]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evd]))
    from linear_attention_05_amd import accounting as acc
    dec_bytes = Bsz * Hd * acc.decode_bytes_per_head_token(Dd, Dd, 2)
    return dict(
        transforms="q/k L2 norm, g=-exp(u), beta=sigmoid(b), inside the kernels (raw inputs)",
        prefill_workload=f"B=1 T={N} H={H} D={D} bf16",
        prefill_k1_ms=round(k1, 4), prefill_k2_ms=round(k2, 4),
        prefill_ms=round(k1 + k2, 4), prefill_mtok_s=round(N / ((k1 + k2) * 1e-3) / 1e6, 3),
        torch_prepass_ms=round(pre, 4),
        decode_workload=f"B={Bsz} H={Hd} D={Dd} bf16, {decode_steps} steps, each beside a "
                        "plain step on the same state",
        decode_us_per_step=round(dec_ms * 1e3, 2),
        decode_gbps=round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
        decode_plain_us_per_step=round(dec_plain * 1e3, 2))


def bench_positions(reps=10, warmup=50):
    """States at arbitrary positions (kda_prefill_chunked_at) on the headline
    prefill: whole calls with four mid-chunk positions, interleaved with plain
    calls on the same inputs."""
    import numpy as np
    import torch
    import linear_attention_05_amd as K
    from synth import make_workload

    x = make_workload(PREFILL_WORKLOAD)
    N, H, D = x.total_tokens, x.H, x.Dk
    args = [dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    s0 = dev(x.initial_state)
    o = torch.empty(N, H, D, device="cuda")
    fs = torch.empty(1, H, D, D, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_size(N, 1, H, D, D), dtype=torch.uint8, device="cuda")
    vals = [1000, 3000, 5000, N - 1]
    offs = torch.tensor([0, len(vals)], dtype=torch.int32, device="cuda")
    pv = torch.tensor(vals, dtype=torch.int32, device="cuda")
    ps = torch.empty(len(vals), H, D, D, device="cuda")

    def plain():
        K.kda_prefill_chunked(*args, initial_state=s0, final_state=fs, o=o, workspace=ws)

    def at():
        K.kda_prefill_chunked_at(*args, offs, pv, pos_states=ps, initial_state=s0,
                                 final_state=fs, o=o, workspace=ws)

    for _ in range(warmup):
        plain()
        at()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        plain()
        e[1].record()
        at()
        e[2].record()
    torch.cuda.synchronize()
    t_plain = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    t_at = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    return dict(workload=f"prefill B=1 T={N} H={H} D={D} bf16, states after {vals} tokens",
                plain_ms=round(t_plain, 4), with_positions_ms=round(t_at, 4),
                overhead_ms=round(t_at - t_plain, 4))


def hbm_ceilings():
    """Practical HBM rates of plain torch kernels on 1 GiB (context for the
    roofline fractions): read-only (sum), write-only (fill), copy (read+write)."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("read_sum", lambda: a.sum(), 1 << 30),
                            ("write_fill", lambda: b.fill_(2.0), 1 << 30),
                            ("copy", lambda: b.copy_(a), 2 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_gbps"] = round(moved / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9, 1)
    del a, b
    return out


def roofline(bytes_, ms, traffic=None):
    gbps = bytes_ / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
            "frac": round(gbps / 8000.0, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clock after about 20 ms of prefill calls (~60
    # calls at the headline shape): the default warm-up covers that
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "few_heads", "long_varlen",
                                       "decode_small", "strong_decay"],
                    default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip timing the long-context and varlen prefill workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a known-size "
                         "reference dispatch for hardware traffic counters)")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="first run one fp16 8192^3 GEMM (a known-FLOP reference dispatch for "
                         "matrix-core counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py: this KDA core build runs on one GPU; --gpus {args.gpus} "
                  f"(WORLD_SIZE={world}) is not supported. Independent (sequence, head) "
                  "pairs would shard across GPUs without communication.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import linear_attention_05_amd as K
    K.load_library()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.mfma_calibration:
        a = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
        b = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mm(a, b)
        torch.cuda.synchronize()
        del a, b

    out = {}
    if args.only == "long_varlen":
        out["prefill_workloads"] = [bench_prefill_workload(2), bench_prefill_workload(3)]
        out["kernel_source_sha"] = kernel_source_sha()
        print(json.dumps(out), flush=True)
        return
    if args.only == "few_heads":
        out["few_heads"] = [bench_few_heads(4), bench_few_heads(1)]
        out["kernel_source_sha"] = kernel_source_sha()
        print(json.dumps(out), flush=True)
        return
    if args.only in ("decode_small", "strong_decay"):
        out["decode_small_batches" if args.only == "decode_small" else args.only] = (
            bench_decode_small() if args.only == "decode_small" else bench_strong_decay())
        out["kernel_source_sha"] = kernel_source_sha()
        print(json.dumps(out), flush=True)
        return
    if args.only in ("all", "prefill"):
        p = bench_prefill(args.steps, args.warmup)
        step_ms = p["wall_ms"]
        mtok = p["n_tok"] / (step_ms * 1e-3) / 1e6
        k1 = roofline(p["k1_bytes"], p["k1_ms"], measured_traffic("k1_prep"))
        k2 = roofline(p["k2_bytes"], p["k2_ms"], measured_traffic("k2_scan"))
        # Headline roofline: the method's algorithmic (compulsory) bytes of one
        # call over the dominant kernel's event-timed duration; beside it the
        # same bytes over the whole call, and the two kernels' counter traffic
        # against those bytes (above 1: the K1 -> K2 handoff's round trip).
        dom_name, dom_ms = ("k2_scan", p["k2_ms"]) if p["k2_ms"] >= p["k1_ms"] else ("k1_prep", p["k1_ms"])
        comp = p["compulsory_bytes"]
        t1, t2 = measured_traffic("k1_prep"), measured_traffic("k2_scan")
        path_traffic = t1 + t2 if (t1 is not None and t2 is not None) else None
        dominant = dict(roofline(comp, dom_ms, measured_traffic(dom_name)), kernel=dom_name,
                        algorithmic_bytes=comp, kernel_ms=round(dom_ms, 4),
                        whole_call_frac=round(comp / (step_ms * 1e-3) / 8e12, 4),
                        path_traffic=path_traffic,
                        traffic_over_algorithmic=(round(path_traffic / comp, 3)
                                                  if path_traffic is not None else None))
        out.update({
            "metric": "KDA prefill Mtok/s & TFLOP/s (H=32,D=128); decode state HBM GB/s vs peak",
            "value": round(mtok, 3), "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in; f16 MFMA, f32 accum/state",
            "data": "synthetic (seeded; q,k L2-normalised N(0,1); v N(0,1); g=-exp(N(-4,0.5)); "
                    "beta=sigmoid(N(0,1)); S0 N(0,0.02))",
            "config": {"workload": "KDA prefill B=1 T=8192 H=32 Dk=Dv=128 C=64 bf16, "
                                   "fp32 initial+final state", "seq_len": p["n_tok"],
                       "heads": p["H"], "head_dim": p["D"], "chunk": 64},
            "roofline": dominant,
            "prefill": {
                "event_ms_per_step": round(p["event_ms"], 4),
                "tflops_algorithmic": round(p["flops"] / (step_ms * 1e-3) / 1e12, 2),
                "tflops_frac_of_bf16_mfma_peak": round(p["flops"] / (step_ms * 1e-3) / 2.5e15, 4),
                "flops_per_step": p["flops"],
                "path_compulsory_bytes": p["compulsory_bytes"],
                "path_roofline_frac": round(p["compulsory_bytes"] / (step_ms * 1e-3) / 8e12, 4),
                "k1_prep": dict(k1, ms=round(p["k1_ms"], 4), bytes=p["k1_bytes"],
                                mfma=measured_mfma("k1_prep")),
                "k2_scan": dict(k2, ms=round(p["k2_ms"], 4), bytes=p["k2_bytes"],
                                mfma=measured_mfma("k2_scan")),
            },
        })
    if args.only in ("all", "decode"):
        d = bench_decode(args.decode_steps, min(args.warmup, args.decode_steps))
        rd = roofline(d["bytes"], d["kernel_ms"], measured_traffic("decode"))
        out["decode"] = dict(
            workload="KDA decode B=512 H=32 D=128 bf16, fp32 state [512,32,128,128] in place",
            steps=args.decode_steps, us_per_step=round(d["kernel_ms"] * 1e3, 2),
            wall_us_per_step=round(d["wall_ms"] * 1e3, 2), state_bytes_per_step=d["bytes"],
            gbps=rd["achieved"], frac_of_peak=rd["frac"], roofline=dict(rd, kernel="decode"))
        if "metric" not in out:
            out.update({"metric": "KDA decode state HBM GB/s", "value": rd["achieved"],
                        "unit": "GB/s", "n_gpus": 1, "steps": args.decode_steps,
                        "warmup": args.warmup, "ms_per_step": round(d["wall_ms"], 4),
                        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                        "dtype": "bf16 in; f32 state", "data": "synthetic",
                        "config": {"workload": out["decode"]["workload"]},
                        "roofline": out["decode"]["roofline"]})
    if args.only in ("all", "prefill") and not args.no_extra_workloads:
        out["prefill_workloads"] = [bench_prefill_workload(2), bench_prefill_workload(3)]
        out["few_heads"] = [bench_few_heads(4), bench_few_heads(1)]
    if args.only == "all" and not args.no_extra_workloads:
        out["frontend"] = bench_frontend()
        out["positions"] = bench_positions()
        out["decode_small_batches"] = bench_decode_small()
        out["strong_decay"] = bench_strong_decay()
        out["hbm_ceilings"] = hbm_ceilings()
    if args.only in ("all", "prefill") and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p["inputs"])
        out["cpu_baseline"]["seconds"] = round(out["cpu_baseline"]["seconds"], 2)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 5)
    out["kernel_source_sha"] = kernel_source_sha()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
