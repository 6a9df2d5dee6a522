"""CPU tests of the C ABI: the library loads, exports every symbol include/kda.h
declares, sizes workspaces, and rejects invalid arguments before any HIP call
(fake pointers are safe here because validation fails first)."""

import ctypes
import os
import re

import pytest

from linear_attention_05_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INV, UNS, WS = B.KDA_OK, B.KDA_ERR_INVALID_ARG, B.KDA_ERR_UNSUPPORTED, B.KDA_ERR_WORKSPACE
A = 0x100000  # fake, 256-byte aligned "device" address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert B.version() >= 300  # 0.3.0: kda_prefill_chunked_at
    for s in range(5):
        assert B.status_string(s).startswith("KDA_")
    assert "unknown" in B.status_string(99)


def ws_size(N=8192, S=1, H=32, Dk=128, Dv=128, chunk=64, dt=B.KDA_BF16):
    return B.workspace_size(N, S, H, Dk, Dv, dt, chunk)


def test_workspace_size():
    per_chunk_bf16 = (192 * 128 + 6144) * 2 + 4 * 128
    assert per_chunk_bf16 == 61952
    table = 256 + 64 * 256 * 8 * 4  # sequence tables + store sink
    assert ws_size() == table + 32 * (8192 // 64 + 1) * per_chunk_bf16
    per_chunk_f32 = (192 * 64 + 6144) * 4 + 4 * 64
    assert ws_size(256, 1, 2, 64, 64, 64, B.KDA_F32) == table + 2 * 5 * per_chunk_f32
    assert ws_size(Dk=96) == 0
    assert ws_size(chunk=32) == 0
    assert ws_size(N=-1) == 0
    assert ws_size(S=0) == 0
    assert ws_size(dt=7) == 0
    assert ws_size(N=0, S=3) > 0


def prefill(**kw):
    a = dict(q=A, k=A, v=A, dt=B.KDA_BF16, g=A, beta=A, cu=None, S=1, N=256, H=2, Dk=128,
             Dv=128, chunk=64, s0=None, sf=A, ci=0, ck=None, ckr=0, o=A, ws=A,
             wsb=10 ** 12, stream=None)
    a.update(kw)
    return B.prefill_raw(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["cu"], a["S"],
                         a["N"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["s0"], a["sf"],
                         a["ci"], a["ck"], a["ckr"], a["o"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(g=None), INV),
    (dict(beta=None), INV), (dict(o=None), INV),
    (dict(N=-5), INV), (dict(H=0), INV), (dict(S=0), INV), (dict(dt=3), INV),
    (dict(Dk=96), UNS), (dict(Dv=32), UNS), (dict(chunk=128), UNS), (dict(N=2 ** 31), UNS),
    (dict(H=2 ** 18), UNS),                            # H * D * 64 past 32-bit row offsets
    (dict(S=2), INV),                                  # several sequences need cu_seqlens
    (dict(ci=-64), INV), (dict(ci=96), UNS),           # interval not a multiple of 64
    (dict(ci=128), INV),                               # interval without a buffer
    (dict(ci=128, ck=A, ckr=-1), INV),
    (dict(ck=A), INV), (dict(ckr=3), INV),             # buffer without an interval
    (dict(q=A + 8), INV), (dict(g=A + 4), INV), (dict(o=A + 2), INV), (dict(sf=A + 8), INV),
    (dict(ws=None), WS), (dict(wsb=1000), WS), (dict(ws=A + 16), INV),
])
def test_prefill_validation(kw, status):
    assert prefill(**kw) == status


@pytest.mark.parametrize("phases,status", [(0, INV), (4, INV), (7, INV)])
def test_prefill_phases_validation(phases, status):
    st = B.prefill_phases_raw(A, A, A, B.KDA_BF16, A, A, None, 1, 256, 2, 128, 128, 64, None, A,
                              0, None, 0, A, A, 10 ** 12, phases, None)
    assert st == status


@pytest.mark.parametrize("front,kw,status", [
    (8, {}, INV), (0xFFFFFFFF, {}, INV),               # unknown front-end bits
    (B.FRONT_ALL, dict(q=None), INV), (B.FRONT_ALL, dict(Dk=96), UNS),
    (B.FRONT_ALL, dict(wsb=1000), WS), (B.FRONT_GATE, dict(phases=0), INV),
])
def test_prefill_ex_validation(front, kw, status):
    a = dict(q=A, Dk=128, wsb=10 ** 12, phases=3)
    a.update(kw)
    st = B.prefill_ex_raw(a["q"], A, A, B.KDA_BF16, A, A, None, 1, 256, 2, a["Dk"], 128, 64,
                          None, A, 0, None, 0, A, A, a["wsb"], a["phases"], front, None)
    assert st == status


@pytest.mark.parametrize("front,kw,status", [
    (8, {}, INV), (16, dict(B=0), INV),                # unknown bits, even for a no-op
    (B.FRONT_ALL, dict(B=0), OK), (B.FRONT_L2NORM_QK, dict(Dk=32), UNS),
    (B.FRONT_BETA_SIGMOID, dict(st=None), INV),
])
def test_decode_ex_validation(front, kw, status):
    a = dict(B=4, Dk=128, st=A)
    a.update(kw)
    st = B.decode_ex_raw(A, A, A, B.KDA_BF16, A, A, a["B"], 2, a["Dk"], 128, a["st"], A, front,
                         None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(npos=-1), INV),
    (dict(offs=None), INV), (dict(vals=None), INV), (dict(ps=None), INV),
    (dict(offs=A + 2), INV), (dict(vals=A + 1), INV), (dict(ps=A + 8), INV),
    (dict(front=16), INV), (dict(phases=0), INV), (dict(Dk=96), UNS), (dict(wsb=1000), WS),
    (dict(npos=2 ** 30), UNS),                         # num_pos * H overflows int32
])
def test_prefill_at_validation(kw, status):
    a = dict(npos=3, offs=A, vals=A, ps=A, front=0, phases=3, Dk=128, wsb=10 ** 12)
    a.update(kw)
    st = B.prefill_at_raw(A, A, A, B.KDA_BF16, A, A, None, 1, 256, 2, a["Dk"], 128, 64, None, A,
                          0, None, 0, A, a["offs"], a["vals"], a["npos"], a["ps"], A, a["wsb"],
                          a["phases"], a["front"], None)
    assert st == status


def test_prefill_workspace_exact_boundary():
    need = ws_size(256, 1, 2, 128, 128)
    assert prefill(wsb=need - 1) == WS


def decode(**kw):
    a = dict(q=A, k=A, v=A, dt=B.KDA_BF16, g=A, beta=A, B=4, H=2, Dk=128, Dv=128, st=A, o=A,
             stream=None)
    a.update(kw)
    return B.decode_raw(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["B"], a["H"],
                        a["Dk"], a["Dv"], a["st"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), OK),                                   # no-op, nothing launched
    (dict(B=-1), INV), (dict(H=0), INV), (dict(dt=2), INV),
    (dict(Dk=32), UNS), (dict(Dv=256), UNS),
    (dict(q=None), INV), (dict(st=None), INV), (dict(o=None), INV), (dict(beta=None), INV),
    (dict(st=A + 4), INV), (dict(v=A + 2), INV),
])
def test_decode_validation(kw, status):
    assert decode(**kw) == status


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import linear_attention_05_amd as K
    x = torch.zeros(1, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K.kda_decode_step(x, x, x, torch.zeros(1, 1, 64), torch.zeros(1, 1),
                          torch.zeros(1, 1, 64, 64))


def test_binding_rejects_wrong_checkpoint_and_position_shapes():
    """The library writes checkpoint rows [0, rows) of a [rows, H, Dk, Dv]
    buffer and reads one position per element of pos_values: a tensor of any
    other shape is refused before any pointer reaches it (checked before the
    device, so plain CPU tensors show it)."""
    torch = pytest.importorskip("torch")
    import linear_attention_05_amd as K
    N, H, D = 128, 2, 64
    q, k, v, g = (torch.zeros(N, H, D) for _ in range(4))
    beta = torch.zeros(N, H)
    for bad in (torch.zeros(2, H, D), torch.zeros(2, H + 1, D, D), torch.zeros(2 * H * D * D),
                torch.zeros(2, H, D, D + 1), torch.zeros(2, H, D // 2, D)):
        with pytest.raises(ValueError, match="ckpt_states"):
            K.kda_prefill_chunked(q, k, v, g, beta, ckpt_interval=64, ckpt_states=bad)
    offs = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="pos_values"):
        K.kda_prefill_chunked_at(q, k, v, g, beta, offs, torch.zeros(2, 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="pos_states"):
        K.kda_prefill_chunked_at(q, k, v, g, beta, offs, torch.zeros(3, dtype=torch.int32),
                                 pos_states=torch.zeros(2, H, D, D))
    # shapes right, tensors on the CPU: refused for where they live
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_prefill_chunked(q, k, v, g, beta, ckpt_interval=64,
                              ckpt_states=torch.zeros(2, H, D, D))


def prefill_noalloc(**kw):
    a = dict(q=A, k=A, v=A, dt=B.KDA_BF16, g=A, beta=A, cu=None, S=1, N=256, H=2, Dk=128,
             Dv=128, chunk=64, s0=None, sf=A, ci=0, ck=None, ckr=0, o=A, stream=None)
    a.update(kw)
    return B.prefill_noalloc_raw(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["cu"],
                                 a["S"], a["N"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["s0"],
                                 a["sf"], a["ci"], a["ck"], a["ckr"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(o=None), INV), (dict(N=-1), INV), (dict(Dk=96), UNS),
    (dict(S=2), INV), (dict(ci=96), UNS), (dict(v=A + 2), INV),
    # more scratch than the library's fixed 128 MiB: refused, nothing launched
    (dict(N=4288, H=32), WS), (dict(N=1 << 20, H=32), WS),
])
def test_prefill_noalloc_validation(kw, status):
    """Every refusal happens before any HIP call (these run without a GPU)."""
    assert prefill_noalloc(**kw) == status


def test_noalloc_limit_is_the_stated_one():
    """The stated limit: one sequence of 4,224 tokens fits at H = 32, D = 128,
    bf16 (its workspace need is at most 128 MiB); 4,288 does not."""
    assert ws_size(N=4224) <= 128 << 20 < ws_size(N=4288)
