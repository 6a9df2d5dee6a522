"""Algorithmic work and traffic of the KDA core (what the method itself must
compute or move), used for roofline reporting.

Pages' figures (Kimi K3 report, "Key data"): a decode step costs about 7*D^2
FLOPs and about 8*D^2 bytes of fp32 recurrent-state traffic per head and
token, and the prefill costs O(T*D^2) FLOPs and O(T*C + T*D + D^2) memory.
The constants for the prefill below are this library's own convention."""

from __future__ import annotations

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 / fp16 MFMA
FP32_PEAK_TFLOPS = 157.3


def decode_flops_per_head_token(Dk: int, Dv: int) -> int:
    """Decay D_k*D_v, S'^T k and S'^T q 2*D_k*D_v each, rank-1 write 2*D_k*D_v:
    7*D^2 for D_k = D_v = D, the pages' count."""
    return 7 * Dk * Dv


def decode_state_bytes_per_head_token(Dk: int, Dv: int) -> int:
    """One fp32 read and one fp32 write of the state: 8*D^2 for D_k = D_v = D."""
    return 8 * Dk * Dv


def io_bytes_per_token_head(Dk: int, Dv: int, in_bytes: int) -> int:
    """Compulsory token traffic: q, k, v in the input dtype, g fp32, beta fp32, o fp32."""
    return (2 * Dk + Dv) * in_bytes + 4 * Dk + 4 + 4 * Dv


def decode_bytes_per_head_token(Dk: int, Dv: int, in_bytes: int) -> int:
    return decode_state_bytes_per_head_token(Dk, Dv) + io_bytes_per_token_head(Dk, Dv, in_bytes)


def prefill_flops_per_token_head(Dk: int, Dv: int, C: int = 64) -> int:
    """The eight chunk products of the chunked form at full C-tiles:
    A, P (C*C*Dk each), W (C*C*Dk), U0 (C*C*Dv), W S, Qd S, Kc^T U (Dk*Dv*C
    each, per C tokens) and P U (C*C*Dv): 6*Dk*Dv + 2*C*(3*Dk + 2*Dv)."""
    return 6 * Dk * Dv + 2 * C * (3 * Dk + 2 * Dv)


def prefill_compulsory_bytes(n_tok: int, H: int, Dk: int, Dv: int, in_bytes: int,
                             n_state_reads: int, n_state_writes: int) -> int:
    return (n_tok * H * io_bytes_per_token_head(Dk, Dv, in_bytes)
            + (n_state_reads + n_state_writes) * H * Dk * Dv * 4)


def handoff_bytes_per_chunk_head(Dk: int, op_bytes: int) -> int:
    """K1 -> K2 handoff block: -W, Qd, Kc^T (64*Dk each), the lower-triangular
    P and Ainv*diag(beta) (the six of eight 16x32 frags of each 64x64 matrix
    that hold entries) in the MFMA operand type, plus Gamma_last (Dk fp32)."""
    return (192 * Dk + 6144) * op_bytes + 4 * Dk


def k1_bytes(n_tok: int, H: int, Dk: int, in_bytes: int, op_bytes: int, n_chunks: int) -> int:
    """K1 reads q, k, g, beta and writes one handoff block per chunk and head."""
    return (n_tok * H * (2 * Dk * in_bytes + 4 * Dk + 4)
            + n_chunks * H * handoff_bytes_per_chunk_head(Dk, op_bytes))


def k2_bytes(n_tok: int, H: int, Dk: int, Dv: int, in_bytes: int, op_bytes: int,
             n_chunks: int, n_state_reads: int, n_state_writes: int) -> int:
    """K2 reads the handoff once and v, writes o, and reads/writes states."""
    return (n_chunks * H * handoff_bytes_per_chunk_head(Dk, op_bytes)
            + n_tok * H * (Dv * in_bytes + 4 * Dv)
            + (n_state_reads + n_state_writes) * H * Dk * Dv * 4)
