"""Torch-tensor front end of the KDA core library (same names as the C ABI).

PyTorch supplies device memory and the stream; this module only checks
tensor properties, allocates outputs the caller did not pass, and forwards raw
pointers to libkda.so. All arithmetic happens in the library's HIP kernels."""

from __future__ import annotations

import torch

from . import _binding as B

CHUNK = 64


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return B.KDA_BF16
    if t.dtype == torch.float32:
        return B.KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_props(t, name, dtype=None, shape=None):
    """dtype, shape (None entries match any size) and contiguity."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(w is None or int(n) == int(w)
                                            for n, w in zip(t.shape, shape))
        if not ok:
            want = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_place(t, name, device):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check(t, name, dtype=None, shape=None, device=None):
    _check_props(t, name, dtype, shape)
    _check_place(t, name, device)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def kda_prefill_workspace_size(total_tokens, num_seqs, H, Dk, Dv, dtype=torch.bfloat16,
                               chunk_size=CHUNK) -> int:
    code = B.KDA_BF16 if dtype == torch.bfloat16 else B.KDA_F32
    return B.workspace_size(total_tokens, num_seqs, H, Dk, Dv, code, chunk_size)


def kda_prefill_scan_segments(total_tokens, num_seqs, H, Dk, Dv, dtype=torch.bfloat16,
                              chunk_size=CHUNK) -> int:
    """Segments of the chunk-parallel scan kda_prefill_chunked uses for these
    sizes on the current device with a workspace of kda_prefill_workspace_size
    bytes (1 = plain scan; include/kda.h, kda_prefill_scan_segments)."""
    code = B.KDA_BF16 if dtype == torch.bfloat16 else B.KDA_F32
    return B.scan_segments(total_tokens, num_seqs, H, Dk, Dv, code, chunk_size)


def kda_prefill_chunked(q, k, v, g, beta, *, cu_seqlens=None, num_seqs=None,
                        initial_state=None, output_final_state=True, final_state=None,
                        ckpt_interval=0, num_checkpoints=None, ckpt_states=None, o=None,
                        workspace=None, phases=B.PHASE_PREPARE | B.PHASE_SCAN, frontend=0):
    """Chunked KDA prefill (see include/kda.h, kda_prefill_chunked).

    q, k [N, H, Dk], v [N, H, Dv] (bf16 or fp32, one dtype); g [N, H, Dk] fp32;
    beta [N, H] fp32; cu_seqlens int32 [S+1] on the GPU or None (one sequence).
    With ckpt_interval > 0 the caller gives num_checkpoints (= sum_s
    floor(L_s / ckpt_interval)) or a preallocated ckpt_states.
    phases selects prepare (K1), scan (K2) or both (kda_prefill_chunked_phases);
    a scan-only call must reuse the workspace of a preceding prepare.
    frontend: KDA_FRONT_* bits (FRONT_L2NORM_QK, FRONT_GATE, FRONT_BETA_SIGMOID)
    applied inside the kernels to raw q/k, g (= u) and beta (= logits)
    (kda_prefill_chunked_ex); 0 uses the inputs as given.
    Returns (o, final_state or None, ckpt_states or None)."""
    o, fs, ck, _ = _prefill(q, k, v, g, beta, cu_seqlens, num_seqs, initial_state,
                            output_final_state, final_state, ckpt_interval, num_checkpoints,
                            ckpt_states, o, workspace, phases, frontend, None, None, None)
    return o, fs, ck


def kda_prefill_chunked_at(q, k, v, g, beta, pos_offsets, pos_values, *, pos_states=None,
                           cu_seqlens=None, num_seqs=None, initial_state=None,
                           output_final_state=True, final_state=None, ckpt_interval=0,
                           num_checkpoints=None, ckpt_states=None, o=None, workspace=None,
                           phases=B.PHASE_PREPARE | B.PHASE_SCAN, frontend=0):
    """kda_prefill_chunked that also returns the states after the first P tokens
    of a sequence for every requested P (include/kda.h, kda_prefill_chunked_at).

    pos_offsets int32 [S+1] and pos_values int32 [num_pos] on the GPU: the
    positions of sequence s are pos_values[pos_offsets[s]:pos_offsets[s+1]]
    (non-decreasing token counts, 0 <= P <= L_s).
    Returns (o, final_state or None, ckpt_states or None, pos_states)."""
    return _prefill(q, k, v, g, beta, cu_seqlens, num_seqs, initial_state, output_final_state,
                    final_state, ckpt_interval, num_checkpoints, ckpt_states, o, workspace,
                    phases, frontend, pos_offsets, pos_values, pos_states)


def _prefill(q, k, v, g, beta, cu_seqlens, num_seqs, initial_state, output_final_state,
             final_state, ckpt_interval, num_checkpoints, ckpt_states, o, workspace, phases,
             frontend, pos_offsets, pos_values, pos_states):
    """Argument checks, output allocation and the call of the matching entry point."""
    dev = q.device
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [tokens, heads, dim]")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    if num_seqs is None:
        num_seqs = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    # every caller-supplied tensor's dtype and shape first (so that a wrong
    # shape is reported before anything else), then where it lives
    given = [(q, "q", q.dtype, (N, H, Dk)), (k, "k", q.dtype, (N, H, Dk)),
             (v, "v", q.dtype, (N, H, Dv)), (g, "g", torch.float32, (N, H, Dk)),
             (beta, "beta", torch.float32, (N, H)),
             (cu_seqlens, "cu_seqlens", torch.int32, (num_seqs + 1,)),
             (initial_state, "initial_state", torch.float32, (num_seqs, H, Dk, Dv)),
             (o, "o", torch.float32, (N, H, Dv)),
             (final_state, "final_state", torch.float32, (num_seqs, H, Dk, Dv)),
             # the library writes rows [0, ckpt_states.shape[0]) of [rows, H, Dk, Dv]
             (ckpt_states, "ckpt_states", torch.float32, (None, H, Dk, Dv)),
             (workspace, "workspace", torch.uint8, None)]
    if pos_offsets is not None or pos_values is not None:
        if pos_offsets is None or pos_values is None:
            raise ValueError("pos_offsets and pos_values go together")
        npos = int(pos_values.numel())
        given += [(pos_offsets, "pos_offsets", torch.int32, (num_seqs + 1,)),
                  (pos_values, "pos_values", torch.int32, (npos,)),
                  (pos_states, "pos_states", torch.float32, (npos, H, Dk, Dv))]
    for t, name, dt, shape in given:
        _check_props(t, name, dt, shape)
    for t, name, _, _ in given:
        _check_place(t, name, dev)
    if o is None:
        o = torch.empty((N, H, Dv), dtype=torch.float32, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((num_seqs, H, Dk, Dv), dtype=torch.float32, device=dev)
    if ckpt_interval > 0 and ckpt_states is None:
        if num_checkpoints is None:
            raise ValueError("ckpt_interval > 0 needs num_checkpoints or ckpt_states")
        ckpt_states = torch.empty((max(int(num_checkpoints), 0), H, Dk, Dv),
                                  dtype=torch.float32, device=dev)
    need = B.workspace_size(N, num_seqs, H, Dk, Dv, code, CHUNK)
    if need == 0:
        raise B.KdaError(B.KDA_ERR_UNSUPPORTED, "kda_prefill_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ck_ptr = _ptr(ckpt_states) if ckpt_interval > 0 else None
    ck_rows = int(ckpt_states.shape[0]) if ckpt_interval > 0 else 0
    if ckpt_interval > 0 and ckpt_states.numel() == 0:
        # zero checkpoint rows: any aligned non-null pointer is never written
        ck_ptr = workspace.data_ptr()
    head = (_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), _ptr(cu_seqlens), num_seqs, N,
            H, Dk, Dv, CHUNK, _ptr(initial_state), _ptr(final_state), int(ckpt_interval), ck_ptr,
            ck_rows, _ptr(o))
    tail = (_ptr(workspace), workspace.numel(), int(phases))
    if pos_offsets is not None:
        if pos_states is None:
            pos_states = torch.empty((npos, H, Dk, Dv), dtype=torch.float32, device=dev)
        st = B.prefill_at_raw(*head, _ptr(pos_offsets), _ptr(pos_values), npos,
                              _ptr(pos_states), *tail, int(frontend), _stream(dev))
        where = "kda_prefill_chunked_at"
    elif frontend:
        st = B.prefill_ex_raw(*head, *tail, int(frontend), _stream(dev))
        where = "kda_prefill_chunked_ex"
    else:
        st = B.prefill_phases_raw(*head, *tail, _stream(dev))
        where = "kda_prefill_chunked"
    if st != B.KDA_OK:
        raise B.KdaError(st, where)
    return o, final_state, ckpt_states, pos_states


def kda_decode_step(q, k, v, g, beta, state, o=None, frontend=0):
    """One decode step, state [B, H, Dk, Dv] fp32 updated in place (include/kda.h).
    frontend: KDA_FRONT_* bits applied to raw inputs (kda_decode_step_ex).
    Returns o [B, H, Dv] fp32."""
    dev = q.device
    Bsz, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    _check(q, "q", q.dtype, (Bsz, H, Dk), dev)
    _check(k, "k", q.dtype, (Bsz, H, Dk), dev)
    _check(v, "v", q.dtype, (Bsz, H, Dv), dev)
    _check(g, "g", torch.float32, (Bsz, H, Dk), dev)
    _check(beta, "beta", torch.float32, (Bsz, H), dev)
    _check(state, "state", torch.float32, (Bsz, H, Dk, Dv), dev)
    if o is None:
        o = torch.empty((Bsz, H, Dv), dtype=torch.float32, device=dev)
    _check(o, "o", torch.float32, (Bsz, H, Dv), dev)
    if frontend:
        st = B.decode_ex_raw(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), Bsz, H, Dk,
                             Dv, _ptr(state), _ptr(o), int(frontend), _stream(dev))
    else:
        st = B.decode_raw(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), Bsz, H, Dk, Dv,
                          _ptr(state), _ptr(o), _stream(dev))
    if st != B.KDA_OK:
        raise B.KdaError(st, "kda_decode_step")
    return o
