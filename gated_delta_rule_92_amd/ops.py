"""Thin PyTorch-facing binding over the C ABI (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in libkda.so's kernels. Outputs are allocated here with
``torch.empty`` and filled by the library.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_GATES = {"logdecay": _lib.KDA_GATE_LOGDECAY, "cumsum": _lib.KDA_GATE_CUMSUM,
          "logits": _lib.KDA_GATE_LOGITS, "softplus": _lib.KDA_GATE_SOFTPLUS}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.KDA_BFLOAT16
    if t.dtype == torch.float32:
        return _lib.KDA_FLOAT32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def gate(z: torch.Tensor, A_log: Optional[torch.Tensor] = None, g_min: float = -5.0,
         chunk: int = 0, cu_seqlens: Optional[torch.Tensor] = None,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """g = g_min * sigmoid(exp(A_log[h]) * z), then (chunk > 0) the
    chunk-local inclusive cumsum. z: fp32 [B, T, H, Dk]."""
    lib = _lib.load()
    _need(z, "z", torch.float32)
    B, T, H, Dk = z.shape
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, z.device)
    N = 0
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, z.device)
        N = cu_seqlens.numel() - 1
    g = torch.empty_like(z) if out is None else out
    _need(g, "out", torch.float32, z.device)
    with torch.cuda.device(z.device):
        rc = lib.kda_gate(_ptr(z), _ptr(A_log), float(g_min), _ptr(cu_seqlens), N, B, T, H, Dk,
                          int(chunk), _ptr(g), _stream(z.device))
    _lib.check(rc, "kda_gate")
    return g


def workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, N: int, chunk: int = 64,
                   dtype=torch.bfloat16) -> int:
    lib = _lib.load()
    import ctypes
    out = ctypes.c_size_t(0)
    code = _lib.KDA_BFLOAT16 if dtype == torch.bfloat16 else _lib.KDA_FLOAT32
    _lib.check(lib.kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, N, chunk, code, ctypes.byref(out)),
               "kda_chunk_fwd_workspace_size")
    return int(out.value)


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
              A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
              scale: float = 1.0, output_final_state: bool = True,
              o: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, output: bool = True
              ) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Chunkwise KDA forward. q, k: [B, T, H, Dk]; v: [B, T, H, Dv] (bf16 or
    fp32); g: fp32 [B, T, H, Dk] (log-decay, its chunk cumsum, or logits per
    `gate`); beta: fp32 [B, T, H]; initial_state: fp32 [N, H, Dk, Dv].
    Returns (o, final_state); with output=False only the final state is
    computed and o is None."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (N, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    if not output:
        o = None
        output_final_state = True
    elif o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    if o is not None:
        _need(o, "o", dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, dev)
    with torch.cuda.device(dev):
        ws_bytes = workspace_size(B, T, H, Dk, Dv, N, chunk, dt)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _GATES[gate],
                               _ptr(A_log), float(g_min), _ptr(beta), _ptr(initial_state),
                               _ptr(cu_seqlens), N, B, T, H, Dk, Dv, int(chunk), float(scale),
                               _ptr(o), _ptr(final_state), _ptr(workspace), ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_fwd")
    return o, final_state


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, o: torch.Tensor, final_state: Optional[torch.Tensor],
                      initial_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
                      A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
                      scale: float = 1.0) -> None:
    """kda_chunk_fwd_noalloc: chunk_fwd into caller-provided o [B, T, H, Dv] and
    final_state [N, H, Dk, Dv] (or None), with the library's static device
    scratch as the workspace; neither this binding nor the library allocates."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3] or o.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, g, beta, o")
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != (N, H, Dk, Dv):
                raise ValueError(f"{name} must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                       _GATES[gate], _ptr(A_log), float(g_min), _ptr(beta),
                                       _ptr(initial_state), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                                       int(chunk), float(scale), _ptr(o), _ptr(final_state),
                                       _stream(dev))
    _lib.check(rc, "kda_chunk_fwd_noalloc")


def chunk_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, out_gate: torch.Tensor,
                    norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                    initial_state: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
                    A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
                    scale: float = 1.0, output_final_state: bool = True,
                    y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """chunk_fwd followed by the block's output epilogue:
    y = sigmoid(out_gate) * RMSNorm(o) * norm_weight (per token-head over Dv).
    out_gate: [B, T, H, Dv] in q's dtype; norm_weight: fp32 [Dv] or None.
    Returns (y, final_state)."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("out_gate", out_gate)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3] or out_gate.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, g, beta, out_gate")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (N, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", torch.float32, dev)
        if tuple(norm_weight.shape) != (Dv,):
            raise ValueError("norm_weight must be [Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    _need(y, "y", dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        ws_bytes = workspace_size(B, T, H, Dk, Dv, N, chunk, dt)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                     _GATES[gate], _ptr(A_log), float(g_min), _ptr(beta),
                                     _ptr(initial_state), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                                     int(chunk), float(scale), _ptr(out_gate), _ptr(norm_weight),
                                     float(eps), _ptr(y), _ptr(final_state), _ptr(workspace),
                                     ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_fwd_gated")
    return y, final_state


def gated_rmsnorm(o: torch.Tensor, out_gate: torch.Tensor, norm_weight: Optional[torch.Tensor] = None,
                  eps: float = 1e-6, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The output epilogue alone: y = sigmoid(out_gate) * RMSNorm(o) * norm_weight
    over the last dimension. o, out_gate: [..., Dv] (bf16 or fp32)."""
    lib = _lib.load()
    dev = o.device
    _need(o, "o", None, dev)
    _need(out_gate, "out_gate", o.dtype, dev)
    if out_gate.shape != o.shape:
        raise ValueError("o and out_gate must have the same shape")
    Dv = o.shape[-1]
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", torch.float32, dev)
    if y is None:
        y = torch.empty_like(o)
    _need(y, "y", o.dtype, dev)
    rows = o.numel() // Dv
    with torch.cuda.device(dev):
        rc = lib.kda_gated_rmsnorm(_ptr(o), _ptr(out_gate), _dtype_code(o), _ptr(norm_weight),
                                   float(eps), rows, Dv, _ptr(y), _stream(dev))
    _lib.check(rc, "kda_gated_rmsnorm")
    return y


def transition(k: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
               cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
               A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
               M: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
               ) -> torch.Tensor:
    """State map of each (sequence, head): fp32 M [N, H, Dk, Dk] with
    S_final = M @ S_initial + S_final(S_initial = 0). k: [B, T, H, Dk] bf16."""
    lib = _lib.load()
    dev = k.device
    _need(k, "k", None, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = k.shape
    if g.shape != k.shape or beta.shape != k.shape[:3]:
        raise ValueError("shape mismatch among k, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    if M is None:
        M = torch.empty((N, H, Dk, Dk), dtype=torch.float32, device=dev)
    _need(M, "M", torch.float32, dev)
    # the transition's workspace holds only the order of packed sequences
    ws_bytes = workspace_size(B, T, H, Dk, Dk, N, chunk, k.dtype) if cu_seqlens is not None else 0
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_transition(_ptr(k), _dtype_code(k), _ptr(g), _GATES[gate], _ptr(A_log),
                                      float(g_min), _ptr(beta), _ptr(cu_seqlens), N, B, T, H, Dk,
                                      int(chunk), _ptr(M), _ptr(workspace), ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_transition")
    return M


def compose_states(M: torch.Tensor, b: torch.Tensor, initial_state: Optional[torch.Tensor],
                   nseq: int, P: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Entry states of P consecutive segments per sequence: starts[s*P] =
    initial_state[s], starts[s*P+p+1] = M[s*P+p] @ starts[s*P+p] + b[s*P+p].
    M: fp32 [nseq*P, H, Dk, Dk]; b: fp32 [nseq*P, H, Dk, Dv]."""
    lib = _lib.load()
    dev = b.device
    _need(M, "M", torch.float32, dev)
    _need(b, "b", torch.float32, dev)
    _, H, Dk, Dv = b.shape
    if b.shape[0] != nseq * P or tuple(M.shape) != (nseq * P, H, Dk, Dk):
        raise ValueError("M must be [nseq*P, H, Dk, Dk] and b [nseq*P, H, Dk, Dv]")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (nseq, H, Dk, Dv):
            raise ValueError("initial_state must be [nseq, H, Dk, Dv]")
    if out is None:
        out = torch.empty_like(b)
    _need(out, "out", torch.float32, dev)
    with torch.cuda.device(dev):
        rc = lib.kda_compose_states(_ptr(M), _ptr(b), _ptr(initial_state), nseq, P, H, Dk, Dv,
                                    _ptr(out), _stream(dev))
    _lib.check(rc, "kda_compose_states")
    return out


def chunk_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, segments: int = 8,
                    gate: str = "logdecay", A_log: Optional[torch.Tensor] = None,
                    g_min: float = -5.0, chunk: int = 64, scale: float = 1.0
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The chunk forward with every sequence cut into `segments` consecutive
    pieces that run in parallel (the one-GPU form of a context split), one
    kda_chunk_fwd_split call: per piece its state map and zero-start final
    state, the entry states chained per sequence, then every piece from its
    entry state. Same results as chunk_fwd up to rounding. Returns
    (o, final_state)."""
    import ctypes
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (N, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    out = ctypes.c_size_t(0)
    _lib.check(lib.kda_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, N, int(segments), int(chunk),
                                                      _dtype_code(q), ctypes.byref(out)),
               "kda_chunk_fwd_split_workspace_size")
    ws_len = int(out.value)
    workspace = torch.empty(ws_len, dtype=torch.uint8, device=dev) if ws_len > 0 else None
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_fwd_split(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                     _GATES[gate], _ptr(A_log), float(g_min), _ptr(beta),
                                     _ptr(initial_state), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                                     int(chunk), int(segments), float(scale), _ptr(o),
                                     _ptr(final_state), _ptr(workspace), ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_fwd_split")
    return o, final_state


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor, gate: str = "logdecay",
                   A_log: Optional[torch.Tensor] = None, g_min: float = -5.0,
                   scale: float = 1.0, o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token. q, k: [N, H, Dk]; v: [N, H, Dv]; g: fp32 [N, H, Dk];
    beta: fp32 [N, H]; state: fp32 [N, H, Dk, Dv], updated in place. Returns o."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError("state must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, Dv), dtype=dt, device=dev)
    with torch.cuda.device(dev):
        rc = lib.kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                    _GATES[gate], _ptr(A_log), float(g_min), _ptr(beta),
                                    _ptr(state), N, H, Dk, Dv, float(scale), _ptr(o),
                                    _stream(dev))
    _lib.check(rc, "kda_recurrent_step")
    return o


def bwd_workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, N: int, chunk: int = 64,
                       dtype=torch.bfloat16) -> int:
    """kda_chunk_bwd_workspace_size: bytes of the backward workspace, with the
    region of the scans' context split where dense sequences (N == B) of this
    shape take it on the current device."""
    lib = _lib.load()
    import ctypes
    out = ctypes.c_size_t(0)
    code = _lib.KDA_BFLOAT16 if dtype == torch.bfloat16 else _lib.KDA_FLOAT32
    _lib.check(lib.kda_chunk_bwd_workspace_size(B, T, H, Dk, Dv, N, chunk, code,
                                                ctypes.byref(out)),
               "kda_chunk_bwd_workspace_size")
    return int(out.value)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, do: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              d_final_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
              A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
              scale: float = 1.0, want_dh0: bool = True,
              workspace: Optional[torch.Tensor] = None, saved: bool = False) -> dict:
    """Gradients of chunk_fwd: given do [B, T, H, Dv] and d_final_state
    [N, H, Dk, Dv] (None = zero), returns a dict with dq, dk, dv (input
    dtype), dg (fp32, w.r.t. the per-token log-decay), dbeta (fp32) and dh0
    (fp32 [N, H, Dk, Dv], or None when want_dh0 is False). gate is
    "logdecay" (g = log-decay) or "logits" (g = z). saved=True calls
    kda_chunk_bwd_saved: workspace must be the one chunk_fwd_train filled from
    the same inputs."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3] or do.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, g, beta, do")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != (N, H, Dk, Dv):
                raise ValueError(f"{name} must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
           "dh0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dh0
           else None}
    ws_bytes = bwd_workspace_size(B, T, H, Dk, Dv, N, chunk, dt)
    if workspace is None:
        if saved:
            raise ValueError("saved=True needs the workspace chunk_fwd_train filled")
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    fn = lib.kda_chunk_bwd_saved if saved else lib.kda_chunk_bwd
    with torch.cuda.device(dev):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _GATES[gate],
                               _ptr(A_log), float(g_min), _ptr(beta), _ptr(initial_state),
                               _ptr(cu_seqlens), N, B, T, H, Dk, Dv, int(chunk), float(scale),
                               _ptr(do), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
                               _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                               _ptr(out["dh0"]), _ptr(workspace), ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_bwd_saved" if saved else "kda_chunk_bwd")
    return out


def chunk_fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, gate: str = "logdecay",
                    A_log: Optional[torch.Tensor] = None, g_min: float = -5.0, chunk: int = 64,
                    scale: float = 1.0, output_final_state: bool = True,
                    bwd_workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """kda_chunk_fwd_train: chunk_fwd's (o, final_state) and, in the same
    pass, the backward's checkpoints in a backward workspace (allocated when
    bwd_workspace is None). Returns (o, final_state, bwd_workspace); pass the
    workspace to chunk_bwd(..., saved=True) with the same inputs. Its size
    decides whether both calls take the context split of long dense
    sequences (bwd_workspace_size includes it where it applies), so the two
    calls must get the same tensor."""
    lib = _lib.load()
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape or \
            beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (N, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, dev)
    o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) \
        if output_final_state else None
    ws_bytes = bwd_workspace_size(B, T, H, Dk, Dv, N, chunk, dt)
    if bwd_workspace is None:
        bwd_workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_len = bwd_workspace.numel() * bwd_workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.kda_chunk_fwd_train(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g),
                                     _GATES[gate], _ptr(A_log), float(g_min), _ptr(beta),
                                     _ptr(initial_state), _ptr(cu_seqlens), N, B, T, H, Dk, Dv,
                                     int(chunk), float(scale), _ptr(o), _ptr(final_state),
                                     _ptr(bwd_workspace), ws_len, _stream(dev))
    _lib.check(rc, "kda_chunk_fwd_train")
    return o, final_state, bwd_workspace


def gate_bwd(z: torch.Tensor, dg: torch.Tensor, A_log: Optional[torch.Tensor] = None,
             g_min: float = -5.0, want_dA: bool = True,
             dz: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gradient of g = g_min * sigmoid(exp(A_log[h]) z) w.r.t. z and A_log.
    z, dg: fp32 [..., H, Dk]. Returns (dz, dA_log [H] or None)."""
    lib = _lib.load()
    _need(z, "z", torch.float32)
    _need(dg, "dg", torch.float32, z.device)
    if dg.shape != z.shape:
        raise ValueError("dg must have z's shape")
    H, Dk = z.shape[-2], z.shape[-1]
    rows = z.numel() // (H * Dk)
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, z.device)
    if dz is None:
        dz = torch.empty_like(z)
    _need(dz, "dz", torch.float32, z.device)
    dA = torch.empty(H, dtype=torch.float32, device=z.device) if want_dA else None
    with torch.cuda.device(z.device):
        rc = lib.kda_gate_bwd(_ptr(z), _ptr(A_log), float(g_min), _ptr(dg), rows, H, Dk, _ptr(dz),
                              _ptr(dA), _stream(z.device))
    _lib.check(rc, "kda_gate_bwd")
    return dz, dA


def device_status(clear: bool = False, device: Optional[torch.device] = None) -> int:
    """kda_device_status: the sticky device-side failure flags of the current
    (or given) device, KDA_DEVICE_WAIT_TIMEOUT | KDA_DEVICE_DECAY_OUT_OF_RANGE
    bits; waits for the device's current stream. clear=True resets them."""
    import ctypes
    lib = _lib.load()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        _lib.check(lib.kda_device_status(ctypes.byref(out), int(bool(clear)), _stream(dev)),
                   "kda_device_status")
    return int(out.value)


def debug_set_spin_limit(polls: int) -> None:
    """kda_debug_set_spin_limit (testing aid): polls before a bounded wait of
    the pipelined kernel gives up; 0 restores the default."""
    _lib.check(_lib.load().kda_debug_set_spin_limit(int(polls)), "kda_debug_set_spin_limit")
