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
          "logits": _lib.KDA_GATE_LOGITS}


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
              workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward. q, k: [B, T, H, Dk]; v: [B, T, H, Dv] (bf16 or
    fp32); g: fp32 [B, T, H, Dk] (log-decay, its chunk cumsum, or logits per
    `gate`); beta: fp32 [B, T, H]; initial_state: fp32 [N, H, Dk, Dv].
    Returns (o, final_state)."""
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
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    _need(o, "o", dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, dev)
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
