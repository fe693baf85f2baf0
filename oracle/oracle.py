"""ctypes wrapper around ``kda_oracle.c`` (fp64, CPU, test infrastructure only).

Sources, cited by page title and section:
  [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华" (stevenstage.github.io,
             posts/blog7), sections "Kimi Delta Attention" (KDA equation) and
             "Chunkwise parallel form" (gamma equation, new-gate equation).

Every array crossing this wrapper is converted to contiguous float64 numpy;
bf16 inputs therefore enter as their exact (already rounded) values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_NAME = "libkda_oracle.so"
_lib = None


def host_threads() -> int:
    """Threads the oracle runs on by default: the cores this process may use,
    capped by OMP_NUM_THREADS (16 when unset), the host share of one GPU."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        avail = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        cap = 16
    return max(1, min(avail, cap if cap > 0 else 16))


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def build_oracle(src: str = _SRC, out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (-O2, no fast-math). Returns the .so path."""
    out = out or library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu99", "-Wall", "-shared", "-fPIC", src, "-o", tmp,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None and os.environ.get("KDA_ORACLE_LIB"):
        # a build of the same source with sanitizers (the CPU sanitizer test)
        _lib = _bind(ctypes.CDLL(os.environ["KDA_ORACLE_LIB"]))
    if _lib is None:
        if not os.path.exists(library_path()) or (
                os.path.getmtime(library_path()) < os.path.getmtime(_SRC)):
            build_oracle()
        _lib = _bind(ctypes.CDLL(library_path()))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kda_oracle_gate.argtypes = [dp, dp, ctypes.c_double, ctypes.c_long, ctypes.c_int,
                                    ctypes.c_int, dp]
    lib.kda_oracle_gate.restype = None
    lib.kda_oracle_cumsum.argtypes = [dp, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, dp]
    lib.kda_oracle_cumsum.restype = None
    lib.kda_oracle_recurrence.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, dp, dp, ctypes.c_int]
    lib.kda_oracle_recurrence.restype = ctypes.c_int
    lib.kda_oracle_gate_bwd.argtypes = [dp, dp, ctypes.c_double, dp, ctypes.c_long, ctypes.c_int,
                                        ctypes.c_int, dp, dp]
    lib.kda_oracle_gate_bwd.restype = None
    lib.kda_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp,
                                        dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_backward.restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact upcast on the CPU
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _cu_array(cu, n_tokens: int, batch: int) -> np.ndarray:
    if cu is None:
        T = n_tokens // batch
        return np.arange(batch + 1, dtype=np.int32) * T
    if hasattr(cu, "detach"):
        cu = cu.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int32))


def oracle_gate(z, A=None, g_min: float = -5.0, lib_path: Optional[str] = None) -> np.ndarray:
    """g = g_min * sigmoid(exp(A_h) z) over z of shape [..., H, Dk] (fp64).

    [KDA-blog §Chunkwise parallel form, new-gate equation]
    """
    lib = _load(lib_path)
    z64 = _f64(z)
    H, Dk = z64.shape[-2], z64.shape[-1]
    rows = z64.size // (H * Dk)
    A64 = None if A is None else _f64(A).reshape(H)
    out = np.empty_like(z64)
    lib.kda_oracle_gate(_dp(z64), _dp(A64), float(g_min), rows, H, Dk, _dp(out))
    return out


def oracle_cumsum(g, chunk: int, cu_seqlens=None, lib_path: Optional[str] = None) -> np.ndarray:
    """Chunk-local inclusive cumsum of g [B, T, H, Dk] (restarting at every
    sequence start and every `chunk` tokens from it).

    [KDA-blog §Chunkwise parallel form, gamma equation]
    """
    lib = _load(lib_path)
    g64 = _f64(g)
    B, T, H, Dk = g64.shape
    cu = _cu_array(cu_seqlens, B * T, B)
    out = np.empty_like(g64)
    lib.kda_oracle_cumsum(_dp(g64), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                          len(cu) - 1, H, Dk, int(chunk), _dp(out))
    return out


def oracle_recurrence(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                      scale: float = 1.0, nthreads: Optional[int] = None,
                      lib_path: Optional[str] = None):
    """Token-by-token fp64 KDA recurrence.

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
    initial_state: [N, H, Dk, Dv] or None (zeros); cu_seqlens: [N+1] with
    B == 1, or None (N = B dense sequences). g is the per-token log-decay.
    Returns (o [B, T, H, Dv], final_state [N, H, Dk, Dv]) as float64.

    [KDA-blog §Kimi Delta Attention, KDA equation]
    """
    lib = _load(lib_path)
    q64, k64, v64, g64, b64 = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, Dk = q64.shape
    Dv = v64.shape[-1]
    cu = _cu_array(cu_seqlens, B * T, B)
    N = len(cu) - 1
    h064 = None if initial_state is None else _f64(initial_state)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    hT = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    nthreads = nthreads or host_threads()
    rc = lib.kda_oracle_recurrence(_dp(q64), _dp(k64), _dp(v64), _dp(g64), _dp(b64),
                                   _dp(h064), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   N, H, Dk, Dv, float(scale), _dp(o), _dp(hT), int(nthreads))
    if rc != 0:
        raise ValueError("oracle: invalid arguments")
    return o, hT


def oracle_backward(q, k, v, g, beta, do, initial_state=None, d_final_state=None,
                    cu_seqlens=None, scale: float = 1.0, nthreads: Optional[int] = None,
                    lib_path: Optional[str] = None):
    """Gradients of the token recurrence (fp64): given do [B, T, H, Dv] (the
    gradient w.r.t. o) and d_final_state [N, H, Dk, Dv] (w.r.t. the final
    state, None = zero), returns a dict with dq, dk, dg [B, T, H, Dk],
    dv [B, T, H, Dv], dbeta [B, T, H] and dh0 [N, H, Dk, Dv]. g is the
    per-token log-decay, as in oracle_recurrence; dg is the gradient w.r.t. it.

    [KDA-blog §Kimi Delta Attention, KDA equation], differentiated step by
    step in reverse order (the pages give no backward).
    """
    lib = _load(lib_path)
    q64, k64, v64, g64, b64, do64 = (_f64(x) for x in (q, k, v, g, beta, do))
    B, T, H, Dk = q64.shape
    Dv = v64.shape[-1]
    cu = _cu_array(cu_seqlens, B * T, B)
    N = len(cu) - 1
    h064 = None if initial_state is None else _f64(initial_state)
    dhT64 = None if d_final_state is None else _f64(d_final_state)
    out = {"dq": np.zeros_like(q64), "dk": np.zeros_like(k64), "dv": np.zeros_like(v64),
           "dg": np.zeros_like(g64), "dbeta": np.zeros_like(b64),
           "dh0": np.zeros((N, H, Dk, Dv), dtype=np.float64)}
    nthreads = nthreads or host_threads()
    rc = lib.kda_oracle_backward(_dp(q64), _dp(k64), _dp(v64), _dp(g64), _dp(b64), _dp(h064),
                                 cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), N, H, Dk, Dv,
                                 float(scale), _dp(do64), _dp(dhT64), _dp(out["dq"]),
                                 _dp(out["dk"]), _dp(out["dv"]), _dp(out["dg"]),
                                 _dp(out["dbeta"]), _dp(out["dh0"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle backward: invalid arguments or out of memory")
    return out


def oracle_gate_backward(z, dg, A=None, g_min: float = -5.0, lib_path: Optional[str] = None):
    """Gradient of g = g_min * sigmoid(exp(A_h) z) (z, dg: [..., H, Dk]):
    returns (dz, dA) with dA [H] the gradient w.r.t. A_h (None if A is None).

    [KDA-blog §Chunkwise parallel form, new-gate equation], differentiated.
    """
    lib = _load(lib_path)
    z64, dg64 = _f64(z), _f64(dg)
    H, Dk = z64.shape[-2], z64.shape[-1]
    rows = z64.size // (H * Dk)
    A64 = None if A is None else _f64(A).reshape(H)
    dz = np.empty_like(z64)
    dA = None if A is None else np.empty(H, dtype=np.float64)
    lib.kda_oracle_gate_bwd(_dp(z64), _dp(A64), float(g_min), _dp(dg64), rows, H, Dk, _dp(dz),
                            _dp(dA))
    return dz, dA


def oracle_forward(q, k, v, z, beta, initial_state=None, cu_seqlens=None, A=None,
                   g_min: float = -5.0, scale: float = 1.0, nthreads: Optional[int] = None,
                   lib_path: Optional[str] = None):
    """Gate then recurrence: g = g_min * sigmoid(exp(A_h) z), alpha = exp(g).

    [KDA-blog §Chunkwise parallel form, new-gate equation; §Kimi Delta
    Attention, KDA equation]
    """
    g = oracle_gate(z, A, g_min, lib_path=lib_path)
    return oracle_recurrence(q, k, v, g, beta, initial_state, cu_seqlens, scale, nthreads,
                             lib_path=lib_path)


def oracle_gate_softplus(z, A=None) -> np.ndarray:
    """The pages' earlier, unbounded gate: g = -exp(A_h) * softplus(z), with
    softplus(z) = log(1 + e^z) written as max(z, 0) + log1p(e^{-|z|}) so that
    it neither overflows nor loses its small values. z: [..., H, Dk]; A: [H]
    or None (e^{A_h} = 1). fp64 numpy.

    [KDA-blog §Chunkwise parallel form, old-gate equation]
    """
    z64 = _f64(z)
    sp = np.maximum(z64, 0.0) + np.log1p(np.exp(-np.abs(z64)))
    scale = 1.0 if A is None else np.exp(_f64(A))[:, None]
    return -scale * sp


def oracle_forward_softplus(q, k, v, z, beta, initial_state=None, cu_seqlens=None, A=None,
                            scale: float = 1.0, nthreads: Optional[int] = None,
                            lib_path: Optional[str] = None):
    """The unbounded-gate forward: g = -exp(A_h) softplus(z), alpha = exp(g),
    then the token recurrence.

    [KDA-blog §Chunkwise parallel form, old-gate equation; §Kimi Delta
    Attention, KDA equation]
    """
    g = oracle_gate_softplus(z, A)
    return oracle_recurrence(q, k, v, g, beta, initial_state, cu_seqlens, scale, nthreads,
                             lib_path=lib_path)


def gather_units(x, cu, units: Sequence[tuple]):
    """Pack the rows of the listed (sequence, head) units of a [1, Ttot, H, ...]
    or [B, T, H, ...] tensor into [1, sum T_n, 1, ...] (fp64) with its own
    cu_seqlens, so the oracle can compute a sample of units one by one."""
    x64 = _f64(x)
    B, T = x64.shape[0], x64.shape[1]
    cu = _cu_array(cu, B * T, B)
    flat = x64.reshape((B * T,) + x64.shape[2:])
    parts = [flat[cu[n]:cu[n + 1], h][:, None] for (n, h) in units]
    lens = [cu[n + 1] - cu[n] for (n, _) in units]
    new_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return np.concatenate(parts, axis=0)[None], new_cu
