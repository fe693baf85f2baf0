"""Shared helpers for the GPU parity tests (tests call the HIP path through the
C ABI via the thin binding, and the fp64 oracle on the CPU)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle_forward

TOL_FP32 = 1e-4   # max|d| / max|ref| for fp32 inputs
TOL_BF16 = 2e-2   # max|d| / max|ref| for bf16 inputs (fp32 accumulation)
# Denominator floor: references whose magnitude is below fp32's normal range
# (e.g. a state decayed by e^{-480}) are compared in absolute terms, since the
# kernel's fp32 result is correctly 0 there.
REF_FLOOR = 1e-30


def tol_for(dtype) -> float:
    return TOL_FP32 if dtype == torch.float32 else TOL_BF16


def rel_err(x, ref) -> float:
    x = np.asarray(x.detach().cpu().double() if hasattr(x, "detach") else x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = max(float(np.abs(ref).max()), REF_FLOOR)
    return float(np.abs(x - ref).max() / den)


def to_dev(d: dict, device="cuda") -> dict:
    out = dict(d)
    for key in ("q", "k", "v", "beta", "z", "h0", "cu_seqlens"):
        if out.get(key) is not None:
            out[key] = out[key].to(device)
    return out


def oracle_units(d: dict, units, cols=None, A=None, g_min=-5.0, scale=1.0):
    """Oracle on a sample of (sequence, head) units of a (possibly GPU)
    problem `d`, optionally restricted to value columns `cols` (exact by
    column separability). Returns lists of (o [L, Dv'], hT [Dk, Dv'])."""
    cu = d.get("cu_seqlens")
    cu_h = None if cu is None else cu.cpu().numpy()
    T = d["q"].shape[1]
    res = []
    for (n, h) in units:
        if cu_h is None:
            sl = (n, slice(None), h)
        else:
            sl = (0, slice(int(cu_h[n]), int(cu_h[n + 1])), h)
        q = d["q"][sl].cpu()[None, :, None]
        k = d["k"][sl].cpu()[None, :, None]
        v = d["v"][sl].cpu()
        z = d["z"][sl].cpu()[None, :, None]
        beta = d["beta"][sl].cpu()[None, :, None]
        h0 = d.get("h0")
        h0u = None if h0 is None else h0[n, h].cpu()
        if cols is not None:
            v = v[:, cols]
            if h0u is not None:
                h0u = h0u[:, cols]
        Au = None if A is None else A[h:h + 1].cpu()
        o, hT = oracle_forward(q, k, v[None, :, None], z, beta,
                               None if h0u is None else h0u[None, None], None, Au, g_min, scale)
        res.append((o[0, :, 0], hT[0, 0]))
    del T
    return res


def gpu_units(o, hT, d: dict, units, cols=None):
    """The same units cut out of the GPU outputs (moved to the host)."""
    cu = d.get("cu_seqlens")
    cu_h = None if cu is None else cu.cpu().numpy()
    res = []
    for (n, h) in units:
        if cu_h is None:
            ou = o[n, :, h]
        else:
            ou = o[0, int(cu_h[n]):int(cu_h[n + 1]), h]
        su = hT[n, h]
        if cols is not None:
            ou, su = ou[:, cols], su[:, cols]
        res.append((ou.float().cpu().numpy(), su.float().cpu().numpy()))
    return res


def compare_units(gpu, ref):
    """Errors measured over all sampled units jointly (max over elements)."""
    go = np.concatenate([g[0].ravel() for g in gpu])
    ro = np.concatenate([r[0].ravel() for r in ref])
    gs = np.concatenate([g[1].ravel() for g in gpu])
    rs = np.concatenate([r[1].ravel() for r in ref])
    return rel_err(go, ro), rel_err(gs, rs)
