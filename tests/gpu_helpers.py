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


def oracle_full_errors(d: dict, o, hT, seqs=None, heads=None, max_tok_heads: int = 1 << 22,
                       A=None, g_min: float = -5.0, scale: float = 1.0):
    """max|gpu - oracle| and max|oracle| over EVERY element of o and of the
    final state, for the listed sequences (all by default) and heads (all by
    default) of a problem `d` whose tensors may live on the GPU.

    The oracle runs on batches of consecutive whole sequences (consecutive
    sequences are contiguous in both the dense and the packed layout) holding
    at most `max_tok_heads` token·heads, and for longer sequences on groups of
    heads, so host memory stays bounded. Returns a dict with the maxima
    (d_o, r_o, d_s, r_s) and the element counts compared."""
    q, k, v, z, beta = d["q"], d["k"], d["v"], d["z"], d["beta"]
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = d.get("cu_seqlens")
    if cu is None:
        N = B
        starts = np.arange(B + 1, dtype=np.int64) * T
    else:
        starts = cu.cpu().numpy().astype(np.int64)
        N = len(starts) - 1
    seqs = list(range(N)) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    assert heads == list(range(heads[0], heads[-1] + 1)), "heads must be consecutive"
    flat = lambda x: x.reshape((B * T,) + tuple(x.shape[2:]))  # noqa: E731
    qf, kf, vf, zf, bf, of = flat(q), flat(k), flat(v), flat(z), flat(beta), flat(o)
    h0 = d.get("h0")
    # batches of consecutive sequences, then head groups that fit the budget
    batches, cur, cur_tok = [], [], 0
    for n in seqs:
        L = int(starts[n + 1] - starts[n])
        if cur and (cur[-1] != n - 1 or (cur_tok + L) * len(heads) > max_tok_heads):
            batches.append(cur)
            cur, cur_tok = [], 0
        cur.append(n)
        cur_tok += L
    if cur:
        batches.append(cur)
    st = {"d_o": 0.0, "r_o": 0.0, "d_s": 0.0, "r_s": 0.0, "n_o": 0, "n_s": 0}
    for batch in batches:
        a, b = int(starts[batch[0]]), int(starts[batch[-1] + 1])
        L = b - a
        hg = max(1, min(len(heads), max_tok_heads // max(L, 1)))
        for g0 in range(0, len(heads), hg):
            h0i, h1i = heads[g0], heads[min(g0 + hg, len(heads)) - 1] + 1
            sl = (slice(a, b), slice(h0i, h1i))
            sub = lambda x: x[sl].contiguous().cpu()[None]  # noqa: E731
            lens = [int(starts[n + 1] - starts[n]) for n in batch]
            sub_cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
            h0s = None if h0 is None else h0[batch[0]:batch[-1] + 1, h0i:h1i].contiguous().cpu()
            As = None if A is None else A[h0i:h1i].cpu()
            ro, rs = oracle_forward(sub(qf), sub(kf), sub(vf), sub(zf), sub(bf), h0s, sub_cu, As,
                                    g_min, scale)
            go = of[sl].float().cpu().numpy()
            gs = hT[batch[0]:batch[-1] + 1, h0i:h1i].float().cpu().numpy()
            ro = ro[0]
            if go.size:
                st["d_o"] = max(st["d_o"], float(np.abs(go - ro).max()))
                st["r_o"] = max(st["r_o"], float(np.abs(ro).max()))
                assert np.isfinite(go).all()
            st["d_s"] = max(st["d_s"], float(np.abs(gs - rs).max()))
            st["r_s"] = max(st["r_s"], float(np.abs(rs).max()))
            assert np.isfinite(gs).all()
            st["n_o"] += go.size
            st["n_s"] += gs.size
            del ro, rs, go, gs
    return st


def full_errors_ratio(st: dict):
    """(err_o, err_state) = max|d| / max|ref| from oracle_full_errors."""
    return (st["d_o"] / max(st["r_o"], REF_FLOOR), st["d_s"] / max(st["r_s"], REF_FLOOR))
