"""Test-only numpy (fp64) renderings of the chunkwise-parallel form.

Sources, cited by page title and section:
  [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Chunkwise
             parallel form": the gamma equation (cumulative per-channel decay
             inside a chunk), the W/U equation (W = M (Gamma*K), U = M V), the
             pseudo-value definition (V~ = U - W S) and the A/O equation
             (A = Tril[(Q*Gamma)(K/Gamma)^T], O = (Gamma*Q) S + A V~).

The page names the auxiliary matrix M without printing it and does not print
the state hand-off between chunks. Both are derived here from the KDA
equation (section "Kimi Delta Attention") by unrolling it inside a chunk:

    S_r = Diag(Gamma_r) S_0 + sum_{i<=r} Diag(Gamma_r / Gamma_i) k_i d_i^T
    (I + A_kk) D = Diag(beta) (V - (Gamma*K) S_0),
    A_kk[r, i] = beta_r sum_c k_r[c] k_i[c] Gamma_r[c] / Gamma_i[c]   (i < r)

so M = (I + A_kk)^{-1} Diag(beta), D = V~, o_r = S_r^T q_r gives the A/O
equation with an inclusive Tril, and the state leaving the chunk is
S_C = Diag(Gamma_C) S_0 + (K * Gamma_C / Gamma)^T V~.

`chunk_form_pages` writes these formulas out directly. `chunk_form_tiled` is
the same algebra arranged the way the GPU kernel arranges it (16-token tiles
with per-tile reference points, block forward substitution, optional bf16
rounding at the points where the kernel rounds), so that the arrangement can
be checked on the CPU before any kernel runs. Neither is the oracle; the
tests compare both against it.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) via fp32, return fp64."""
    x32 = np.asarray(x, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32).astype(np.float64)


def chunk_form_pages(q, k, v, g, beta, S0, C):
    """One unit: q, k, g [T, Dk]; v [T, Dv]; beta [T]; S0 [Dk, Dv] (fp64)."""
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        G = np.cumsum(g[s:e], axis=0)            # log gamma^r, inclusive
        Gam = np.exp(G)
        L = e - s
        Akk = np.tril((b[:, None] * (K * Gam)) @ (K / Gam).T, -1)
        M = np.linalg.inv(np.eye(L) + Akk) @ np.diag(b)
        W = M @ (Gam * K)
        U = M @ V
        Vt = U - W @ S
        A = np.tril((Q * Gam) @ (K / Gam).T)
        o[s:e] = (Gam * Q) @ S + A @ Vt
        S = Gam[-1][:, None] * S + (K * (Gam[-1] / Gam)).T @ Vt
    return o, S


def _inv_unit_lower(A):
    """(I + A)^{-1} for strictly-lower A by forward substitution."""
    n = A.shape[0]
    Tm = np.zeros_like(A)
    for r in range(n):
        Tm[r, r] = 1.0
        for j in range(r):
            Tm[r, j] = -np.dot(A[r, j:r], Tm[j:r, j])
    return Tm


def chunk_form_tiled(q, k, v, g, beta, S0, C=64, tile=16, round_bf16=False):
    """The kernel's arrangement of the chunk form (one unit, fp64 arithmetic).

    Within a chunk, tile I covers rows [16I, 16I+16). rho_I is the cumulative
    log-decay just before tile I (rho_0 = 0). Every exponent that appears is
    one of e^{G_r - rho_I} <= 1, e^{rho_I - G_i} <= e^{16|g_min|} (diagonal
    tiles) or a product of factors <= 1, so nothing overflows in fp32 when
    g >= g_min = -5.
    """
    rnd = bf16_round if round_bf16 else (lambda x: x)
    T, Dk = q.shape
    Dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((T, Dv))
    nt = C // tile
    for s in range(0, T, C):
        e = min(s + C, T)
        L = e - s
        Q = np.zeros((C, Dk)); K = np.zeros((C, Dk)); V = np.zeros((C, Dv))
        gg = np.zeros((C, Dk)); b = np.zeros(C)
        Q[:L], K[:L], V[:L], gg[:L], b[:L] = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e]
        G = np.cumsum(gg, axis=0)
        rho = np.zeros((nt + 1, Dk))
        for I in range(1, nt + 1):
            rho[I] = G[tile * I - 1]
        GC = G[-1]
        tix = np.arange(C) // tile
        E = np.exp(G - rho[tix])
        Einv = np.exp(rho[tix] - G)
        Kl = rnd(K * E)
        Ql = rnd(Q * E)
        Kd = rnd(K * Einv)
        Kg = rnd((K * E) * np.exp(rho[tix]))
        Qg = rnd((Q * E) * np.exp(rho[tix]))
        Kt = rnd((K * Einv * np.exp(rho[tix + 1] - rho[tix])) * np.exp(GC - rho[tix + 1]))
        Akk = np.zeros((C, C)); Aqk = np.zeros((C, C))
        for I in range(nt):
            ri = slice(tile * I, tile * I + tile)
            for J in range(I + 1):
                rj = slice(tile * J, tile * J + tile)
                right = Kd[rj] if I == J else rnd(Kd[rj] * np.exp(rho[I] - rho[J]))
                a_kk = b[ri][:, None] * (Kl[ri] @ right.T)
                a_qk = Ql[ri] @ right.T
                if I == J:
                    a_kk = np.tril(a_kk, -1)
                    a_qk = np.tril(a_qk)
                Akk[ri, rj] = a_kk
                Aqk[ri, rj] = a_qk
        Aqk = rnd(Aqk)
        Tdiag = [rnd(_inv_unit_lower(Akk[tile * I:tile * I + tile, tile * I:tile * I + tile]))
                 for I in range(nt)]
        Akk_off = rnd(Akk)
        Sop = rnd(S)
        Y = V - Kg @ Sop
        X = np.zeros((C, Dv))
        for I in range(nt):
            ri = slice(tile * I, tile * I + tile)
            acc = b[ri][:, None] * Y[ri]
            for J in range(I):
                rj = slice(tile * J, tile * J + tile)
                acc = acc - Akk_off[ri, rj] @ X[rj]
            X[ri] = rnd(Tdiag[I] @ rnd(acc))
        O = Qg @ Sop + Aqk @ X
        o[s:e] = O[:L]
        S = np.exp(GC)[:, None] * S + Kt.T @ X
    return o, S


def tile_backward(q, k, v, g, beta, S0, do, dST, tile=16, scale=1.0):
    """Backward of one unit in the 16-token tile arrangement of the GPU
    backward (three passes), fp64.

    q, k, g: [T, Dk]; v, do: [T, Dv]; beta: [T]; S0, dST: [Dk, Dv].
    Inside a tile with inclusive cumulative log-decay G (natural log),
    Gamma = e^G, Kg = K*Gamma, Qg = scale*Q*Gamma, Kt = K*e^{G_L-G},
    Akk = beta_r sum_c k_r k_i e^{G_r-G_i} (i < r), Aqk = scale sum_c q_r k_i
    e^{G_r-G_i} (i <= r), T = (I + Akk)^{-1}:
      forward   U = V - Kg S,  V~ = T (beta U),  S' = Diag(Gamma_L) S + Kt^T V~
      reverse   dV~ = Kt dS' + Aqk^T dO,  dY = T^T dV~,
                dS = Diag(Gamma_L) dS' + Qg^T dO - Kg^T (beta dY)
      per tile  the products' derivatives, chained into q, k, G, then
                dg = reverse cumulative sum of dG inside the tile.
    The decay factors of the tile products are split at a reference point
    rho (G of the tile's eighth token); the products do not depend on rho,
    so its own derivative is zero.
    Returns dq, dk, dv, dg, dbeta, dS0.
    """
    T, Dk = k.shape
    Dv = v.shape[1]
    nt = (T + tile - 1) // tile
    tiles = [(j * tile, min(T, (j + 1) * tile)) for j in range(nt)]

    def prep(a, b):
        G = np.cumsum(g[a:b], axis=0)
        L = b - a
        Gam = np.exp(G)
        Kg = k[a:b] * Gam
        Qg = scale * q[a:b] * Gam
        Kt = k[a:b] * np.exp(G[L - 1] - G)
        rho = G[min(7, L - 1)]
        Kl, Ql, Kd = k[a:b] * np.exp(G - rho), scale * q[a:b] * np.exp(G - rho), k[a:b] * np.exp(rho - G)
        At = np.tril(Kl @ Kd.T, -1)
        Akk = beta[a:b, None] * At
        Aqk = np.tril(Ql @ Kd.T)
        Tm = np.linalg.inv(np.eye(L) + Akk)
        return dict(G=G, Gam=Gam, Kg=Kg, Qg=Qg, Kt=Kt, Kl=Kl, Ql=Ql, Kd=Kd, At=At, Aqk=Aqk,
                    T=Tm, GL=Gam[L - 1], rho=rho)

    # pass 1: states entering each tile, U and V~
    S = S0.copy()
    Ss, Us, Vts = [], [], []
    for (a, b) in tiles:
        p = prep(a, b)
        Ss.append(S.copy())
        U = v[a:b] - p["Kg"] @ S
        Vt = p["T"] @ (beta[a:b, None] * U)
        Us.append(U)
        Vts.append(Vt)
        S = p["GL"][:, None] * S + p["Kt"].T @ Vt
    # pass 2: state gradients leaving each tile, dY
    dS = dST.copy()
    dSs, dYs = [None] * nt, [None] * nt
    for j in reversed(range(nt)):
        a, b = tiles[j]
        p = prep(a, b)
        dSs[j] = dS.copy()
        dVt = p["Kt"] @ dS + p["Aqk"].T @ do[a:b]
        dY = p["T"].T @ dVt
        dYs[j] = dY
        dS = p["GL"][:, None] * dS + p["Qg"].T @ do[a:b] - p["Kg"].T @ (beta[a:b, None] * dY)
    dS0 = dS
    # pass 3: per-tile gradients
    dq, dk, dg = np.zeros_like(q), np.zeros_like(k), np.zeros_like(g)
    dv, dbeta = np.zeros_like(v), np.zeros_like(beta)
    for j, (a, b) in enumerate(tiles):
        p = prep(a, b)
        L = b - a
        Sj, dSp, U, Vt, dY = Ss[j], dSs[j], Us[j], Vts[j], dYs[j]
        bt = beta[a:b]
        dO = do[a:b]
        dQg = dO @ Sj.T
        dKg = -(bt[:, None] * dY) @ Sj.T
        dKt = Vt @ dSp.T
        dGL = np.sum(dSp * Sj, axis=1)
        dAqk = np.tril(dO @ Vt.T)
        dA = -np.tril(dY @ Vt.T, -1)
        dbeta[a:b] = np.sum(dY * U, axis=1) + np.sum(dA * p["At"], axis=1)
        dv[a:b] = bt[:, None] * dY
        dAt = bt[:, None] * dA
        # the diagonal Aqk[t, t] = scale q_t . k_t has no decay factor: its
        # gradient goes to q and k directly and never enters dG
        dAd = np.diag(dAqk).copy()
        dAqk = np.tril(dAqk, -1)
        dQl = dAqk @ p["Kd"]
        dKl = dAt @ p["Kd"]
        dKd = dAqk.T @ p["Ql"] + dAt.T @ p["Kl"]
        G, rho = p["G"], p["rho"]
        dq[a:b] = scale * (dQg * p["Gam"] + dQl * np.exp(G - rho) + dAd[:, None] * k[a:b])
        dk[a:b] = (dKg * p["Gam"] + dKt * np.exp(G[L - 1] - G) + dKl * np.exp(G - rho)
                   + dKd * np.exp(rho - G) + dAd[:, None] * scale * q[a:b])
        dG = (dQg * p["Qg"] + dKg * p["Kg"] - dKt * p["Kt"] + dQl * p["Ql"] + dKl * p["Kl"]
              - dKd * p["Kd"])
        dG[L - 1] += np.sum(dKt * p["Kt"], axis=0) + dGL * p["GL"]
        dg[a:b] = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dg, dbeta, dS0
