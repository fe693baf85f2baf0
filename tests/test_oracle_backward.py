"""Pins of the fp64 backward oracle (gradients of the KDA recurrence and of
the gate) against what the mathematics fixes.

Sources, cited by page title and section:
  [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华": section "Kimi Delta
             Attention" (KDA equation), section "Chunkwise parallel form"
             (new-gate equation). The pages give no backward pass; what is
             pinned here is that the oracle's gradients are the derivatives
             of the (separately pinned) forward oracle.

Pins:
  * central finite differences of the forward oracle, for every element of
    every input (q, k, v, g, beta, initial state), on a varlen batch with an
    empty sequence and a non-unit output scale;
  * Euler's identity for functions linear in their argument: o and the final
    state are jointly linear in (v, initial state), and o is linear in q;
  * one-token closed forms of dv, dbeta, dq and the initial-state gradient;
  * zero cotangents give zero gradients; an empty sequence passes the
    final-state gradient straight through;
  * gate: finite differences of the forward gate, and the closed form at
    z = 0 (sigmoid' = 1/4);
  * planted mistakes in a copy of the oracle's C source each fail the
    finite-difference pin.
"""
import subprocess

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle_backward, oracle_gate, oracle_gate_backward, oracle_recurrence
from oracle.oracle import _SRC

CU = np.array([0, 4, 4, 7], dtype=np.int32)   # lengths 4, 0, 3


def _problem(rng, T, H, Dk, Dv, N):
    q = rng.standard_normal((1, T, H, Dk))
    k = rng.standard_normal((1, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, Dv))
    g = -5.0 * expit(rng.standard_normal((1, T, H, Dk)))
    beta = expit(rng.standard_normal((1, T, H)))
    h0 = rng.standard_normal((N, H, Dk, Dv))
    do = rng.standard_normal((1, T, H, Dv))
    dhT = rng.standard_normal((N, H, Dk, Dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), do, dhT


def _loss(x, do, dhT, cu, scale, lib_path=None):
    o, hT = oracle_recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu, scale,
                              nthreads=1, lib_path=lib_path)
    return float(np.sum(o * do) + np.sum(hT * dhT))


def _fd_grads(x, do, dhT, cu, scale, eps=1e-5):
    fd = {}
    for name, arr in x.items():
        grad = np.zeros_like(arr)
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(x, do, dhT, cu, scale)
            flat[i] = keep - eps
            lm = _loss(x, do, dhT, cu, scale)
            flat[i] = keep
            gflat[i] = (lp - lm) / (2 * eps)
        fd[name] = grad
    return fd


_NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}


def _fd_mismatch(got, fd):
    """Worst relative disagreement over all inputs."""
    worst = 0.0
    for name, ref in fd.items():
        err = np.max(np.abs(got[_NAMES[name]] - ref)) / max(1.0, np.max(np.abs(ref)))
        worst = max(worst, err)
    return worst


def _fd_case():
    rng = np.random.default_rng(7)
    x, do, dhT = _problem(rng, int(CU[-1]), 2, 3, 2, len(CU) - 1)
    return x, do, dhT, 0.7


def test_backward_matches_finite_differences():
    x, do, dhT, scale = _fd_case()
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, CU, scale,
                          nthreads=1)
    fd = _fd_grads(x, do, dhT, CU, scale)
    assert _fd_mismatch(got, fd) < 1e-7


def test_backward_linear_identities():
    """o and hT are linear in (v, h0) jointly, so for L = <do, o> + <dhT, hT>
    Euler's identity gives <dv, v> + <dh0, h0> = L; o is linear in q and hT
    does not depend on q, so <dq, q> = <do, o>."""
    rng = np.random.default_rng(8)
    cu = np.array([0, 50, 50, 81], dtype=np.int32)
    x, do, dhT = _problem(rng, 81, 2, 16, 8, 3)
    o, hT = oracle_recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu, 1.3)
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, cu, 1.3)
    L = np.sum(o * do) + np.sum(hT * dhT)
    lhs = np.sum(got["dv"] * x["v"]) + np.sum(got["dh0"] * x["h0"])
    assert abs(lhs - L) <= 1e-10 * max(1.0, abs(L))
    assert abs(np.sum(got["dq"] * x["q"]) - np.sum(o * do)) <= 1e-10 * max(1.0, abs(L))


def test_backward_one_token_closed_forms():
    """One token from state S0: Sb = Diag(e^g) S0, u = Sb^T k,
    d = beta (v - u), S1 = Sb + k d^T, o = s S1^T q. With G = dhT + s q do^T
    (the total gradient on S1): dv = beta G^T k, dbeta = (G^T k).(v - u),
    dq = s S1 do and dS0 = Diag(e^g) (I - beta k k^T) G (the map
    S -> (I - beta k k^T) S is symmetric, so it is its own adjoint)."""
    rng = np.random.default_rng(9)
    Dk, Dv, s = 5, 4, 0.6
    cu = np.array([0, 1], dtype=np.int32)
    x, do, dhT = _problem(rng, 1, 1, Dk, Dv, 1)
    q, k, v, g = (x[n][0, 0, 0] for n in ("q", "k", "v", "g"))
    b = x["beta"][0, 0, 0]
    S0, dS1 = x["h0"][0, 0], dhT[0, 0]
    Sb = np.exp(g)[:, None] * S0
    u = Sb.T @ k
    S1 = Sb + np.outer(k, b * (v - u))
    G = dS1 + s * np.outer(q, do[0, 0, 0])
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, cu, s)
    np.testing.assert_allclose(got["dv"][0, 0, 0], b * (G.T @ k), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dbeta"][0, 0, 0], (G.T @ k) @ (v - u), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dq"][0, 0, 0], s * S1 @ do[0, 0, 0], rtol=1e-12, atol=1e-12)
    ref_dS0 = np.exp(g)[:, None] * ((np.eye(Dk) - b * np.outer(k, k)) @ G)
    np.testing.assert_allclose(got["dh0"][0, 0], ref_dS0, rtol=1e-12, atol=1e-12)


def test_backward_pure_decay_closed_forms():
    """beta = 0 on every token [KDA-blog §Kimi Delta Attention, KDA
    equation]: nothing is written, S_t = Diag(e^{G_t}) S0 with G_t the
    inclusive cumulative log-decay, o_t = s S_t^T q_t. Then, with
    Gtot_t = sum_{t' >= t} Diag(e^{G_t' - G_t}) s q_t' do_t'^T
    + Diag(e^{G_T - G_t}) dhT the total gradient on S_t:
    dq_t = s S_t do_t, dk = dv = 0,
    dS0 = sum_t Diag(e^{G_t}) s q_t do_t^T + Diag(e^{G_T}) dhT,
    dg_tau = sum_{t >= tau} dL/dG_t with
    dL/dG_t[c] = e^{G_t[c]} S0[c,:] . (s q_t[c] do_t + [t = T] dhT[c,:]),
    and dbeta_t = (Gtot_t^T k_t) . (v_t - S_t^T k_t), the derivative of the
    write term beta_t k_t (v_t - S^T k_t)^T at beta = 0, over 37 tokens."""
    rng = np.random.default_rng(11)
    T, Dk, Dv, s = 37, 6, 5, 0.7
    cu = np.array([0, T], dtype=np.int32)
    x, do, dhT = _problem(rng, T, 1, Dk, Dv, 1)
    x["beta"][:] = 0.0
    q, k, v, g = (x[n][0, :, 0] for n in ("q", "k", "v", "g"))
    dO, S0, dST = do[0, :, 0], x["h0"][0, 0], dhT[0, 0]
    G = np.cumsum(g, axis=0)                        # [T, Dk], inclusive
    E = np.exp(G)
    S = E[:, :, None] * S0[None]                    # S_t, [T, Dk, Dv]
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, cu, s)
    np.testing.assert_allclose(got["dq"][0, :, 0], s * np.einsum("tcv,tv->tc", S, dO),
                               rtol=1e-12, atol=1e-12)
    assert not np.any(got["dk"]) and not np.any(got["dv"])
    dS0 = s * np.einsum("tc,tc,tv->cv", E, q, dO) + E[-1][:, None] * dST
    np.testing.assert_allclose(got["dh0"][0, 0], dS0, rtol=1e-12, atol=1e-12)
    dG = s * q * E * np.einsum("cv,tv->tc", S0, dO)
    dG[-1] += E[-1] * np.sum(S0 * dST, axis=1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    np.testing.assert_allclose(got["dg"][0, :, 0], dg, rtol=1e-11, atol=1e-12)
    dbeta = np.empty(T)
    for t in range(T):
        R = np.exp(G[t:] - G[t])                    # e^{G_t' - G_t}, [T - t, Dk]
        Gtot = s * np.einsum("uc,uc,uv->cv", R, q[t:], dO[t:]) + R[-1][:, None] * dST
        dbeta[t] = (Gtot.T @ k[t]) @ (v[t] - S[t].T @ k[t])
    np.testing.assert_allclose(got["dbeta"][0, :, 0], dbeta, rtol=1e-11, atol=1e-12)


def test_backward_zero_cotangent_and_empty_sequence():
    rng = np.random.default_rng(10)
    x, do, dhT = _problem(rng, int(CU[-1]), 2, 4, 3, 3)
    zero = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], np.zeros_like(do), x["h0"],
                           None, CU)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert not np.any(zero[name]), name
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, CU)
    assert np.array_equal(got["dh0"][1], dhT[1])     # sequence 1 is empty


def test_gate_backward_matches_finite_differences_and_closed_form():
    rng = np.random.default_rng(11)
    z = rng.standard_normal((2, 3, 4, 5)) * 3
    A = rng.standard_normal(4)
    dg = rng.standard_normal(z.shape)
    dz, dA = oracle_gate_backward(z, dg, A, -5.0)
    eps = 1e-6
    fd_z = (oracle_gate(z + eps, A, -5.0) - oracle_gate(z - eps, A, -5.0)) / (2 * eps) * dg
    np.testing.assert_allclose(dz, fd_z, rtol=1e-7, atol=1e-9)
    for h in range(4):
        Ap, Am = A.copy(), A.copy()
        Ap[h] += eps
        Am[h] -= eps
        fd = np.sum((oracle_gate(z, Ap, -5.0) - oracle_gate(z, Am, -5.0)) * dg) / (2 * eps)
        assert abs(dA[h] - fd) <= 1e-7 * max(1.0, abs(fd))
    # z = 0: sigmoid'(0) = 1/4, so dz = dg g_min e^A / 4 and dA = 0
    z0 = np.zeros((1, 1, 2, 3))
    dg0 = np.ones_like(z0)
    dz0, dA0 = oracle_gate_backward(z0, dg0, np.array([0.0, np.log(2.0)]), -5.0)
    np.testing.assert_allclose(dz0[0, 0, 0], -1.25, rtol=1e-15)
    np.testing.assert_allclose(dz0[0, 0, 1], -2.5, rtol=1e-15)
    assert not np.any(dA0)
    dz_none, dA_none = oracle_gate_backward(z0, dg0, None, -5.0)
    np.testing.assert_allclose(dz_none, -1.25, rtol=1e-15)
    assert dA_none is None


MUTANTS = [
    # drop the write-back path of u = Sb^T k into the state gradient
    ("dS[i * Dv + j] += kt[i] * dd[j];", "(void)0;"),
    # forget that d carries beta: dv = dd
    ("dvt[j] = bt * dd[j];", "dvt[j] = dd[j];"),
    # decay gradient against the undecayed state
    ("acc += dS[i * Dv + j] * Sb[i * Dv + j];", "acc += dS[i * Dv + j] * Sp[i * Dv + j];"),
    # read o before the write instead of after it
    ("acc += S[i * Dv + j] * dot[j];", "acc += Sp[i * Dv + j] * dot[j];"),
]


@pytest.mark.parametrize("old,new", MUTANTS, ids=["no-dS-from-u", "dv-no-beta", "dg-undecayed",
                                                   "dq-old-state"])
def test_planted_mistakes_fail_the_pin(tmp_path, old, new):
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=gnu99", "-shared", "-fPIC", str(path), "-o", lib, "-lm",
                    "-lpthread"], check=True)
    x, do, dhT, scale = _fd_case()
    got = oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["h0"], dhT, CU, scale,
                          nthreads=1, lib_path=lib)
    fd = _fd_grads(x, do, dhT, CU, scale)   # from the unmodified forward
    assert _fd_mismatch(got, fd) > 1e-3


@pytest.mark.parametrize("betas", ["sigmoid", "zeros"])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 50])
def test_tile_arrangement_matches_oracle(T, betas):
    """The 16-token tile arrangement the GPU backward uses (forward scan for
    U and V~, reverse scan for dY and the state gradients, then per-tile
    gradients through the decay factors), written in fp64 numpy, gives the
    oracle's gradients to rounding; with "zeros" some beta are 0 or 1e-35
    (tokens that write nothing, whose beta gradient is still nonzero)."""
    from tests.chunk_mirror import tile_backward
    rng = np.random.default_rng(12 + T)
    Dk, Dv = 8, 6
    q = rng.standard_normal((T, Dk))
    k = rng.standard_normal((T, Dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, Dv))
    g = -5.0 * expit(rng.standard_normal((T, Dk)))
    beta = expit(rng.standard_normal(T))
    if betas == "zeros":
        beta[::3] = 0.0
        beta[1::5] = 1e-35
    S0, dST = rng.standard_normal((Dk, Dv)), rng.standard_normal((Dk, Dv))
    do = rng.standard_normal((T, Dv))
    got = tile_backward(q, k, v, g, beta, S0, do, dST, scale=0.8)
    e = lambda x: x[None, :, None]  # noqa: E731
    ref = oracle_backward(e(q), e(k), e(v), e(g), e(beta), e(do), S0[None, None], dST[None, None],
                          None, 0.8)
    for name, x in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got):
        r = ref[name].reshape(x.shape)
        assert np.max(np.abs(x - r)) <= 1e-12 * max(1.0, np.max(np.abs(r))), name
