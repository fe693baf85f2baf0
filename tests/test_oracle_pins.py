"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Sources, cited by page title and section:
  [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华": section "Kimi Delta
             Attention" (KDA equation; delta-rule equation: the written value
             replaces the old one with weight beta), section "Chunkwise
             parallel form" (gamma, W/U, pseudo-value and A/O equations; the
             statement that the chunk form equals the token recurrence
             exactly; the new-gate equation and its range (g_min, 0)).
  [Baidu-1]  "Kimi K3 Core Techniques Explained ...", §1.2 (g_min = -5).

None of these pins retypes the oracle's loop: each checks a closed form, an
invariant, a hand-worked example, a library routine or an independently
written brute force.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle_cumsum, oracle_gate, oracle_recurrence
from tests.chunk_mirror import chunk_form_pages, chunk_form_tiled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, B, T, H, Dk, Dv, g_min=-5.0, unit=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    beta = expit(rng.standard_normal((B, T, H)))
    g = g_min * expit(rng.standard_normal((B, T, H, Dk)))
    return q, k, v, g, beta


# ----------------------------------------------------------------- gate ---

def test_gate_closed_forms():
    """g = g_min sigmoid(e^A z) at points where sigmoid has a closed form."""
    spec = json.load(open(os.path.join(GOLDEN, "gate_closed_forms.json")))
    for case in spec["cases"]:
        z = np.full((1, 1, 1, 1), case["z"])
        A = np.array([case["A"]])
        g = oracle_gate(z, A, spec["g_min"])
        assert abs(g.item() - case["g"]) <= 1e-14 * abs(case["g"]), case


def test_gate_matches_library_sigmoid_and_range():
    """Agreement with scipy's expit in fp64; range [g_min, 0]; monotone in z."""
    rng = np.random.default_rng(0)
    z = rng.standard_normal((3, 5, 4, 16)) * 8
    A = rng.standard_normal(4)
    g = oracle_gate(z, A, -5.0)
    ref = -5.0 * expit(np.exp(A)[None, None, :, None] * z)
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-300)
    assert g.min() >= -5.0 and g.max() <= 0.0
    zs = np.sort(rng.standard_normal(1000) * 10).reshape(1, 1000, 1, 1)
    gs = oracle_gate(zs, None, -5.0).ravel()
    assert np.all(np.diff(gs) <= 0)          # decreasing in z (g_min < 0)
    lim = oracle_gate(np.array([40.0, -40.0, -800.0]).reshape(1, 3, 1, 1), None, -5.0).ravel()
    assert lim[0] == -5.0 and -1e-16 < lim[1] < 0 and lim[2] == 0.0


def test_softplus_gate_closed_forms_and_library():
    """The pages' earlier gate g = -e^{A_h} softplus(z): softplus(0) = ln 2,
    softplus(ln 3) = ln 4, equality with numpy's logaddexp(0, z), the
    asymptotes (z for z >> 0, e^z for z << 0), sign and monotonicity."""
    from oracle import oracle_gate_softplus
    z = np.array([[[0.0, np.log(3.0), 40.0, -40.0, 1e-8]]])
    g = oracle_gate_softplus(z)
    np.testing.assert_allclose(g[0, 0, :2], [-np.log(2.0), -np.log(4.0)], rtol=1e-15)
    np.testing.assert_allclose(g[0, 0, 2], -40.0, rtol=1e-15)
    np.testing.assert_allclose(g[0, 0, 3], -np.exp(-40.0), rtol=1e-12)
    gA = oracle_gate_softplus(z, np.array([np.log(2.0)]))
    np.testing.assert_allclose(gA, 2.0 * g, rtol=1e-15)
    rng = np.random.default_rng(9)
    zz = 10 * rng.standard_normal((3, 4, 2, 16))
    A = rng.standard_normal(2)
    np.testing.assert_allclose(oracle_gate_softplus(zz, A),
                               -np.exp(A)[:, None] * np.logaddexp(0.0, zz), rtol=1e-13)
    assert np.all(oracle_gate_softplus(zz, A) < 0)
    zs = np.sort(zz.reshape(-1))
    assert np.all(np.diff(oracle_gate_softplus(zs[None, None, :])[0, 0]) <= 0)


def test_cumsum_matches_numpy_per_chunk():
    """Inclusive chunk-local cumsum (gamma equation) == numpy.cumsum on every
    chunk segment, chunks restarting at each sequence start (ragged tails)."""
    rng = np.random.default_rng(1)
    lens = [1, 63, 64, 65, 130, 0, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = rng.standard_normal((1, cu[-1], 3, 8))
    out = oracle_cumsum(g, 64, cu)
    for n in range(len(lens)):
        for s in range(cu[n], cu[n + 1], 64):
            e = min(s + 64, cu[n + 1])
            np.testing.assert_allclose(out[0, s:e], np.cumsum(g[0, s:e], axis=0),
                                       rtol=1e-13, atol=1e-13)
    dense = oracle_cumsum(g[:, :192].reshape(2, 96, 3, 8), 32)
    for b in range(2):
        for s in range(0, 96, 32):
            np.testing.assert_allclose(dense[b, s:s + 32],
                                       np.cumsum(g[0, 96 * b + s:96 * b + s + 32], axis=0),
                                       rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------- recurrence ---

def test_hand_worked_example():
    """3 tokens, d = 2, worked by hand from the KDA equation."""
    spec = json.load(open(os.path.join(GOLDEN, "hand_worked_recurrence.json")))
    x = {key: np.array(val) for key, val in spec["inputs"].items()}
    q, k, v = (x[n][None, :, None, :] for n in ("q", "k", "v"))
    g = np.log(x["alpha"])[None, :, None, :]
    beta = x["beta"][None, :, None]
    o, S = oracle_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, :, 0], np.array(spec["expected"]["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], np.array(spec["expected"]["final_state"]), rtol=0,
                               atol=1e-14)


def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(exp(sum_{i<=t} g_i)) S_0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta = _rand_problem(rng, 2, 40, 3, 8, 6)
    beta[:] = 0.0
    S0 = rng.standard_normal((2, 3, 8, 6))
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    cum = np.cumsum(g, axis=1)                                 # [B,T,H,Dk]
    St = np.exp(cum)[..., None] * S0[:, None]                  # [B,T,H,Dk,Dv]
    o_ref = np.einsum("bthkv,bthk->bthv", St, q)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, St[:, -1], rtol=1e-12, atol=1e-14)
    o0, S0z = oracle_recurrence(q, k, v, g, beta)              # zero state stays zero
    assert np.all(o0 == 0) and np.all(S0z == 0)


def test_orthonormal_key_recall():
    """alpha = 1, beta = 1, orthonormal keys, S_0 = 0: S_t = sum_j k_j v_j^T,
    so querying k_j returns v_j for j <= t and 0 for j > t."""
    rng = np.random.default_rng(3)
    Dk, Dv, T = 16, 5, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:T]                                               # orthonormal rows
    v = rng.standard_normal((T, Dv))
    beta = np.ones((1, T, 1))
    g = np.zeros((1, T, 1, Dk))
    for j in range(T):
        q = np.tile(keys[j], (T, 1))[None, :, None, :]
        o, S = oracle_recurrence(q, keys[None, :, None, :], v[None, :, None, :], g, beta)
        for t in range(T):
            expect = v[j] if j <= t else np.zeros(Dv)
            np.testing.assert_allclose(o[0, t, 0], expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], keys.T @ v, rtol=0, atol=1e-12)


def test_overwrite_recalls_latest_value():
    """Delta rule with beta = 1 and a unit key written twice: the second write
    replaces the first, so the query returns the later value."""
    rng = np.random.default_rng(4)
    Dk, Dv = 8, 4
    kvec = rng.standard_normal(Dk); kvec /= np.linalg.norm(kvec)
    v1, v2 = rng.standard_normal(Dv), rng.standard_normal(Dv)
    k = np.stack([kvec, kvec])[None, :, None, :]
    v = np.stack([v1, v2])[None, :, None, :]
    q = k.copy()
    o, _ = oracle_recurrence(q, k, v, np.zeros((1, 2, 1, Dk)), np.ones((1, 2, 1)))
    np.testing.assert_allclose(o[0, 0, 0], v1, atol=1e-13)
    np.testing.assert_allclose(o[0, 1, 0], v2, atol=1e-13)


def _brute_force_unit(q, k, v, g, beta, S0):
    """Dense products: P_t = (I - b k k^T) Diag(alpha_t); S_T = P_T..P_1 S_0 +
    sum_j P_T..P_{j+1} b_j k_j v_j^T; o_t = S_t^T q_t. Written with explicit
    matrices and a fresh product for every t (no running state)."""
    T, Dk = q.shape
    I = np.eye(Dk)
    P = [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    outs, states = [], []
    for t in range(T):
        St = np.linalg.multi_dot([*P[t::-1], S0]) if t > 0 else P[0] @ S0
        for j in range(t + 1):
            prod = I
            for m in range(j + 1, t + 1):
                prod = P[m] @ prod
            St = St + prod @ (beta[j] * np.outer(k[j], v[j]))
        outs.append(St.T @ q[t])
        states.append(St)
    return np.array(outs), states[-1]


@pytest.mark.parametrize("T", [1, 2, 7, 16])
def test_brute_force_dense_products(T):
    rng = np.random.default_rng(10 + T)
    Dk, Dv, H = 6, 5, 2
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, Dk, Dv)
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    for h in range(H):
        o_ref, S_ref = _brute_force_unit(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                         beta[0, :, h], S0[0, h])
        scale = max(np.abs(o_ref).max(), 1.0)
        np.testing.assert_allclose(o[0, :, h], o_ref, rtol=0, atol=1e-12 * scale)
        np.testing.assert_allclose(S[0, h], S_ref, rtol=0, atol=1e-12 * max(np.abs(S_ref).max(), 1))


def test_linearity_in_values_and_state():
    """o and S_T are jointly linear in (V, S_0) for fixed q, k, g, beta."""
    rng = np.random.default_rng(5)
    q, k, v1, g, beta = _rand_problem(rng, 1, 50, 2, 8, 4)
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = rng.standard_normal((2, 1, 2, 8, 4))
    a, b = 0.7, -1.3
    o1, S1 = oracle_recurrence(q, k, v1, g, beta, s1)
    o2, S2 = oracle_recurrence(q, k, v2, g, beta, s2)
    o3, S3 = oracle_recurrence(q, k, a * v1 + b * v2, g, beta, a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + b * S2, rtol=1e-11, atol=1e-12)


def test_output_scale_is_a_plain_factor():
    rng = np.random.default_rng(55)
    q, k, v, g, beta = _rand_problem(rng, 1, 20, 1, 8, 4)
    o1, S1 = oracle_recurrence(q, k, v, g, beta)
    o2, S2 = oracle_recurrence(q, k, v, g, beta, scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(S1, S2)


def test_split_and_resume():
    """The run on [0, T) equals [T1, T) started from the final state of [0, T1)."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta = _rand_problem(rng, 1, 90, 2, 8, 6)
    S0 = rng.standard_normal((1, 2, 8, 6))
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    T1 = 37
    oa, Sa = oracle_recurrence(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    ob, Sb = oracle_recurrence(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-13)


def _state_map(k, g, beta):
    """Per head, the product of the per-token state maps
    (I - beta_t k_t k_t^T) Diag(e^{g_t}), latest token leftmost, written out
    directly (numpy, fp64) for one sequence. Returns [H, Dk, Dk]."""
    _, T, H, Dk = k.shape
    out = np.empty((H, Dk, Dk))
    for h in range(H):
        Mh = np.eye(Dk)
        for t in range(T):
            kt = k[0, t, h]
            step = (np.eye(Dk) - beta[0, t, h] * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, h]))
            Mh = step @ Mh
        out[h] = Mh
    return out


def test_state_map_is_affine_and_equals_the_product_of_token_maps():
    """S_T(S_0) = M S_0 + S_T(0), with M the product of the per-token maps;
    the run with v = 0 from S_0 = I yields M (what kda_chunk_transition
    computes)."""
    rng = np.random.default_rng(61)
    q, k, v, g, beta = _rand_problem(rng, 1, 23, 2, 6, 5)
    M = _state_map(k, g, beta)
    eye = np.broadcast_to(np.eye(6), (1, 2, 6, 6)).copy()
    _, M_run = oracle_recurrence(q, k, np.zeros((1, 23, 2, 6)), g, beta, eye)
    np.testing.assert_allclose(M_run[0], M, rtol=1e-12, atol=1e-13)
    S0 = rng.standard_normal((1, 2, 6, 5))
    _, S_from = oracle_recurrence(q, k, v, g, beta, S0)
    _, S_zero = oracle_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(S_from[0], np.einsum("hij,hjc->hic", M, S0[0]) + S_zero[0],
                               rtol=1e-12, atol=1e-13)


def test_segment_composition_equals_the_unsplit_run():
    """A sequence cut into segments: entry states chained from each segment's
    map and zero-start final state, then every segment re-run from its entry
    state, reproduce the unsplit outputs and final state."""
    rng = np.random.default_rng(62)
    T, H, Dk, Dv = 100, 2, 6, 5
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, Dk, Dv)
    S_init = rng.standard_normal((1, H, Dk, Dv))
    o_ref, S_ref = oracle_recurrence(q, k, v, g, beta, S_init)
    bounds = [0, 31, 32, 64, 100]   # includes a one-token segment
    start = S_init[0]
    outs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        sl = (slice(None), slice(a, b))
        eye = np.broadcast_to(np.eye(Dk), (1, H, Dk, Dk)).copy()
        _, M = oracle_recurrence(q[sl], k[sl], np.zeros((1, b - a, H, Dk)), g[sl], beta[sl], eye)
        _, b0 = oracle_recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl])
        o_seg, _ = oracle_recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], start[None])
        outs.append(o_seg)
        start = np.einsum("hij,hjc->hic", M[0], start) + b0[0]
    np.testing.assert_allclose(np.concatenate(outs, axis=1), o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(start, S_ref[0], rtol=1e-11, atol=1e-12)


def test_varlen_equals_independent_runs():
    """Packed sequences with cu_seqlens == independent per-sequence runs
    (bit-for-bit), including an empty sequence (final = initial)."""
    rng = np.random.default_rng(7)
    lens = [5, 0, 33, 64, 17]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta = _rand_problem(rng, 1, int(cu[-1]), 3, 8, 4)
    h0 = rng.standard_normal((len(lens), 3, 8, 4))
    o, S = oracle_recurrence(q, k, v, g, beta, h0, cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = oracle_recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl],
                                   h0[n:n + 1])
        np.testing.assert_array_equal(o[:, sl], on)
        np.testing.assert_array_equal(S[n], Sn[0])
    np.testing.assert_array_equal(S[1], h0[1])


def test_value_column_separability():
    """o[:, J] and S_T[:, J] depend only on v[:, J] and S_0[:, J]."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta = _rand_problem(rng, 1, 70, 2, 8, 6)
    S0 = rng.standard_normal((1, 2, 8, 6))
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    J = [1, 4]
    oj, Sj = oracle_recurrence(q, k, v[..., J], g, beta, S0[..., J])
    np.testing.assert_array_equal(oj, o[..., J])
    np.testing.assert_array_equal(Sj, S[..., J])


def test_state_norm_bound():
    """With |k| = 1, beta in [0, 1] and alpha <= 1, (I - b k k^T) Diag(alpha)
    has spectral norm <= 1, so |S_t|_2 <= |S_0|_2 + sum_{i<=t} beta_i |v_i|."""
    rng = np.random.default_rng(9)
    T = 60
    q, k, v, g, beta = _rand_problem(rng, 1, T, 1, 8, 8)
    S0 = rng.standard_normal((1, 1, 8, 8))
    bound = np.linalg.norm(S0[0, 0], 2)
    for t in range(1, T + 1):
        _, S = oracle_recurrence(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0)
        bound += beta[0, t - 1, 0] * np.linalg.norm(v[0, t - 1, 0])
        assert np.linalg.norm(S[0, 0], 2) <= bound * (1 + 1e-12)


# -------------------------------------------------- chunk-form equivalence ---

@pytest.mark.parametrize("C,T", [(16, 48), (32, 77), (64, 64), (64, 200), (64, 1)])
def test_chunk_form_of_the_pages_equals_recurrence(C, T):
    """The page states the chunkwise form equals the token recurrence exactly;
    the W/U, pseudo-value and A/O equations (with the derived M and state
    hand-off) must reproduce the oracle to fp64 rounding."""
    rng = np.random.default_rng(100 + C + T)
    q, k, v, g, beta = _rand_problem(rng, 1, T, 1, 16, 12)
    S0 = rng.standard_normal((1, 1, 16, 12)) * 0.1
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    oc, Sc = chunk_form_pages(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                              S0[0, 0], C)
    assert np.abs(oc - o[0, :, 0]).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(Sc - S[0, 0]).max() <= 1e-12 * np.abs(S).max()


@pytest.mark.parametrize("T,gconst", [(200, None), (64, -5.0), (130, 0.0), (17, None)])
def test_tiled_arrangement_equals_recurrence(T, gconst):
    """The GPU arrangement (16-token tiles, reference points, block forward
    substitution, factored exponentials) in fp64 == oracle, including the
    extreme gate g = g_min everywhere (largest in-tile reciprocal e^{80})."""
    rng = np.random.default_rng(200 + T)
    q, k, v, g, beta = _rand_problem(rng, 1, T, 1, 32, 16)
    if gconst is not None:
        g[:] = gconst
    S0 = rng.standard_normal((1, 1, 32, 16)) * 0.1
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    ot, St = chunk_form_tiled(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                              S0[0, 0])
    assert np.abs(ot - o[0, :, 0]).max() <= 1e-11 * np.abs(o).max()
    assert np.abs(St - S[0, 0]).max() <= 1e-11 * np.abs(S).max()


@pytest.mark.parametrize("gconst", [None, -5.0])
def test_bf16_rounding_budget(gconst):
    """bf16 rounding at every operand the kernel rounds keeps max|d|/max|ref|
    well inside the 2e-2 budget (prediction for the GPU bf16 path)."""
    rng = np.random.default_rng(300)
    T, D = 512, 128
    q, k, v, g, beta = _rand_problem(rng, 1, T, 1, D, D)
    if gconst is not None:
        g[:] = gconst
    from tests.chunk_mirror import bf16_round
    q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    S0 = rng.standard_normal((1, 1, D, D)) * 0.02
    o, S = oracle_recurrence(q, k, v, g, beta, S0)
    ot, St = chunk_form_tiled(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                              S0[0, 0], round_bf16=True)
    err_o = np.abs(ot - o[0, :, 0]).max() / np.abs(o).max()
    err_s = np.abs(St - S[0, 0]).max() / np.abs(S).max()
    assert err_o < 5e-3 and err_s < 5e-3, (err_o, err_s)
