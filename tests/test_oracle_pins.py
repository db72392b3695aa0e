"""Pins for the fp64 oracle: checks against things other than the oracle itself.

* a hand-worked two-token example (tests/golden/hand_k2v2_t2.json);
* brute force in exact rational arithmetic from the unrolled product form of
  the recurrence (transition matrices multiplied out), on tiny shapes with
  K != V so that any transposition shows;
* closed forms: one token, beta = 0, strong decay, orthonormal-key
  retrieval, K = V = 1;
* an independent fp64 chunked WY evaluation (triangular solve per chunk);
* invariants: split-call continuity, varlen = separate calls, grouped heads =
  repeated heads, V-column independence;
* mutation checks: deliberately broken copies of the oracle's C source must
  fail at least one of the pins above.

The recurrence is the Gated DeltaNet rule S_t = exp(g_t) S_{t-1}(I - beta_t k_t
k_t^T) + beta_t v_t k_t^T, o_t = scale S_t q_t (the layer the FlashQLA pages
optimise; agentlenshq.com blog "GDN chunked-prefill optimisation"; gates in
(0,1) per its "AutoCP" section).  States are stored as S^T, [K, V].
"""
import json
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(a):
    return np.asarray(a, dtype=np.float32)


def rand_case(rng, B, T, Hqk, Hv, K, V, g_scale=0.5, unit=True, h0=True, N=None):
    q = f32(rng.standard_normal((B, T, Hqk, K)))
    k = f32(rng.standard_normal((B, T, Hqk, K)))
    if unit:
        q = f32(q / np.linalg.norm(q, axis=-1, keepdims=True))
        k = f32(k / np.linalg.norm(k, axis=-1, keepdims=True))
    v = f32(rng.standard_normal((B, T, Hv, V)))
    g = f32(-g_scale * rng.random((B, T, Hv)))
    beta = f32(rng.random((B, T, Hv)))
    N = B if N is None else N
    s0 = f32(0.3 * rng.standard_normal((N, Hv, K, V))) if h0 else None
    return q, k, v, g, beta, s0


# ---------------------------------------------------------------- golden

def test_hand_worked_example():
    d = json.load(open(os.path.join(HERE, "golden", "hand_k2v2_t2.json")))
    q = np.array(d["q_rows"])[None, :, None, :]
    k = np.array(d["k_rows"])[None, :, None, :]
    v = np.array(d["v_rows"])[None, :, None, :]
    g = np.array(d["g"])[None, :, None]
    b = np.array(d["beta"])[None, :, None]
    h0 = np.array(d["initial_state"])[None, None]
    o, ht = oracle.fwd(q, k, v, g, b, scale=d["scale"], initial_state=h0)
    np.testing.assert_array_equal(o[0, :, 0], np.array(d["expected_o"]))
    np.testing.assert_array_equal(ht[0, 0], np.array(d["expected_final_state"]))


# ---------------------------------------------------------------- brute force

def _frac_mat(a):
    return [[Fraction(float(x)) for x in row] for row in a]


def _mm(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][t] * B[t][j] for t in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _brute_force_head(q, k, v, g, beta, scale, S0):
    """Unrolled product form in exact rationals, one (sequence, v-head):
    S_t = S_0 M_1..M_t + sum_{s<=t} beta_s v_s k_s^T M_{s+1}..M_t,
    M_s = a_s (I - beta_s k_s k_s^T), a_s = exp(g_s) (taken as its double value).
    Returns o [T, V] and S_T^T [K, V] as floats."""
    T, K = k.shape
    V = v.shape[1]
    eye = [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]
    Ms = []
    for t in range(T):
        a = Fraction(math.exp(float(g[t])))
        b = Fraction(float(beta[t]))
        kk = [Fraction(float(x)) for x in k[t]]
        Ms.append([[a * (eye[i][j] - b * kk[i] * kk[j]) for j in range(K)] for i in range(K)])
    S0f = _frac_mat(S0)  # V x K
    outs = []
    S_T = None
    for t in range(T):
        # S0 M_1..M_t
        acc = S0f
        for s in range(t + 1):
            acc = _mm(acc, Ms[s])
        total = [row[:] for row in acc]
        for s in range(t + 1):
            b = Fraction(float(beta[s]))
            term = [[b * Fraction(float(v[s][i])) * Fraction(float(k[s][j])) for j in range(K)] for i in range(V)]
            for r in range(s + 1, t + 1):
                term = _mm(term, Ms[r])
            total = [[total[i][j] + term[i][j] for j in range(K)] for i in range(V)]
        qq = [Fraction(float(x)) for x in q[t]]
        sc = Fraction(float(scale))
        outs.append([float(sc * sum((total[i][j] * qq[j] for j in range(K)), Fraction(0))) for i in range(V)])
        S_T = total
    return np.array(outs), np.array([[float(S_T[i][j]) for i in range(V)] for j in range(K)])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_exact_rational(seed):
    rng = np.random.default_rng(seed)
    B, T, Hqk, Hv, K, V = 1, 5, 1, 2, 3, 4
    q, k, v, g, beta, s0 = rand_case(rng, B, T, Hqk, Hv, K, V, g_scale=0.7, unit=False)
    beta = f32(1.5 * beta)  # beta up to 1.5 exercises the (I - beta k k^T) term harder
    scale = 0.75
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0)
    for j in range(Hv):
        ob, Sb = _brute_force_head(q[0, :, 0], k[0, :, 0], v[0, :, j], g[0, :, j], beta[0, :, j], scale,
                                   s0[0, j].T)
        np.testing.assert_allclose(o[0, :, j], ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[0, j], Sb, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_single_token_closed_form():
    rng = np.random.default_rng(5)
    q, k, v, g, beta, _ = rand_case(rng, 1, 1, 1, 1, 8, 6, h0=False)
    scale = 0.3
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale)
    b = float(beta[0, 0, 0])
    kk, vv, qq = k[0, 0, 0].astype(np.float64), v[0, 0, 0].astype(np.float64), q[0, 0, 0].astype(np.float64)
    # S = beta v k^T  ->  stored S^T = beta k v^T ;  o = scale beta (k.q) v
    np.testing.assert_allclose(ht[0, 0], b * np.outer(kk, vv), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], scale * b * np.dot(kk, qq) * vv, rtol=1e-13, atol=1e-15)


def test_beta_zero_closed_form():
    rng = np.random.default_rng(6)
    T, K, V = 37, 8, 5
    q, k, v, g, beta, s0 = rand_case(rng, 1, T, 1, 1, K, V)
    beta = np.zeros_like(beta)
    scale = 0.5
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0)
    G = np.cumsum(g[0, :, 0].astype(np.float64))
    H0 = s0[0, 0].astype(np.float64)
    np.testing.assert_allclose(ht[0, 0], math.exp(G[-1]) * H0, rtol=1e-12)
    expect = scale * np.exp(G)[:, None] * (q[0, :, 0].astype(np.float64) @ H0)
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-11, atol=1e-15)


def test_strong_decay_forgets_state():
    rng = np.random.default_rng(7)
    T, K, V = 20, 8, 8
    q, k, v, g, beta, s0 = rand_case(rng, 1, T, 1, 1, K, V)
    g = np.full_like(g, -50.0)
    s0 = f32(100.0 * s0)
    scale = 1.0
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0)
    kk, vv, qq = (x[0, :, 0].astype(np.float64) for x in (k, v, q))
    bb = beta[0, :, 0].astype(np.float64)
    np.testing.assert_allclose(ht[0, 0], bb[-1] * np.outer(kk[-1], vv[-1]), rtol=1e-12, atol=1e-18)
    expect = (bb * np.sum(kk * qq, axis=1))[:, None] * vv
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-12, atol=1e-18)


def test_orthonormal_key_retrieval():
    rng = np.random.default_rng(8)
    K = V = 8
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = f32(Q.T)[None, :, None, :]  # token t uses key = row t of an orthonormal basis
    # float32 rounding breaks exact orthonormality slightly; the closed form holds to ~1e-6
    q = f32(rng.standard_normal((1, K, 1, K)))
    v = f32(rng.standard_normal((1, K, 1, V)))
    g = np.zeros((1, K, 1), np.float32)
    beta = np.ones((1, K, 1), np.float32)
    s0 = f32(rng.standard_normal((1, 1, K, V)))
    o, ht = oracle.fwd(q, k, v, g, beta, scale=1.0, initial_state=s0)
    H = ht[0, 0]  # S^T ; S k_j = H^T k_j
    for j in range(K):
        np.testing.assert_allclose(H.T @ k[0, j, 0].astype(np.float64), v[0, j, 0], atol=5e-6)


def test_scalar_recurrence():
    rng = np.random.default_rng(9)
    T = 50
    q, k, v, g, beta, s0 = rand_case(rng, 1, T, 1, 1, 1, 1, unit=False)
    scale = 1.25
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0)
    s = float(s0[0, 0, 0, 0])
    for t in range(T):
        a = math.exp(float(g[0, t, 0]))
        b = float(beta[0, t, 0])
        kt = float(k[0, t, 0, 0])
        s = a * (1.0 - b * kt * kt) * s + b * float(v[0, t, 0, 0]) * kt
        assert o[0, t, 0, 0] == pytest.approx(scale * s * float(q[0, t, 0, 0]), rel=1e-12, abs=1e-15)
    assert ht[0, 0, 0, 0] == pytest.approx(s, rel=1e-12)


# ---------------------------------------------------------------- independent chunked form

def chunked_wy(q, k, v, g, beta, scale, s0, C, cu=None):
    """fp64 chunked WY evaluation, written independently of the oracle: per chunk,
    A = strict-lower(beta_i e^{G_i-G_s} k_i.k_s), T = (I + A)^-1 by triangular
    solve, W = T diag(beta e^G) K, U = T diag(beta) V, v' = U - W H,
    O = scale (diag(e^G) Q H + causal(e^{G_i-G_s} q_i.k_s) v'),
    H <- e^{G_last} H + (diag(e^{G_last - G}) K)^T v'."""
    B, Tn, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    if cu is None:
        seqs = [(b, 0, Tn) for b in range(B)]
    else:
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, Tn, Hv, V))
    ht = np.zeros((len(seqs), Hv, K, V))
    for n, (b, t0, t1) in enumerate(seqs):
        for j in range(Hv):
            i = j // grp
            H = np.zeros((K, V)) if s0 is None else s0[n, j].astype(np.float64)
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                Q = q[b, c0:c1, i].astype(np.float64)
                Kc = k[b, c0:c1, i].astype(np.float64)
                Vc = v[b, c0:c1, j].astype(np.float64)
                bt = beta[b, c0:c1, j].astype(np.float64)
                G = np.cumsum(g[b, c0:c1, j].astype(np.float64))
                D = G[:, None] - G[None, :]
                Dm = np.where(np.tril(np.ones_like(D)) > 0, D, -np.inf)
                A = np.tril(bt[:, None] * np.exp(Dm) * (Kc @ Kc.T), -1)
                L = np.eye(len(G)) + A
                W = solve_triangular(L, (bt * np.exp(G))[:, None] * Kc, lower=True, unit_diagonal=True)
                U = solve_triangular(L, bt[:, None] * Vc, lower=True, unit_diagonal=True)
                vp = U - W @ H
                P = np.exp(Dm) * (Q @ Kc.T)
                o[b, c0:c1, j] = scale * (np.exp(G)[:, None] * (Q @ H) + P @ vp)
                H = np.exp(G[-1]) * H + (np.exp(G[-1] - G)[:, None] * Kc).T @ vp
            ht[n, j] = H
    return o, ht


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_wy_cross_form(C):
    rng = np.random.default_rng(10 + C)
    B, T, Hqk, Hv, K, V = 2, 150, 2, 4, 16, 12
    q, k, v, g, beta, s0 = rand_case(rng, B, T, Hqk, Hv, K, V, g_scale=0.4)
    scale = K ** -0.5
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0)
    oc, hc = chunked_wy(q, k, v, g, beta, scale, s0, C)
    np.testing.assert_allclose(o, oc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ht, hc, rtol=1e-10, atol=1e-12)


def test_chunked_wy_cross_form_varlen():
    rng = np.random.default_rng(20)
    lens = [70, 0, 1, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, g, beta, s0 = rand_case(rng, 1, T, 1, 3, 16, 8, N=len(lens))
    o, ht = oracle.fwd(q, k, v, g, beta, scale=0.25, initial_state=s0, cu_seqlens=cu)
    oc, hc = chunked_wy(q, k, v, g, beta, 0.25, s0, 64, cu=cu)
    np.testing.assert_allclose(o, oc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ht, hc, rtol=1e-10, atol=1e-12)
    # the empty sequence hands its initial state straight through
    np.testing.assert_array_equal(ht[1], s0[1].astype(np.float64))


# ---------------------------------------------------------------- invariants

def test_split_call_continuity():
    rng = np.random.default_rng(30)
    q, k, v, g, beta, s0 = rand_case(rng, 1, 90, 1, 2, 8, 8)
    o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0)
    T1 = 37
    o1, h1 = oracle.fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], scale=0.5, initial_state=s0)
    o2, h2 = oracle.fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], scale=0.5,
                        initial_state=h1.astype(np.float32))
    # the handed-over state is rounded to float32, so agreement is to float32 precision
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=2e-5, atol=2e-6)
    np.testing.assert_allclose(h2, ht, rtol=2e-5, atol=2e-6)
    np.testing.assert_array_equal(o1, o[:, :T1])


def test_varlen_equals_separate_calls():
    rng = np.random.default_rng(31)
    lens = [33, 64, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, s0 = rand_case(rng, 1, int(cu[-1]), 2, 4, 8, 6, N=len(lens))
    o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        on, hn = oracle.fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], scale=0.5,
                            initial_state=s0[n:n + 1])
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(ht[n:n + 1], hn)


def test_grouped_heads_equal_repeated_heads():
    rng = np.random.default_rng(32)
    q, k, v, g, beta, s0 = rand_case(rng, 2, 40, 2, 6, 8, 4)
    o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0)
    qr = np.repeat(q, 3, axis=2)  # v-head j <- qk-head j // 3
    kr = np.repeat(k, 3, axis=2)
    o2, ht2 = oracle.fwd(qr, kr, v, g, beta, scale=0.5, initial_state=s0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ht, ht2)


def test_v_column_independence():
    rng = np.random.default_rng(33)
    q, k, v, g, beta, s0 = rand_case(rng, 1, 50, 1, 1, 8, 10)
    o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0)
    cols = [1, 4, 7]
    o2, ht2 = oracle.fwd(q, k, v[..., cols], g, beta, scale=0.5, initial_state=s0[..., cols])
    np.testing.assert_allclose(o2, o[..., cols], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(ht2, ht[..., cols], rtol=1e-14, atol=1e-16)


def test_state_norm_bound():
    """For unit keys and beta in [0, 2] the bracket (I - beta k k^T) has 2-norm <= 1,
    so ||H_t|| <= a_t ||H_{t-1}|| + beta_t ||v_t|| (spectral norms)."""
    rng = np.random.default_rng(34)
    T = 30
    q, k, v, g, beta, s0 = rand_case(rng, 1, T, 1, 1, 6, 5)
    beta = f32(2.0 * beta)
    H = s0
    for t in range(T):
        _, H1 = oracle.fwd(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1], beta[:, t:t + 1],
                           scale=1.0, initial_state=H)
        lhs = np.linalg.norm(H1[0, 0], 2)
        rhs = math.exp(float(g[0, t, 0])) * np.linalg.norm(H[0, 0].astype(np.float64), 2) \
            + float(beta[0, t, 0]) * np.linalg.norm(v[0, t, 0].astype(np.float64))
        assert lhs <= rhs * (1 + 1e-6)
        H = H1.astype(np.float32)


# ---------------------------------------------------------------- chunk cumsum

def test_chunk_cumsum_closed_form_and_restart():
    g = np.full((1, 150, 2), -0.5, np.float32)
    out = oracle.chunk_cumsum(g, chunk=64)
    idx = np.arange(150) % 64
    np.testing.assert_array_equal(out[0, :, 0], -0.5 * (idx + 1))
    rng = np.random.default_rng(40)
    lens = [10, 70, 0, 65]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = f32(-rng.random((1, int(cu[-1]), 3)))
    out = oracle.chunk_cumsum(g, chunk=64, cu_seqlens=cu)
    for n in range(len(lens)):
        for c0 in range(int(cu[n]), int(cu[n + 1]), 64):
            c1 = min(c0 + 64, int(cu[n + 1]))
            np.testing.assert_allclose(out[0, c0:c1], np.cumsum(g[0, c0:c1].astype(np.float64), axis=0),
                                       rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- mutation checks

def _pins_pass(lib) -> bool:
    """Run the pins against an oracle library; False as soon as one fails."""
    try:
        rng = np.random.default_rng(0)
        q, k, v, g, beta, s0 = rand_case(rng, 1, 4, 1, 2, 3, 4, g_scale=0.7, unit=False)
        o, ht = oracle.fwd(q, k, v, g, beta, scale=0.75, initial_state=s0, lib=lib)
        for j in range(2):
            ob, Sb = _brute_force_head(q[0, :, 0], k[0, :, 0], v[0, :, j], g[0, :, j], beta[0, :, j], 0.75,
                                       s0[0, j].T)
            if not (np.allclose(o[0, :, j], ob, rtol=1e-10, atol=1e-12)
                    and np.allclose(ht[0, j], Sb, rtol=1e-10, atol=1e-12)):
                return False
        rng = np.random.default_rng(1)
        q, k, v, g, beta, s0 = rand_case(rng, 2, 70, 2, 4, 8, 6)
        o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0, lib=lib)
        oc, hc = chunked_wy(q, k, v, g, beta, 0.5, s0, 16)
        if not (np.allclose(o, oc, rtol=1e-9, atol=1e-11) and np.allclose(ht, hc, rtol=1e-9, atol=1e-11)):
            return False
        lens = [20, 0, 33]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        q, k, v, g, beta, s0 = rand_case(rng, 1, int(cu[-1]), 1, 2, 4, 3, N=3)
        o, ht = oracle.fwd(q, k, v, g, beta, scale=0.5, initial_state=s0, cu_seqlens=cu, lib=lib)
        oc, hc = chunked_wy(q, k, v, g, beta, 0.5, s0, 16, cu=cu)
        return bool(np.allclose(o, oc, rtol=1e-9, atol=1e-11) and np.allclose(ht, hc, rtol=1e-9, atol=1e-11))
    except ValueError:
        return False


MUTANTS = {
    "no_decay": ("for (int e = 0; e < K * V; ++e) H[e] *= a;", "for (int e = 0; e < K * V; ++e) H[e] *= 1.0;"),
    "decay_after_update": ("        /* decay */\n        for (int e = 0; e < K * V; ++e) H[e] *= a;\n", ""),
    "residual_sign": ("u[c] = b * ((double)vt[c] - p[c]);", "u[c] = b * ((double)vt[c] + p[c]);"),
    "no_beta": ("u[c] = b * ((double)vt[c] - p[c]);", "u[c] = ((double)vt[c] - p[c]);"),
    "beta_only_on_v": ("u[c] = b * ((double)vt[c] - p[c]);", "u[c] = b * (double)vt[c] - p[c];"),
    "gqa_modulo": ("const int i = j / grp;", "const int i = j % J->Hqk;"),
    "output_uses_k": ("const double qd = (double)qt[d];", "const double qd = (double)kt[d];"),
    "state_transposed_h0": ("for (int e = 0; e < K * V; ++e) H[e] = (double)s[e];",
                            "for (int e = 0; e < K * V; ++e) H[e] = (double)s[(e % V) * K + e / V];"),
    "varlen_offset": ("*r0 = J->cu[n];", "*r0 = J->cu[n] + (n > 0);"),
    "no_scale": ("ot[c] = J->scale * p[c];", "ot[c] = p[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    if name == "decay_after_update":
        # move the decay to after the rank-1 update instead of dropping it
        src = src.replace(old, new)
        src = src.replace("        /* o = scale H^T q */",
                          "        for (int e = 0; e < K * V; ++e) H[e] *= a;\n        /* o = scale H^T q */")
    else:
        src = src.replace(old, new)
    d = tempfile.mkdtemp()
    try:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "m.so")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-o", so, c, "-lm", "-lpthread"], check=True)
        lib = oracle.load_library(so)
        assert not _pins_pass(lib), f"mutant {name} slipped through the pins"
    finally:
        shutil.rmtree(d)


def test_unmutated_oracle_passes_mutation_harness():
    assert _pins_pass(oracle._load())
