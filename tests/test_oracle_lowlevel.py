"""Pins of the oracle's low-level outputs (the pages' low-level forward returns
g, A, o, h, final_state; aisparkup.com FlashQLA wiki, "low-level API"):

* chunk_wy_inverse (A): beta = 0 gives the identity; a two-token chunk worked
  by hand; and, with chunk_states, the chunked WY identity -- W = T diag(beta
  e^G) K, U = T diag(beta) V, v' = U - W H, O = scale (diag(e^G) Q H +
  causal(e^{G_i-G_s} q_i.k_s) v'), H' = e^{G_last} H + (diag(e^{G_last-G}) K)^T
  v' -- reproduces the token-by-token recurrence's o and every next chunk
  state, chunk by chunk.  That identity is exact, so a wrong sign, index,
  decay or beta in either function fails it.
* chunk_states (h): the first state of a sequence is its initial state; the
  state after its last chunk (through the WY step) is the recurrence's final
  state.
"""
import numpy as np
import pytest

import oracle

from test_oracle_pins import f32, rand_case  # noqa: E402


def test_wy_inverse_beta_zero_is_identity():
    rng = np.random.default_rng(1)
    q, k, v, g, beta, _ = rand_case(rng, 1, 100, 1, 2, 8, 4, h0=False)
    A = oracle.chunk_wy_inverse(k, g, np.zeros_like(beta), 2)
    for c0 in (0, 64):
        n = min(64, 100 - c0)
        for j in range(2):
            np.testing.assert_array_equal(A[0, c0:c0 + n, j, :n], np.eye(n))
            np.testing.assert_array_equal(A[0, c0:c0 + n, j, n:], 0.0)


def test_wy_inverse_two_tokens_by_hand():
    # k0 = (1, 0), k1 = (0.6, 0.8): k1.k0 = 0.6; g1 = ln(0.5); beta1 = 0.25
    k = np.array([[[[1.0, 0.0]], [[0.6, 0.8]]]], dtype=np.float32)
    g = np.array([[[-1.0], [np.log(0.5)]]], dtype=np.float32)
    beta = np.array([[[0.9], [0.25]]], dtype=np.float32)
    A = oracle.chunk_wy_inverse(k, g, beta, 1)
    # A~_10 = beta_1 e^{G_1 - G_0} k1.k0 = 0.25 * 0.5 * 0.6; T = [[1, 0], [-A~_10, 1]]
    a10 = 0.25 * float(np.float32(0.5)) * np.float64(np.float32(0.6))
    np.testing.assert_allclose(A[0, 0, 0, :2], [1.0, 0.0], atol=1e-7)
    np.testing.assert_allclose(A[0, 1, 0, :2], [-a10, 1.0], rtol=1e-6)


def _wy_chunk(Q, Kc, Vc, bt, gc, H, T, scale):
    G = np.cumsum(gc)
    W = T @ ((bt * np.exp(G))[:, None] * Kc)
    U = T @ (bt[:, None] * Vc)
    vp = U - W @ H
    D = G[:, None] - G[None, :]
    P = np.where(np.tril(np.ones_like(D)) > 0, np.exp(np.where(np.tril(np.ones_like(D)) > 0, D, 0.0)), 0.0) * (Q @ Kc.T)
    O = scale * (np.exp(G)[:, None] * (Q @ H) + P @ vp)
    Hn = np.exp(G[-1]) * H + (np.exp(G[-1] - G)[:, None] * Kc).T @ vp
    return O, Hn


@pytest.mark.parametrize("varlen", [False, True])
def test_wy_identity_with_chunk_states(varlen):
    rng = np.random.default_rng(7 + varlen)
    if varlen:
        lens = [70, 0, 1, 129, 64]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T, N = 1, int(cu[-1]), len(lens)
    else:
        cu, B, T, N = None, 2, 150, 2
    Hqk, Hv, K, V = 1, 3, 16, 8
    q, k, v, g, beta, s0 = rand_case(rng, B, T, Hqk, Hv, K, V, g_scale=0.4, N=N)
    scale = 0.3
    o, ht = oracle.fwd(q, k, v, g, beta, scale=scale, initial_state=s0, cu_seqlens=cu)
    h = oracle.chunk_states(q, k, v, g, beta, scale=scale, initial_state=s0, cu_seqlens=cu)
    A = oracle.chunk_wy_inverse(k, g, beta, Hv, cu_seqlens=cu)
    seqs = [(b, 0, T) for b in range(B)] if cu is None else [(0, int(cu[n]), int(cu[n + 1] - cu[n])) for n in range(N)]
    total = sum((L + 63) // 64 for _, _, L in seqs)
    assert h.shape == (total, Hv, K, V)
    idx = 0
    grp = Hv // Hqk
    for n, (b, t0, L) in enumerate(seqs):
        nt = (L + 63) // 64
        for c in range(nt):
            c0, c1 = t0 + 64 * c, min(t0 + 64 * c + 64, t0 + L)
            m = c1 - c0
            if c == 0:
                np.testing.assert_array_equal(h[idx], s0[n].astype(np.float64))
            for j in range(Hv):
                i = j // grp
                O, Hn = _wy_chunk(q[b, c0:c1, i].astype(np.float64), k[b, c0:c1, i].astype(np.float64),
                                  v[b, c0:c1, j].astype(np.float64), beta[b, c0:c1, j].astype(np.float64),
                                  g[b, c0:c1, j].astype(np.float64), h[idx + c, j], A[b, c0:c1, j, :m], scale)
                np.testing.assert_allclose(O, o[b, c0:c1, j], rtol=1e-9, atol=1e-11)
                nxt = h[idx + c + 1, j] if c + 1 < nt else ht[n, j]
                np.testing.assert_allclose(Hn, nxt, rtol=1e-9, atol=1e-11)
        idx += nt
