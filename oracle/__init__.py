"""fp64 CPU oracle for the Gated DeltaNet forward and backward.

TEST INFRASTRUCTURE ONLY: ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product package
(``gated_deltanet_chunked_chunk_amd``) never does, and shares no code with it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, one
thread per (sequence, v-head) unit).  This module only compiles that file
with gcc and marshals numpy arrays across ctypes.

Functions and what pins them (tests under ``tests/test_oracle_*.py``):

* ``fwd``            -- per-token gated delta rule (see the C file header).
  Pinned by exact-rational brute force on tiny inputs, closed forms (single
  token, beta = 0, strong decay, orthonormal-key retrieval, K = V = 1), an
  independent chunked WY form, and invariants (split-call continuity,
  varlen = separate calls, grouped heads = repeated heads, V-column
  independence).
* ``chunk_cumsum``   -- chunk-local running sum of g.  Pinned by constant-g
  closed forms and by numpy's cumsum per chunk.
* ``chunk_states``, ``chunk_wy_inverse`` -- the low-level forward's h and A
  by their definitions.  Pinned by beta = 0, a hand-worked two-token example
  and the WY identity against ``fwd``'s states.
* ``bwd``            -- reverse-mode derivative of the same per-token loop.
  Pinned by central finite differences of ``fwd`` in double (directional,
  and the full Jacobian on tiny shapes), by closed forms (one token with an
  initial state; beta = 0), and by mutation checks of its C source.

Inputs are widened to float64 before the call (exact for bf16 / float32
values), so finite differences can perturb them below float32 resolution.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source (gcc, -O2, pthreads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """ctypes handle with the oracle's signatures bound (used by the pin tests to
    load deliberately broken copies of the C source)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.gdn_oracle_fwd.restype = ctypes.c_int
    lib.gdn_oracle_fwd.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_int, P, P, ctypes.c_int]
    lib.gdn_oracle_chunk_cumsum.restype = ctypes.c_int
    lib.gdn_oracle_chunk_cumsum.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P]
    if hasattr(lib, "gdn_oracle_bwd"):
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
        output_final_state=True, n_threads=None, lib=None):
    """Reference forward.  Shapes follow the pages' high-level API:
    q, k [B,T,Hqk,K]; v [B,T,Hv,V]; g, beta [B,T,Hv]; initial_state
    [N,Hv,K,V] (K x V = S^T); cu_seqlens int [N+1] (B must be 1).
    Returns (o float64 [B,T,Hv,V], final_state float64 [N,Hv,K,V] or None).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, Hqk, K = q.shape
    V = v.shape[-1]
    Hv = v.shape[2]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("oracle.fwd: inconsistent shapes")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    h0 = None if initial_state is None else _f64(initial_state)
    if h0 is not None and h0.shape != (N, Hv, K, V):
        raise ValueError("oracle.fwd: initial_state must be [N,Hv,K,V]")
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, T, Hv, V), dtype=np.float64)
    ht = np.zeros((N, Hv, K, V), dtype=np.float64) if output_final_state else None
    rc = (lib or _load()).gdn_oracle_fwd(B, T, Hqk, Hv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                float(scale), _ptr(h0), _ptr(cu), N, _ptr(o), _ptr(ht),
                                int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle.fwd failed with code {rc}")
    return o, ht


def bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None, cu_seqlens=None,
        n_threads=None, lib=None):
    """Reference backward: the gradients of <do, o> + <dht, final_state>
    through ``fwd``'s recurrence (``dht`` None = no gradient into the final
    state).  Returns float64 (dq [B,T,Hqk,K], dk [B,T,Hqk,K], dv [B,T,Hv,V],
    dg [B,T,Hv], dbeta [B,T,Hv], dh0 [N,Hv,K,V]); dq and dk sum the
    contributions of the v-heads that share a key/query head."""
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv) \
            or do.shape != v.shape:
        raise ValueError("oracle.bwd: inconsistent shapes")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu, N = None, B
    h0 = None if initial_state is None else _f64(initial_state)
    dht = None if dht is None else _f64(dht)
    for name, x in (("initial_state", h0), ("dht", dht)):
        if x is not None and x.shape != (N, Hv, K, V):
            raise ValueError(f"oracle.bwd: {name} must be [N,Hv,K,V]")
    if scale is None:
        scale = K ** -0.5
    dq_v = np.zeros((B, T, Hv, K))
    dk_v = np.zeros((B, T, Hv, K))
    dv = np.zeros((B, T, Hv, V))
    dg = np.zeros((B, T, Hv))
    dbeta = np.zeros((B, T, Hv))
    dh0 = np.zeros((N, Hv, K, V))
    rc = (lib or _load()).gdn_oracle_bwd(B, T, Hqk, Hv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         float(scale), _ptr(h0), _ptr(cu), N, _ptr(do), _ptr(dht), _ptr(dq_v),
                                         _ptr(dk_v), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                         int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle.bwd failed with code {rc}")
    grp = Hv // Hqk
    dq = dq_v.reshape(B, T, Hqk, grp, K).sum(axis=3)
    dk = dk_v.reshape(B, T, Hqk, grp, K).sum(axis=3)
    return dq, dk, dv, dg, dbeta, dh0


def chunk_cumsum(g, chunk=64, cu_seqlens=None, lib=None):
    """Chunk-local running sum of g [B,T,H] (float64 result)."""
    g = _f64(g)
    B, T, H = g.shape
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu, N = None, B
    out = np.zeros((B, T, H), dtype=np.float64)
    rc = (lib or _load()).gdn_oracle_chunk_cumsum(B, T, H, chunk, _ptr(g), _ptr(cu), N, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle.chunk_cumsum failed with code {rc}")
    return out


def _seqs(B, T, cu_seqlens):
    """(batch row, first token, length) of every sequence, in order."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[n]), int(cu[n + 1] - cu[n])) for n in range(len(cu) - 1)]


def chunk_states(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, chunk=64, n_threads=None,
                 lib=None):
    """The state at the start of every chunk (the low-level forward's h; wiki,
    "low-level API"), by its plain definition: for chunk c of sequence n, the
    final state of the token-by-token recurrence (`fwd`) run over that
    sequence's first c * chunk tokens from its initial state.  Chunks of all
    sequences in order.  Returns float64 [total_chunks, Hv, K, V] (S^T)."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    h0 = None if initial_state is None else _f64(initial_state)
    out = []
    for n, (b, t0, L) in enumerate(_seqs(B, T, cu_seqlens)):
        start = np.zeros((Hv, K, V)) if h0 is None else h0[n].astype(np.float64)
        for c in range((L + chunk - 1) // chunk):
            if c == 0:
                out.append(start)
                continue
            t1 = t0 + c * chunk
            _, ht = fwd(q[b:b + 1, t0:t1], k[b:b + 1, t0:t1], v[b:b + 1, t0:t1], g[b:b + 1, t0:t1],
                        beta[b:b + 1, t0:t1], scale=scale, initial_state=None if h0 is None else h0[n:n + 1],
                        n_threads=n_threads, lib=lib)
            out.append(ht[0])
    if not out:
        return np.zeros((0, Hv, K, V))
    return np.stack(out)


def chunk_wy_inverse(k, g, beta, H_v, cu_seqlens=None, chunk=64):
    """The WY matrix of every chunk (the low-level forward's A; wiki,
    "low-level API"), by its definition: within a chunk, with G the running
    sum of g from the chunk start, A~_is = beta_i exp(G_i - G_s) k_i.k_s for
    s < i (0 elsewhere) and T = (I + A~)^{-1}; token i of the chunk gets row i
    of T.  v-head j reads key head j // (H_v / H_qk).  A partial last chunk
    uses its own rows only (its T is the leading block of the padded one).
    Returns float64 [B, T, H_v, chunk]."""
    k, g, beta = _f64(k), _f64(g), _f64(beta)
    B, T, Hqk, K = k.shape
    grp = H_v // Hqk
    out = np.zeros((B, T, H_v, chunk))
    for b, t0, L in _seqs(B, T, cu_seqlens):
        for c0 in range(t0, t0 + L, chunk):
            c1 = min(c0 + chunk, t0 + L)
            n = c1 - c0
            strict = np.tril(np.ones((n, n), dtype=bool), -1)
            for j in range(H_v):
                kc = k[b, c0:c1, j // grp].astype(np.float64)
                G = np.cumsum(g[b, c0:c1, j].astype(np.float64))
                decay = np.exp(np.where(strict, G[:, None] - G[None, :], 0.0))
                A = np.where(strict, beta[b, c0:c1, j].astype(np.float64)[:, None] * decay * (kc @ kc.T), 0.0)
                out[b, c0:c1, j, :n] = np.linalg.inv(np.eye(n) + A)
    return out
