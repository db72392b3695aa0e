"""GPU parity of the low-level forward (aisparkup.com FlashQLA wiki, "low-level
API": g, A, o, h, final_state) against the oracle's definitions:

* h (state at every chunk start) vs oracle.chunk_states: relative L2 <= 1e-3 on
  the exact paths (CP off / exact), <= 5e-3 under warm-up CP;
* A (each chunk's WY matrix rows) vs oracle.chunk_wy_inverse: max-abs <= 1e-4
  (entries are O(1); the GPU inverts in fp32 with hi/lo bf16 MFMA merges);
* g vs oracle.chunk_cumsum, o and final_state as in the main parity tests;
* v_new (each chunk's v' = U - W h, kept for the backward) vs the same
  formula evaluated in fp64 from the oracle's h and A (whose composition the
  oracle tests pin to the per-token recurrence): the bar of h.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_chunked_chunk_amd import chunk_gated_delta_rule_fwd
from gated_deltanet_chunked_chunk_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _host(x):
    q, k, v, g, b = (W.to_f32_numpy(x[n]) for n in ("q", "k", "v", "g", "beta"))
    h0 = W.to_f32_numpy(x["initial_state"])
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy()
    return q, k, v, g, b, h0, cu


def _check(name, x, rel_h, **kw):
    q, k, v, g, b, h0, cu = _host(x)
    Hv = v.shape[2]
    g_cum, A, o, h, ht, vn = chunk_gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                        scale=x["scale"], initial_state=x["initial_state"],
                                                        cu_seqlens=x["cu_seqlens"], o_dtype="f32",
                                                        output_v_new=True, **kw)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.fwd(q, k, v, g, b, scale=x["scale"], initial_state=h0, cu_seqlens=cu)
    h_ref = oracle.chunk_states(q, k, v, g, b, scale=x["scale"], initial_state=h0, cu_seqlens=cu)
    a_ref = oracle.chunk_wy_inverse(k, g, b, Hv, cu_seqlens=cu)
    g_ref = oracle.chunk_cumsum(g, 64, cu)
    h_g, a_g = h.cpu().numpy(), A.cpu().numpy()
    assert h_g.shape == h_ref.shape and a_g.shape == a_ref.shape
    eh, ea = rel_l2(h_g, h_ref), float(np.max(np.abs(a_g - a_ref))) if a_g.size else 0.0
    eo, et = rel_l2(o.cpu().numpy(), o_ref), rel_l2(ht.cpu().numpy(), ht_ref)
    eg = float(np.max(np.abs(g_cum.cpu().numpy() - g_ref))) if g_ref.size else 0.0
    print(f"[{name}] rel_l2(h)={eh:.3e} max_abs(A)={ea:.3e} rel_l2(o)={eo:.3e} rel_l2(ht)={et:.3e} "
          f"max_abs(g)={eg:.3e}", flush=True)
    assert np.isfinite(h_g).all() and np.isfinite(a_g).all()
    assert eh <= rel_h and eo <= rel_h and et <= rel_h
    assert ea <= 1e-4
    assert eg <= 1e-4
    vn_ref = _v_new_ref(k, v, g, b, h_ref, a_ref, cu)
    ev = rel_l2(vn.cpu().numpy(), vn_ref)
    print(f"[{name}] rel_l2(v_new)={ev:.3e}", flush=True)
    assert ev <= rel_h


def _v_new_ref(k, v, g, b, h_ref, a_ref, cu):
    """v' = T diag(beta) V - T diag(beta gamma) K h per chunk (zero rows past a sequence end)."""
    B, T, Hqk, K = k.shape
    Hv, V = v.shape[2], v.shape[3]
    seqs = [(bb, 0, T) for bb in range(B)] if cu is None else \
        [(0, int(cu[n]), int(cu[n + 1] - cu[n])) for n in range(len(cu) - 1)]
    out = np.zeros((h_ref.shape[0], Hv, 64, V))
    idx = 0
    for bb, t0, L in seqs:
        for c in range((L + 63) // 64):
            c0, c1 = t0 + 64 * c, min(t0 + 64 * c + 64, t0 + L)
            m = c1 - c0
            for j in range(Hv):
                kc = k[bb, c0:c1, j // (Hv // Hqk)].astype(np.float64)
                bc = b[bb, c0:c1, j].astype(np.float64)
                gam = np.exp(np.cumsum(g[bb, c0:c1, j].astype(np.float64)))
                Tm = a_ref[bb, c0:c1, j, :m]
                out[idx + c, j, :m] = Tm @ (bc[:, None] * v[bb, c0:c1, j]) - Tm @ ((bc * gam)[:, None] * kc) @ h_ref[idx + c, j]
        idx += (L + 63) // 64
    return out


def test_lowlevel_tiny():
    x = W.make_inputs(W.WORKLOADS["gdn_fwd_1x512_h2x2"], device=DEV)
    _check("tiny/off", x, 1e-3, cp="off")


@pytest.mark.parametrize("cp,rel", [("off", 1e-3), ("exact", 1e-3), ("warmup", 5e-3)])
def test_lowlevel_ragged_with_state(cp, rel):
    w = dataclasses.replace(W.WORKLOADS["gdn_fwd_1x512_h2x2"], name="ll", seed=31, B=2, T=700, H_qk=1, H_v=3,
                            h0_std=0.1)
    x = W.make_inputs(w, device=DEV)
    _check(f"ragged/{cp}", x, rel, cp=cp, cp_segment_chunks=3)


def test_lowlevel_varlen():
    w = dataclasses.replace(W.WORKLOADS["gdn_fwd_1x512_h2x2"], name="llv", seed=32, B=1, T=0, H_qk=2, H_v=4,
                            h0_std=0.1)
    x = W.make_inputs(w, device=DEV, lengths=[130, 0, 1, 64, 300])
    _check("varlen/exact", x, 1e-3, cp="exact", cp_segment_chunks=2)
