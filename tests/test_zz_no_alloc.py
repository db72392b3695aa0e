"""The allocation-free forward (gdn_fwd_noalloc, for callers that cannot
allocate device memory) against gdn_fwd with a caller workspace, through the C
ABI: exact context parallelism (the mode whose kernels use a workspace), two
calls in a row with the second on a smaller input, so the second call runs on
the scratch array the first one left behind.  Both entry points launch the same
kernels on the same inputs, so the outputs must agree bit for bit; they are
also held to the exact-path bar against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_chunked_chunk_amd import api
from gated_deltanet_chunked_chunk_amd import _lib as L
from gated_deltanet_chunked_chunk_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL_EXACT = 1e-3


def _rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _call(x, L_seg, no_alloc):
    B, T, Hqk, K = x["q"].shape
    Hv, V = x["v"].shape[2], x["v"].shape[3]
    desc = api.make_desc(B, T, Hqk, Hv, K, V, scale=x["scale"], has_h0=True, want_ht=True, o_dtype="f32",
                         cp="exact", cp_segment_chunks=L_seg)
    info = api.plan(desc)
    assert info["cp"] == "exact" and info["workspace_bytes"] > 0
    o = torch.full((B, T, Hv, V), float("nan"), dtype=torch.float32, device=DEV)
    ht = torch.full((B, Hv, K, V), float("nan"), dtype=torch.float32, device=DEV)
    ptrs = L.FwdPtrs(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(),
                     x["beta"].data_ptr(), x["initial_state"].data_ptr(), None, o.data_ptr(), ht.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    if no_alloc:
        rc = L.lib().gdn_fwd_noalloc(ctypes.byref(desc), ctypes.byref(ptrs), stream)
    else:
        ws = api._workspace(info["workspace_bytes"], DEV)
        rc = L.lib().gdn_fwd(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                             stream)
    L.check(rc)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ht.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    torch.cuda.set_device(DEV)
    cases = [  # (T, H_qk, H_v, segment length); the second call is the smaller one
        (64 * 40 + 17, 2, 8, 3),
        (64 * 9 + 5, 1, 2, 2),
    ]
    for n, (T, Hqk, Hv, L_seg) in enumerate(cases):
        x = W.random_inputs(1, T, Hqk, Hv, seed=300 + n, g_mu=4.0, h0_std=0.1, device=DEV)
        print(f"[noalloc] call {n}: T={T} heads {Hqk}/{Hv} L={L_seg}", flush=True)
        o_na, ht_na = _call(x, L_seg, no_alloc=True)
        o_ws, ht_ws = _call(x, L_seg, no_alloc=False)
        np.testing.assert_array_equal(o_na, o_ws)
        np.testing.assert_array_equal(ht_na, ht_ws)
        q, k, v, g, b = (W.to_f32_numpy(x[m]) for m in ("q", "k", "v", "g", "beta"))
        o_ref, ht_ref = oracle.fwd(q, k, v, g, b, scale=x["scale"], initial_state=W.to_f32_numpy(x["initial_state"]))
        eo, eh = _rel_l2(o_na, o_ref), _rel_l2(ht_na, ht_ref)
        print(f"[noalloc] call {n}: rel_l2(o)={eo:.3e} rel_l2(ht)={eh:.3e}", flush=True)
        assert eo <= REL_EXACT and eh <= REL_EXACT


def test_noalloc_rejects_plans_beyond_its_scratch():
    # 400 one-chunk segments x 1 head x three 64 KiB maps = 75 MiB > 64 MiB
    desc = api.make_desc(1, 64 * 400, 1, 1, 128, 128, scale=128 ** -0.5, cp="exact", cp_segment_chunks=1)
    assert api.plan(desc)["workspace_bytes"] > L.NOALLOC_SCRATCH_BYTES
    o = torch.zeros(1, 64 * 400, 1, 128, dtype=torch.bfloat16, device=DEV)
    z = torch.zeros(1, 64 * 400, 1, 128, dtype=torch.bfloat16, device=DEV)
    gb = torch.zeros(1, 64 * 400, 1, dtype=torch.float32, device=DEV)
    ptrs = L.FwdPtrs(z.data_ptr(), z.data_ptr(), z.data_ptr(), gb.data_ptr(), gb.data_ptr(), None, None,
                     o.data_ptr(), None)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    rc = L.lib().gdn_fwd_noalloc(ctypes.byref(desc), ctypes.byref(ptrs), stream)
    assert rc == L.GDN_EWORKSPACE
    assert b"allocation-free" in L.lib().gdn_last_error()
