"""CPU-side checks of the C ABI: the library loads, exports what include/gdn.h
declares, and its host-only planner validates and plans without touching a
GPU.  No compute entry point is called here."""
import ctypes
import os
import re

import pytest
import torch

import gated_deltanet_chunked_chunk_amd as G
from gated_deltanet_chunked_chunk_amd import _lib as L
from gated_deltanet_chunked_chunk_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = L.lib()
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = L.lib()
    assert lib.gdn_abi_version() == L.ABI_VERSION == 4
    for st in (0, -1, -2, -3, -4):
        assert lib.gdn_status_str(st)
    assert b"unknown" in lib.gdn_status_str(42)


def desc(**kw):
    base = dict(B=1, T=4096, H_qk=2, H_v=4, K=128, V=128)
    base.update({k: kw.pop(k) for k in list(kw) if k in base})
    kw.setdefault("scale", 128 ** -0.5)
    return G.make_desc(base["B"], base["T"], base["H_qk"], base["H_v"], base["K"], base["V"], **kw)


@pytest.mark.parametrize("bad,status", [
    (dict(H_v=3), L.GDN_EINVAL),
    (dict(H_qk=0), L.GDN_EINVAL),
    (dict(T=-1), L.GDN_EINVAL),
    (dict(K=64), L.GDN_EUNSUPPORTED),
    (dict(V=256), L.GDN_EUNSUPPORTED),
    (dict(chunk=32), L.GDN_EUNSUPPORTED),
])
def test_plan_rejects(bad, status):
    d = desc(**bad)
    info = L.FwdPlanInfo()
    rc = L.lib().gdn_fwd_plan(ctypes.byref(d), ctypes.byref(info))
    assert rc == status
    assert L.lib().gdn_last_error()


def test_plan_rejects_bad_cu_seqlens():
    for cu, T in (([1, 5, 10], 10), ([0, 5, 4, 10], 10), ([0, 5, 9], 10)):
        t = torch.tensor(cu, dtype=torch.int32)
        d = desc(T=T, cu_host=t)
        assert L.lib().gdn_fwd_plan(ctypes.byref(d), None) == L.GDN_EINVAL
    t = torch.tensor([0, 5, 10], dtype=torch.int32)
    d = desc(T=10, B=2, cu_host=t)
    assert L.lib().gdn_fwd_plan(ctypes.byref(d), None) == L.GDN_EINVAL


def test_plan_for_workloads():
    d = desc(T=32768, H_qk=16, H_v=16)
    p = G.plan(d)
    assert p["total_chunks"] == 512 and p["cp"] == "warmup"
    assert p["num_segments"] * p["segment_chunks"] >= 512
    assert p["workgroups"] == p["num_segments"] * 16
    d = desc(T=32768, H_qk=16, H_v=16, cp="off")
    p = G.plan(d)
    assert p["cp"] == "off" and p["num_segments"] == 1 and p["segment_chunks"] == 512
    d = desc(T=32768, H_qk=2, H_v=8, cp="warmup", cp_segment_chunks=16)
    p = G.plan(d)
    assert p["num_segments"] == 32 and p["warmup_chunks"] == 0  # no cap: the window is gate-driven
    d = desc(T=32768, H_qk=2, H_v=8, cp="warmup", cp_segment_chunks=16, cp_warmup_chunks=6)
    assert G.plan(d)["warmup_chunks"] == 6
    d = desc(T=32768, H_qk=2, H_v=8, cp="warmup", cp_lambda=1.0)
    assert G.plan(d)["segment_chunks"] == 23  # round(1.0 * sqrt(512))


def test_plan_exact_workspace():
    d = desc(T=32768, H_qk=2, H_v=8, cp="exact", cp_segment_chunks=16)
    p = G.plan(d)
    assert p["cp"] == "exact" and p["num_segments"] == 32
    # per-segment S, M and start state: three [segments][H_v][K][V] fp32 arrays
    assert p["workspace_bytes"] == 3 * 32 * 8 * 128 * 128 * 4
    d = desc(T=32768, H_qk=2, H_v=8, cp="exact", cp_segment_chunks=512)
    p = G.plan(d)
    assert p["cp"] == "off" and p["workspace_bytes"] == 0


def test_plan_varlen_segments():
    x = W.make_inputs(W.WORKLOADS["gdn_fwd_varlen16_65536_h8x24"], T=65536)
    cu = x["cu_seqlens"]
    d = desc(T=65536, H_qk=8, H_v=24, cu_host=cu, cp="warmup", cp_segment_chunks=16)
    p = G.plan(d)
    lens = (cu[1:] - cu[:-1]).tolist()
    chunks = [-(-n // 64) for n in lens]
    assert p["total_chunks"] == sum(chunks)
    assert p["num_segments"] == sum(max(1, -(-c // 16)) for c in chunks)


def test_plan_empty_and_zero_length():
    t = torch.tensor([0, 0, 0], dtype=torch.int32)
    d = desc(T=0, cu_host=t)
    p = G.plan(d)
    assert p["total_chunks"] == 0 and p["num_segments"] == 2  # one empty segment per sequence


def test_fwd_validation_happens_before_any_launch():
    """Invalid pointer sets fail in validation (no HIP call is reached)."""
    lib = L.lib()
    d = desc(T=128, has_h0=True, want_ht=True)
    ws = ctypes.create_string_buffer(4096)
    ptrs = L.FwdPtrs(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None, None, 0x6000, 0x7000)
    # has_h0 without a pointer
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    # misaligned q
    ptrs = L.FwdPtrs(0x1001, 0x2000, 0x3000, 0x4000, 0x5000, 0x8000, None, 0x6000, 0x7000)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    # o overlapping v
    base = 0x100000
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, None, base * 3 + 256, base * 8)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    assert b"o overlaps v" in lib.gdn_last_error()
    # final_state overlapping initial_state
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, None, base * 7, base * 6)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    # device offsets without host offsets
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, base * 10, base * 7, base * 9)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), None, 0, None) == L.GDN_EINVAL
    # low-level outputs: misaligned h, A overlapping o, h overlapping A
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, None, base * 7, base * 8,
                     base * 9 + 8, None)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    assert b"16-byte aligned" in lib.gdn_last_error()
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, None, base * 7, base * 8,
                     None, base * 7 + 512)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    assert b"A overlaps o" in lib.gdn_last_error() or b"o overlaps A" in lib.gdn_last_error()
    ptrs = L.FwdPtrs(base, base * 2, base * 3, base * 4, base * 5, base * 6, None, base * 7, base * 8,
                     base * 9, base * 9 + 4096)
    assert lib.gdn_fwd(ctypes.byref(d), ctypes.byref(ptrs), ws, 4096, None) == L.GDN_EINVAL
    assert b"overlaps" in lib.gdn_last_error()


def test_python_api_refuses_cpu_tensors():
    x = W.random_inputs(1, 64, 1, 1)
    with pytest.raises(ValueError):
        G.chunk_gated_delta_rule(x["q"], x["k"], x["v"], x["g"], x["beta"])


def test_plan_has_no_sequence_length_limit():
    """Buffer resources are per chunk: a sequence whose rows span more than
    2 GiB of a tensor plans fine; only a single chunk must stay below 2 GiB."""
    assert G.plan(desc(T=1 << 24, H_qk=16, H_v=64))["total_chunks"] == (1 << 24) // 64
    d = desc(T=128, H_qk=1, H_v=70000)
    d.o_dtype = L.GDN_DTYPE_F32
    assert L.lib().gdn_fwd_plan(ctypes.byref(d), None) == L.GDN_EUNSUPPORTED
    assert b"per-chunk range" in L.lib().gdn_last_error()


def bdesc(**kw):
    extra = {k: kw.pop(k) for k in ("has_dht", "grad_dtype", "saved_fwd") if k in kw}
    return G.make_bwd_desc(desc(**kw), **extra)


def test_bwd_plan_layout_and_workspace():
    # backward workload shape: 1 x 32768 tokens, 4 key heads, 16 value heads
    p = G.bwd_plan(bdesc(T=32768, H_qk=4, H_v=16, has_h0=True, has_dht=True))
    assert p["total_chunks"] == 512 and p["cp"] == "warmup"
    assert p["workgroups_reverse"] == p["num_segments"] * 16 * 2
    assert p["workgroups_local"] == 512 * 4  # one per (chunk, key head): its v-heads run in turn
    rows, hv, hqk, K = 32768, 16, 4, 128
    n_h = 512 * hv * K * K * 4
    dvp = 512 * hv * 64 * K * 4
    dqk = 2 * rows * hqk * K * 4  # partial key-head sums of dq and dk
    recompute = rows * hv * K * 2 + n_h + rows * hv * 64 * 4 + dvp
    assert p["workspace_bytes"] == n_h + dvp + dqk + recompute
    saved = G.bwd_plan(bdesc(T=32768, H_qk=4, H_v=16, saved_fwd=True))
    assert saved["workspace_bytes"] == n_h + dvp + dqk
    off = G.bwd_plan(bdesc(T=32768, H_qk=4, H_v=16, cp="off"))
    assert off["cp"] == "off" and off["num_segments"] == 1 and off["warmup_chunks"] == 0
    # exact CP: three [segments][H_v][K][V] fp32 arrays for the reverse pass; when
    # the forward is recomputed, the forward's own three as well
    ex = G.bwd_plan(bdesc(T=32768, H_qk=4, H_v=16, cp="exact", cp_segment_chunks=64, saved_fwd=True))
    st = 8 * hv * K * K * 4
    assert ex["cp"] == "exact" and ex["num_segments"] == 8
    assert ex["workspace_bytes"] == n_h + dvp + dqk + 3 * st
    exr = G.bwd_plan(bdesc(T=32768, H_qk=4, H_v=16, cp="exact", cp_segment_chunks=64))
    assert exr["workspace_bytes"] == n_h + dvp + dqk + 3 * st + recompute + 3 * st


def test_bwd_plan_rejects():
    for kw, st in ((dict(K=64), L.GDN_EUNSUPPORTED), (dict(H_v=3), L.GDN_EINVAL)):
        d = bdesc(**kw)
        assert L.lib().gdn_bwd_plan(ctypes.byref(d), None) == st
        assert L.lib().gdn_last_error()
    d = bdesc()
    d.grad_dtype = 7
    assert L.lib().gdn_bwd_plan(ctypes.byref(d), None) == L.GDN_EINVAL


def test_bwd_plan_varlen_entries():
    cu = torch.tensor([0, 100, 100, 300], dtype=torch.int32)
    p = G.bwd_plan(bdesc(T=300, H_qk=1, H_v=2, cu_host=cu, cp="off"))
    assert p["total_chunks"] == 2 + 0 + 4
    assert p["workgroups_local"] == (6 + 1) * 1  # one entry for the empty sequence, one workgroup per key head


def test_bwd_validation_happens_before_any_launch():
    lib = L.lib()
    base = 0x100000
    d = bdesc(T=128, has_h0=True, has_dht=True)
    ws = ctypes.create_string_buffer(1 << 12)
    mk = lambda **o: L.BwdPtrs(**{**dict(q=base, k=2 * base, v=3 * base, g=4 * base, beta=5 * base,  # noqa: E731
                                         initial_state=6 * base, cu_seqlens=None, dO=7 * base,
                                         d_final_state=8 * base, h=None, A=None, dq=9 * base, dk=10 * base,
                                         dv=11 * base, dg=12 * base, dbeta=13 * base,
                                         d_initial_state=14 * base), **o})
    # d_final_state given without has_dht
    d2 = bdesc(T=128, has_h0=True)
    assert lib.gdn_bwd(ctypes.byref(d2), ctypes.byref(mk()), ws, 1 << 12, None) == L.GDN_EINVAL
    # h without A and v_new
    d3 = bdesc(T=128, has_h0=True, has_dht=True, saved_fwd=True)
    assert lib.gdn_bwd(ctypes.byref(d3), ctypes.byref(mk(h=15 * base)), ws, 1 << 12, None) == L.GDN_EINVAL
    assert lib.gdn_bwd(ctypes.byref(d3), ctypes.byref(mk(h=15 * base, A=16 * base)), ws, 1 << 12,
                       None) == L.GDN_EINVAL
    # misaligned dO
    assert lib.gdn_bwd(ctypes.byref(d), ctypes.byref(mk(dO=7 * base + 2)), ws, 1 << 12, None) == L.GDN_EINVAL
    # dv overlapping v
    assert lib.gdn_bwd(ctypes.byref(d), ctypes.byref(mk(dv=3 * base + 256)), ws, 1 << 12, None) == L.GDN_EINVAL
    assert b"dv overlaps v" in lib.gdn_last_error()
    # workspace too small
    assert lib.gdn_bwd(ctypes.byref(d), ctypes.byref(mk()), ws, 1 << 12, None) == L.GDN_EWORKSPACE


def test_chunk_cumsum_rejects_bad_offsets_on_the_host():
    """gdn_chunk_cumsum: offsets without a sequence are rejected before any
    launch; the Python wrapper validates a host copy of the offsets (the
    forward's contract) before handing them to the kernel."""
    lib = L.lib()
    base = 0x100000
    assert lib.gdn_chunk_cumsum(ctypes.c_void_p(base), ctypes.c_void_p(2 * base), 1, 10, 2, 64,
                                ctypes.c_void_p(3 * base), 0, None) == L.GDN_EINVAL
    assert b"num_seqs" in lib.gdn_last_error()
    assert lib.gdn_chunk_cumsum(ctypes.c_void_p(base), ctypes.c_void_p(2 * base), 2, 10, 2, 64,
                                ctypes.c_void_p(3 * base), 1, None) == L.GDN_EINVAL
    from gated_deltanet_chunked_chunk_amd import api
    for cu, B, T in (([0, 5, 12], 1, 10), ([1, 10], 1, 10), ([0, 6, 4, 10], 1, 10), ([0], 1, 0), ([0, 10], 2, 10)):
        with pytest.raises(ValueError):
            api._check_offsets(torch.tensor(cu, dtype=torch.int32), B, T)
    api._check_offsets(torch.tensor([0, 0, 4, 10], dtype=torch.int32), 1, 10)
