"""Memory hygiene of the forward and backward through the C ABI: every output
and the workspace sit inside a larger buffer whose guard bands hold a
sentinel, the outputs themselves start as NaN.  After the call the guard
bands must be untouched (no write outside an output or the workspace), every
output element must be finite (every element written), and the results must
equal those of the ordinary entry points bit for bit.  Cases: ragged tails,
varlen batches with empty and one-token sequences, grouped heads, and the
context-parallel modes whose kernels use the workspace."""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_chunked_chunk_amd import api
from gated_deltanet_chunked_chunk_amd import _lib as L
from gated_deltanet_chunked_chunk_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096  # elements of sentinel on each side (16 KiB of fp32)
SENTINEL = 7.0


class Guarded:
    """A float32 view of `n_bytes` inside a buffer with sentinel guard bands;
    the view starts as NaN."""

    def __init__(self, n_bytes, align=256):
        n = (max(n_bytes, 4) + 3) // 4
        self.buf = torch.full((n + 2 * GUARD + align,), SENTINEL, dtype=torch.float32, device=DEV)
        off = GUARD + ((-(self.buf.data_ptr() + 4 * GUARD)) % align) // 4
        self.off, self.n, self.n_bytes = off, n, n_bytes
        self.buf[off:off + n] = float("nan")

    def ptr(self):
        return self.buf.data_ptr() + 4 * self.off

    def view(self, shape, dtype):
        raw = self.buf[self.off:self.off + self.n]
        return raw.view(torch.uint8)[:self.n_bytes].view(dtype).view(shape)

    def guards_intact(self):
        a = self.buf[:self.off]
        b = self.buf[self.off + self.n:]
        return bool(torch.all(a == SENTINEL)) and bool(torch.all(b == SENTINEL))


def _inputs(case):
    if case == "ragged":
        return W.random_inputs(2, 64 * 5 + 23, 1, 3, seed=61, h0_std=0.1, device=DEV), dict(cp="warmup",
                                                                                           cp_segment_chunks=2)
    if case == "varlen":
        return W.random_inputs(1, 0, 2, 4, seed=62, h0_std=0.1, lengths=[130, 0, 1, 64, 300], device=DEV), \
            dict(cp="exact", cp_segment_chunks=2)
    return W.random_inputs(1, 64 * 9 + 5, 2, 4, seed=63, h0_std=0.1, device=DEV), dict(cp="exact",
                                                                                      cp_segment_chunks=3)


@pytest.mark.parametrize("case", ["ragged", "varlen", "exact"])
def test_forward_writes_exactly_its_outputs(case):
    x, kw = _inputs(case)
    B, T, Hqk, K = x["q"].shape
    Hv, V = x["v"].shape[2], x["v"].shape[3]
    cu_host = x["cu_seqlens"]
    N = B if cu_host is None else cu_host.numel() - 1
    desc = api.make_desc(B, T, Hqk, Hv, K, V, scale=x["scale"], cu_host=cu_host, has_h0=True, want_ht=True,
                         o_dtype="f32", **kw)
    info = api.plan(desc)
    nc = info["total_chunks"]
    outs = {"o": (B, T, Hv, V), "ht": (N, Hv, K, V), "h": (nc, Hv, K, V), "A": (B, T, Hv, 64),
            "vn": (nc, Hv, 64, V)}
    g = {k: Guarded(int(np.prod(s)) * 4) for k, s in outs.items()}
    ws = Guarded(info["workspace_bytes"])
    cu_dev = None if cu_host is None else cu_host.to(DEV)
    ptrs = L.FwdPtrs(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(), x["beta"].data_ptr(),
                     x["initial_state"].data_ptr(), cu_dev.data_ptr() if cu_dev is not None else None,
                     g["o"].ptr(), g["ht"].ptr(), g["h"].ptr(), g["A"].ptr(), g["vn"].ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    L.check(L.lib().gdn_fwd(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.c_void_p(ws.ptr()),
                            info["workspace_bytes"], stream))
    torch.cuda.synchronize()
    print(f"[{case}] cp={info['cp']} workspace={info['workspace_bytes']} chunks={nc}", flush=True)
    for k, s in outs.items():
        assert g[k].guards_intact(), f"write outside {k}"
        assert torch.isfinite(g[k].view(s, torch.float32)).all(), f"{k} not fully written"
    assert ws.guards_intact(), "write outside the workspace"
    ref = api.chunk_gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                         initial_state=x["initial_state"], cu_seqlens=cu_host, output_v_new=True,
                                         o_dtype="f32", **kw)
    _, A, o, h, ht, vn = ref
    for k, r in (("o", o), ("ht", ht), ("h", h), ("A", A), ("vn", vn)):
        assert torch.equal(g[k].view(outs[k], torch.float32), r), k


@pytest.mark.parametrize("case", ["ragged", "varlen", "exact"])
def test_backward_writes_exactly_its_outputs(case):
    x, kw = _inputs(case)
    B, T, Hqk, K = x["q"].shape
    Hv, V = x["v"].shape[2], x["v"].shape[3]
    cu_host = x["cu_seqlens"]
    N = B if cu_host is None else cu_host.numel() - 1
    gen = torch.Generator().manual_seed(64)
    dO = torch.randn(B, T, Hv, V, generator=gen).to(torch.bfloat16).to(DEV)
    dht = (torch.randn(N, Hv, K, V, generator=gen) * 0.01).to(DEV)
    fd = api.make_desc(B, T, Hqk, Hv, K, V, scale=x["scale"], cu_host=cu_host, has_h0=True, **kw)
    desc = api.make_bwd_desc(fd, has_dht=True, grad_dtype="f32", saved_fwd=False)
    info = api.bwd_plan(desc)
    outs = {"dq": (B, T, Hqk, K), "dk": (B, T, Hqk, K), "dv": (B, T, Hv, V), "dg": (B, T, Hv),
            "dbeta": (B, T, Hv), "dh0": (N, Hv, K, V)}
    g = {k: Guarded(int(np.prod(s)) * 4) for k, s in outs.items()}
    ws = Guarded(info["workspace_bytes"])
    cu_dev = None if cu_host is None else cu_host.to(DEV)
    ptrs = L.BwdPtrs(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(), x["beta"].data_ptr(),
                     x["initial_state"].data_ptr(), cu_dev.data_ptr() if cu_dev is not None else None,
                     dO.data_ptr(), dht.data_ptr(), None, None, None, g["dq"].ptr(), g["dk"].ptr(), g["dv"].ptr(),
                     g["dg"].ptr(), g["dbeta"].ptr(), g["dh0"].ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    L.check(L.lib().gdn_bwd(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.c_void_p(ws.ptr()),
                            info["workspace_bytes"], stream))
    torch.cuda.synchronize()
    print(f"[{case}] reverse cp={info['cp']} workspace={info['workspace_bytes']}", flush=True)
    for k, s in outs.items():
        assert g[k].guards_intact(), f"write outside {k}"
        assert torch.isfinite(g[k].view(s, torch.float32)).all(), f"{k} not fully written"
    assert ws.guards_intact(), "write outside the workspace"
    ref = api.chunk_gated_delta_rule_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, scale=x["scale"],
                                         initial_state=x["initial_state"], cu_seqlens=cu_host, d_final_state=dht,
                                         grad_dtype="f32", **kw)
    for k, r in zip(outs, ref):
        assert torch.equal(g[k].view(outs[k], torch.float32), r), k
