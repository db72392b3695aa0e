"""Python entry points over libgdn.  Argument marshalling only: shapes, dtypes
and devices are checked, outputs and the workspace are allocated with torch,
and every step of the computation runs in the library's HIP kernels on the
caller's current stream.

The high-level signature follows the pages' API (aisparkup.com FlashQLA wiki,
"high-level API"; summarylog.com essay, usage example):
``chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
output_final_state, cu_seqlens) -> (o, final_state)``.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib as L


def _cu_host(cu_seqlens) -> Optional[torch.Tensor]:
    if cu_seqlens is None:
        return None
    if isinstance(cu_seqlens, torch.Tensor):
        # a device tensor needs one device-to-host copy for planning (a sync)
        return cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    return torch.as_tensor(list(cu_seqlens), dtype=torch.int32)


def _check_offsets(cu_host: torch.Tensor, B: int, T: int) -> None:
    """The packed-sequence contract: B == 1, at least one sequence, offsets
    starting at 0, non-decreasing, ending at T."""
    if B != 1:
        raise ValueError(f"cu_seqlens requires B == 1 (got {B})")
    if cu_host.dim() != 1 or cu_host.numel() < 2:
        raise ValueError("cu_seqlens needs at least two offsets (one sequence)")
    c = cu_host.tolist()
    if c[0] != 0 or c[-1] != T or any(b < a for a, b in zip(c, c[1:])):
        raise ValueError(f"cu_seqlens must start at 0, be non-decreasing and end at T={T} (got {c[:4]}...{c[-2:]})")


def make_desc(B, T, H_qk, H_v, K, V, *, scale, cu_host=None, has_h0=False, want_ht=False, o_dtype="bf16",
              cp="auto", cp_lambda=0.0, cp_segment_chunks=0, cp_warmup_chunks=0, chunk=64) -> L.FwdDesc:
    d = L.FwdDesc()
    d.B, d.T, d.H_qk, d.H_v, d.K, d.V = int(B), int(T), int(H_qk), int(H_v), int(K), int(V)
    if cu_host is not None:
        d.num_seqs = int(cu_host.numel()) - 1
        d.cu_seqlens_host = ctypes.cast(ctypes.c_void_p(cu_host.data_ptr()), ctypes.POINTER(ctypes.c_int32))
    else:
        d.num_seqs = int(B)
        d.cu_seqlens_host = None
    d.scale = float(scale)
    d.has_h0 = int(bool(has_h0))
    d.want_ht = int(bool(want_ht))
    d.o_dtype = {"bf16": L.GDN_DTYPE_BF16, "f32": L.GDN_DTYPE_F32}[o_dtype]
    d.chunk = int(chunk)
    if cp not in L.CP_MODES:
        raise ValueError(f"cp must be one of {sorted(L.CP_MODES)}")
    d.cp_mode = L.CP_MODES[cp]
    d.cp_lambda = float(cp_lambda)
    d.cp_segment_chunks = int(cp_segment_chunks)
    d.cp_warmup_chunks = int(cp_warmup_chunks)
    return d


def plan(desc: L.FwdDesc) -> dict:
    """Host-only planning (no GPU needed): resolved CP layout and workspace size."""
    info = L.FwdPlanInfo()
    L.check(L.lib().gdn_fwd_plan(ctypes.byref(desc), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in L.FwdPlanInfo._fields_} | {"cp": L.CP_NAMES[info.cp_mode]}


def _workspace(nbytes: int, device) -> torch.Tensor:
    buf = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 1)]


def _need(t: torch.Tensor, name: str, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_gated_delta_rule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                           beta: torch.Tensor, scale: Optional[float] = None,
                           initial_state: Optional[torch.Tensor] = None, output_final_state: bool = False,
                           cu_seqlens=None, *, cp: str = "auto", o_dtype: Optional[str] = None,
                           cp_lambda: float = 0.0, cp_segment_chunks: int = 0, cp_warmup_chunks: int = 0,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gated DeltaNet chunked-prefill forward on the GPU.

    q, k: bf16 [B, T, H_qk, K]; v: bf16 [B, T, H_v, V]; g, beta: fp32 [B, T, H_v];
    initial_state: fp32 [N, H_v, K, V] (S^T per head); cu_seqlens: int32 offsets
    [N + 1] (B must be 1).  Returns (o [B, T, H_v, V], final_state or None).
    ``cp`` selects the intra-GPU context parallelism: "auto", "warmup", "exact", "off".
    Differentiable: when autograd records (an input requires grad), the call
    keeps the forward's chunk states h and WY matrices A and its backward runs
    gdn_bwd on them (dq, dk, dv in the inputs' bf16; dg, dbeta, d initial_state fp32).
    """
    if torch.is_grad_enabled() and any(isinstance(t, torch.Tensor) and t.requires_grad
                                       for t in (q, k, v, g, beta, initial_state)):
        if out is not None:
            raise ValueError("out= cannot be used when autograd records the call")
        return _GDNFunction.apply(q, k, v, g, beta, initial_state, scale, output_final_state, cu_seqlens,
                                  dict(cp=cp, o_dtype=o_dtype, cp_lambda=cp_lambda,
                                       cp_segment_chunks=cp_segment_chunks, cp_warmup_chunks=cp_warmup_chunks))
    o, ht, _, _, _ = _forward(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens, cp=cp,
                           o_dtype=o_dtype, cp_lambda=cp_lambda, cp_segment_chunks=cp_segment_chunks,
                           cp_warmup_chunks=cp_warmup_chunks, out=out, workspace=workspace)
    return o, ht


def chunk_gated_delta_rule_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                               beta: torch.Tensor, scale: Optional[float] = None,
                               initial_state: Optional[torch.Tensor] = None, cu_seqlens=None,
                               output_final_state: bool = True, output_v_new: bool = False, **kw):
    """The pages' low-level forward (aisparkup.com FlashQLA wiki, "low-level
    API"): returns (g, A, o, h, final_state) with
      g  fp32 [B, T, H_v]: the chunk-local running sum of the gates;
      A  fp32 [B, T, H_v, 64]: for each token, its row of its chunk's WY matrix
         (I + A~)^{-1}, A~_is = beta_i exp(G_i - G_s) k_i.k_s (s < i);
      o  [B, T, H_v, V] (bf16 unless o_dtype="f32");
      h  fp32 [total_chunks, H_v, K, V]: S^T at the start of every chunk;
      final_state fp32 [N, H_v, K, V] or None.
    With output_v_new, a sixth element: v_new fp32 [total_chunks, H_v, 64, V],
    every chunk's v' = U - W h (what the backward consumes with h and A).
    Everything except g comes from one gdn_fwd call; g from gdn_chunk_cumsum."""
    o, ht, h, A, vn = _forward(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                               want_h=True, want_a=True, want_vn=output_v_new, **kw)
    g_cum = chunk_cumsum(g, 64, cu_seqlens)
    if output_v_new:
        return g_cum, A, o, h, ht, vn
    return g_cum, A, o, h, ht


def _forward(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens, *, cp: str = "auto",
             o_dtype: Optional[str] = None, cp_lambda: float = 0.0, cp_segment_chunks: int = 0,
             cp_warmup_chunks: int = 0, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, want_h: bool = False, want_a: bool = False,
             want_vn: bool = False):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the forward runs on GPU tensors; there is no CPU path")
    _need(q, "q", torch.bfloat16, dev)
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError(f"bad shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError(f"g and beta must be [B, T, H_v] = {(B, T, Hv)}")
    cu_host = _cu_host(cu_seqlens)
    cu_dev = None
    if cu_host is not None:
        cu_dev = cu_seqlens if (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device == dev
                                and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous()) \
            else cu_host.to(dev)
    N = (cu_host.numel() - 1) if cu_host is not None else B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (N, Hv, K, V):
            raise ValueError(f"initial_state must be [N, H_v, K, V] = {(N, Hv, K, V)}")
    if scale is None:
        scale = K ** -0.5
    if o_dtype is None:
        o_dtype = "bf16"
    desc = make_desc(B, T, Hqk, Hv, K, V, scale=scale, cu_host=cu_host, has_h0=initial_state is not None,
                     want_ht=output_final_state, o_dtype=o_dtype, cp=cp, cp_lambda=cp_lambda,
                     cp_segment_chunks=cp_segment_chunks, cp_warmup_chunks=cp_warmup_chunks)
    info = plan(desc)
    o_t = torch.float32 if o_dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty(B, T, Hv, V, dtype=o_t, device=dev)
    else:
        _need(out, "out", o_t, dev)
    ht = torch.empty(N, Hv, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    h = torch.empty(info["total_chunks"], Hv, K, V, dtype=torch.float32, device=dev) if want_h else None
    A = torch.empty(B, T, Hv, 64, dtype=torch.float32, device=dev) if want_a else None
    vn = torch.empty(info["total_chunks"], Hv, 64, V, dtype=torch.float32, device=dev) if want_vn else None
    if workspace is None or workspace.numel() < info["workspace_bytes"] or workspace.data_ptr() % 256:
        workspace = _workspace(info["workspace_bytes"], dev)
    ptrs = L.FwdPtrs(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                     initial_state.data_ptr() if initial_state is not None else None,
                     cu_dev.data_ptr() if cu_dev is not None else None,
                     out.data_ptr(), ht.data_ptr() if ht is not None else None,
                     h.data_ptr() if h is not None else None, A.data_ptr() if A is not None else None,
                     vn.data_ptr() if vn is not None else None)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        L.check(L.lib().gdn_fwd(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel(), ctypes.c_void_p(stream)))
    return out, ht, h, A, vn


def bwd_plan(desc: L.BwdDesc) -> dict:
    """Host-only planning of the backward (no GPU needed)."""
    info = L.BwdPlanInfo()
    L.check(L.lib().gdn_bwd_plan(ctypes.byref(desc), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in L.BwdPlanInfo._fields_} | {"cp": L.CP_NAMES[info.cp_mode]}


def make_bwd_desc(fwd_desc: L.FwdDesc, *, has_dht=False, grad_dtype="bf16", saved_fwd=False) -> L.BwdDesc:
    d = L.BwdDesc()
    d.fwd = fwd_desc
    d.has_dht = int(bool(has_dht))
    d.grad_dtype = {"bf16": L.GDN_DTYPE_BF16, "f32": L.GDN_DTYPE_F32}[grad_dtype]
    d.saved_fwd = int(bool(saved_fwd))
    return d


def chunk_gated_delta_rule_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                               beta: torch.Tensor, do: torch.Tensor, scale: Optional[float] = None,
                               initial_state: Optional[torch.Tensor] = None, cu_seqlens=None,
                               d_final_state: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None,
                               A: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None, *,
                               cp: str = "auto", grad_dtype: str = "bf16",
                               cp_lambda: float = 0.0, cp_segment_chunks: int = 0, cp_warmup_chunks: int = 0,
                               workspace: Optional[torch.Tensor] = None):
    """Chunked backward of ``chunk_gated_delta_rule``: the gradients of a loss
    with upstream dO (bf16 [B, T, H_v, V]) and optionally d final_state (fp32
    [N, H_v, K, V]).  ``h``, ``A`` and ``v_new`` are the low-level forward's
    chunk states, WY matrices and residuals (``chunk_gated_delta_rule_fwd`` with
    the same arguments and CP settings, ``output_v_new=True``); without them
    the backward recomputes all three.  Returns
    (dq, dk, dv, dg, dbeta, d_initial_state or None); dq, dk, dv in
    ``grad_dtype`` ("bf16" or "f32"), the rest fp32."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the backward runs on GPU tensors; there is no CPU path")
    for t, name, dt in ((q, "q", torch.bfloat16), (k, "k", torch.bfloat16), (v, "v", torch.bfloat16),
                        (g, "g", torch.float32), (beta, "beta", torch.float32), (do, "dO", torch.bfloat16)):
        _need(t, name, dt, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2] or do.shape != v.shape:
        raise ValueError(f"bad shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)} dO {tuple(do.shape)}")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError(f"g and beta must be [B, T, H_v] = {(B, T, Hv)}")
    cu_host = _cu_host(cu_seqlens)
    cu_dev = None
    if cu_host is not None:
        cu_dev = cu_seqlens if (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device == dev
                                and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous()) \
            else cu_host.to(dev)
    N = (cu_host.numel() - 1) if cu_host is not None else B
    for t, name in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if t.shape != (N, Hv, K, V):
                raise ValueError(f"{name} must be [N, H_v, K, V] = {(N, Hv, K, V)}")
    if not ((h is None) == (A is None) == (v_new is None)):
        raise ValueError("h, A and v_new must be given together")
    if scale is None:
        scale = K ** -0.5
    fd = make_desc(B, T, Hqk, Hv, K, V, scale=scale, cu_host=cu_host, has_h0=initial_state is not None,
                   cp=cp, cp_lambda=cp_lambda, cp_segment_chunks=cp_segment_chunks,
                   cp_warmup_chunks=cp_warmup_chunks)
    desc = make_bwd_desc(fd, has_dht=d_final_state is not None, grad_dtype=grad_dtype, saved_fwd=h is not None)
    info = bwd_plan(desc)
    if h is not None:
        _need(h, "h", torch.float32, dev)
        _need(A, "A", torch.float32, dev)
        _need(v_new, "v_new", torch.float32, dev)
        if h.shape != (info["total_chunks"], Hv, K, V) or A.shape != (B, T, Hv, 64) \
                or v_new.shape != (info["total_chunks"], Hv, 64, V):
            raise ValueError("h / A / v_new do not match the forward's low-level output shapes")
    gt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq = torch.empty(B, T, Hqk, K, dtype=gt, device=dev)
    dk = torch.empty(B, T, Hqk, K, dtype=gt, device=dev)
    dv = torch.empty(B, T, Hv, V, dtype=gt, device=dev)
    dg = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    dbeta = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    dh0 = torch.empty(N, Hv, K, V, dtype=torch.float32, device=dev) if initial_state is not None else None
    if workspace is None or workspace.numel() < info["workspace_bytes"] or workspace.data_ptr() % 256:
        workspace = _workspace(info["workspace_bytes"], dev)
    opt = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    ptrs = L.BwdPtrs(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), opt(initial_state),
                     opt(cu_dev), do.data_ptr(), opt(d_final_state), opt(h), opt(A), opt(v_new), dq.data_ptr(),
                     dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), dbeta.data_ptr(), opt(dh0))
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        L.check(L.lib().gdn_bwd(ctypes.byref(desc), ctypes.byref(ptrs), ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel(), ctypes.c_void_p(stream)))
    return dq, dk, dv, dg, dbeta, dh0


class _GDNFunction(torch.autograd.Function):
    """Autograd node: the forward keeps h and A (the low-level outputs), the
    backward hands them to gdn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, scale, output_final_state, cu_seqlens, kw):
        o, ht, h, A, vn = _forward(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                                   want_h=True, want_a=True, want_vn=True, **kw)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, h, A, vn)
        ctx.scale, ctx.cu_seqlens, ctx.kw = scale, cu_seqlens, kw
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g, beta, initial_state, h, A, vn = ctx.saved_tensors
        kw = {n: ctx.kw[n] for n in ("cp", "cp_lambda", "cp_segment_chunks", "cp_warmup_chunks")}
        dq, dk, dv, dg, dbeta, dh0 = chunk_gated_delta_rule_bwd(
            q, k, v, g, beta, do.to(torch.bfloat16).contiguous(), ctx.scale, initial_state, ctx.cu_seqlens,
            None if dht is None else dht.float().contiguous(), h, A, vn, **kw)
        return dq, dk, dv, dg, dbeta, dh0, None, None, None, None


class PreparedForward:
    """A validated forward call with its outputs and workspace allocated once;
    ``__call__`` only enqueues gdn_fwd on the current stream (benchmark loops,
    repeated calls on fixed shapes)."""

    def __init__(self, q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                 cu_seqlens=None, **kw):
        self.o, self.final_state = chunk_gated_delta_rule(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                                                          output_final_state=output_final_state,
                                                          cu_seqlens=cu_seqlens, **kw)
        cu_host = _cu_host(cu_seqlens)
        B, T, Hqk, K = q.shape
        Hv, V = v.shape[2], v.shape[3]
        self._keep = (q, k, v, g, beta, initial_state, cu_host)
        self.desc = make_desc(B, T, Hqk, Hv, K, V, scale=scale if scale is not None else K ** -0.5,
                              cu_host=cu_host, has_h0=initial_state is not None, want_ht=output_final_state,
                              o_dtype=kw.get("o_dtype") or "bf16", cp=kw.get("cp", "auto"),
                              cp_lambda=kw.get("cp_lambda", 0.0), cp_segment_chunks=kw.get("cp_segment_chunks", 0),
                              cp_warmup_chunks=kw.get("cp_warmup_chunks", 0))
        self.info = plan(self.desc)
        self.workspace = _workspace(self.info["workspace_bytes"], q.device)
        self.cu_dev = None if cu_host is None else cu_host.to(q.device)
        self.ptrs = L.FwdPtrs(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                              initial_state.data_ptr() if initial_state is not None else None,
                              self.cu_dev.data_ptr() if self.cu_dev is not None else None,
                              self.o.data_ptr(), self.final_state.data_ptr() if self.final_state is not None else None)
        self.device = q.device

    def __call__(self):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        L.check(L.lib().gdn_fwd(ctypes.byref(self.desc), ctypes.byref(self.ptrs),
                                ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                ctypes.c_void_p(stream)))
        return self.o, self.final_state


def chunk_cumsum(g: torch.Tensor, chunk: int = 64, cu_seqlens=None, out: Optional[torch.Tensor] = None):
    """Chunk-local running sum of g [B, T, H] (fp32), restarting at every chunk
    and sequence start: the transformed g of the pages' low-level forward."""
    dev = g.device
    if dev.type != "cuda":
        raise ValueError("chunk_cumsum runs on a GPU tensor")
    _need(g, "g", torch.float32, dev)
    B, T, H = g.shape
    cu_dev, N = None, B
    if cu_seqlens is not None:
        cu_host = _cu_host(cu_seqlens)  # a device tensor is copied to the host once (a sync)
        _check_offsets(cu_host, B, T)
        cu_dev = cu_host.to(dev)
        N = cu_host.numel() - 1
    if out is None:
        out = torch.empty_like(g)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        L.check(L.lib().gdn_chunk_cumsum(ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(out.data_ptr()), B, T, H,
                                         int(chunk), ctypes.c_void_p(cu_dev.data_ptr()) if cu_dev is not None
                                         else None, N, ctypes.c_void_p(stream)))
    return out


__all__: Sequence[str] = ("chunk_gated_delta_rule", "chunk_gated_delta_rule_fwd", "chunk_cumsum", "plan", "make_desc",
                          "PreparedForward")


class PreparedForwardBackward:
    """A training step on fixed shapes with every buffer allocated once: the
    forward (o, final_state, and the low-level h and A it keeps for the
    backward) then the backward (dq, dk, dv, dg, dbeta, d initial_state) from
    upstream dO and d final_state.  ``forward()`` and ``backward()`` only
    enqueue gdn_fwd / gdn_bwd on the current stream."""

    def __init__(self, q, k, v, g, beta, do, scale=None, initial_state=None, d_final_state=None, cu_seqlens=None,
                 *, cp="auto", grad_dtype="bf16", **kw):
        dev = q.device
        self.device = dev
        _, A, o, h, ht, vn = chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                                                        cu_seqlens=cu_seqlens, output_final_state=True,
                                                        output_v_new=True, cp=cp, **kw)
        self.o, self.final_state, self.h, self.A, self.v_new = o, ht, h, A, vn
        self.grads = chunk_gated_delta_rule_bwd(q, k, v, g, beta, do, scale=scale, initial_state=initial_state,
                                                cu_seqlens=cu_seqlens, d_final_state=d_final_state, h=h, A=A,
                                                v_new=vn, cp=cp, grad_dtype=grad_dtype, **kw)
        cu_host = _cu_host(cu_seqlens)
        B, T, Hqk, K = q.shape
        Hv, V = v.shape[2], v.shape[3]
        sc = scale if scale is not None else K ** -0.5
        self.fdesc = make_desc(B, T, Hqk, Hv, K, V, scale=sc, cu_host=cu_host, has_h0=initial_state is not None,
                               want_ht=True, cp=cp, **kw)
        self.bdesc = make_bwd_desc(make_desc(B, T, Hqk, Hv, K, V, scale=sc, cu_host=cu_host,
                                             has_h0=initial_state is not None, cp=cp, **kw),
                                   has_dht=d_final_state is not None, grad_dtype=grad_dtype, saved_fwd=True)
        self.finfo, self.binfo = plan(self.fdesc), bwd_plan(self.bdesc)
        self.fws = _workspace(self.finfo["workspace_bytes"], dev)
        self.bws = _workspace(self.binfo["workspace_bytes"], dev)
        self.cu_dev = None if cu_host is None else cu_host.to(dev)
        self._keep = (q, k, v, g, beta, do, initial_state, d_final_state, cu_host)
        opt = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        self.fptrs = L.FwdPtrs(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                               opt(initial_state), opt(self.cu_dev), o.data_ptr(), ht.data_ptr(), h.data_ptr(),
                               A.data_ptr(), vn.data_ptr())
        dq, dk, dv, dg, db, dh0 = self.grads
        self.bptrs = L.BwdPtrs(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                               opt(initial_state), opt(self.cu_dev), do.data_ptr(), opt(d_final_state), h.data_ptr(),
                               A.data_ptr(), vn.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                               dg.data_ptr(), db.data_ptr(), opt(dh0))

    def forward(self):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        L.check(L.lib().gdn_fwd(ctypes.byref(self.fdesc), ctypes.byref(self.fptrs),
                                ctypes.c_void_p(self.fws.data_ptr()), self.fws.numel(), ctypes.c_void_p(stream)))

    def backward(self):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        L.check(L.lib().gdn_bwd(ctypes.byref(self.bdesc), ctypes.byref(self.bptrs),
                                ctypes.c_void_p(self.bws.data_ptr()), self.bws.numel(), ctypes.c_void_p(stream)))

    def __call__(self):
        self.forward()
        self.backward()
        return self.grads

