"""Seeded synthetic workloads for the GDN chunked-prefill forward.

This module only draws inputs; it holds none of the method's arithmetic, so
the tests, the benchmark and the oracle can all take their inputs from it.

Shapes and distributions follow the pages' problem statement (aisparkup.com
FlashQLA wiki, "high-level API": q,k [B,T,H_q,K], v [B,T,H_v,V], g and beta
[B,T,H_v], optional initial state and cu_seqlens) and their benchmark
workloads (agentlenshq.com FlashQLA blog, "performance benchmarks" table:
batch 1 x 32768 tokens at the per-GPU head counts of TP shards).  There is no
public dataset behind those numbers; random activations of the same shapes
stand in for them:

* q, k: N(0,1) in float32, L2-normalised per (token, head) in float32, then
  rounded to bfloat16 (round-to-nearest-even).
* v: N(0,1) rounded to bfloat16.
* g: logsigmoid(N(mu, 1)) in float32 (log-decay < 0), mu = 2 or 3.
* beta: sigmoid(N(0,1)) in float32.
* initial_state: N(0, 0.1^2) float32 [N, H_v, K, V] when the workload has one.
* backward workload: dO N(0,1) rounded to bfloat16, d(final_state) N(0, 0.01^2)
  float32 (the second argument of N(0, s) read as a standard deviation, as
  for the initial state).
* varlen lengths: log-uniform in [512, 16384], rescaled to the token total.

Every draw comes from ``torch.Generator().manual_seed(seed)`` on the CPU in the
fixed order q, k, v, g-logit, beta-logit, initial_state, dO, d(final_state);
varlen lengths come first, from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int
    H_qk: int
    H_v: int
    K: int = 128
    V: int = 128
    g_mu: float = 2.0
    h0_std: Optional[float] = None  # None -> zero initial state
    want_ht: bool = True
    num_seqs: int = 0  # >0: varlen with this many packed sequences (B must be 1)
    len_lo: int = 512
    len_hi: int = 16384
    with_grads: bool = False
    cp: tuple = field(default=("auto",))  # context-parallel variants exercised

    @property
    def scale(self) -> float:
        return self.K ** -0.5

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads; index = position in the build's configuration list.
WORKLOADS = {
    # tiny parity case that the oracle finishes in well under a second
    "gdn_fwd_1x512_h2x2": Workload("gdn_fwd_1x512_h2x2", 1000, B=1, T=512, H_qk=2, H_v=2,
                                   g_mu=2.0, h0_std=None),
    # small-model TP1 shard: 16 qk heads, 16 v heads
    "gdn_fwd_1x32768_h16x16": Workload("gdn_fwd_1x32768_h16x16", 1001, B=1, T=32768, H_qk=16, H_v=16,
                                       g_mu=2.0, h0_std=0.1),
    # TP8 shard of a large model: 2 qk heads, 8 v heads; few chains -> context parallelism
    "gdn_fwd_1x32768_h2x8": Workload("gdn_fwd_1x32768_h2x8", 1002, B=1, T=32768, H_qk=2, H_v=8,
                                     g_mu=3.0, h0_std=0.1, cp=("exact", "warmup")),
    # varlen packed batch: 16 sequences, 65536 tokens, 8 qk heads, 24 v heads
    "gdn_fwd_varlen16_65536_h8x24": Workload("gdn_fwd_varlen16_65536_h8x24", 1003, B=1, T=65536,
                                             H_qk=8, H_v=24, g_mu=2.0, h0_std=0.1, num_seqs=16),
    # forward + backward case (backward is a later stage)
    "gdn_fwdbwd_1x32768_h4x16": Workload("gdn_fwdbwd_1x32768_h4x16", 1004, B=1, T=32768, H_qk=4, H_v=16,
                                         g_mu=2.0, h0_std=0.1, with_grads=True),
}
WORKLOAD_ORDER = list(WORKLOADS)


def varlen_lengths(rng: np.random.Generator, n: int, total: int, lo: int, hi: int) -> np.ndarray:
    """n lengths, log-uniform in [lo, hi], rescaled so that they sum to total.

    Recipe: draw lo * (hi/lo)**U, then alternately rescale to the total and
    clip to [lo, hi] until stable; floor; give the integer residual to the
    longest sequences that still have room below hi.
    """
    if n * lo > total or n * hi < total:
        raise ValueError("varlen_lengths: total not reachable within [lo, hi]")
    x = lo * (hi / lo) ** rng.random(n)
    for _ in range(100):
        y = np.clip(x * (total / x.sum()), lo, hi)
        if np.allclose(y, x, rtol=0, atol=1e-9):
            break
        x = y
    out = np.floor(x).astype(np.int64)
    resid = int(total - out.sum())
    for idx in np.argsort(-out, kind="stable"):
        if resid == 0:
            break
        room = min(hi - int(out[idx]), resid) if resid > 0 else max(lo - int(out[idx]), resid)
        out[idx] += room
        resid -= room
    assert int(out.sum()) == total and out.min() >= lo and out.max() <= hi
    return out


def _unit_bf16(x: torch.Tensor) -> torch.Tensor:
    """Per-(token, head) L2 normalisation in float32, then bf16 rounding (caller-side
    input preparation; the method itself does no normalisation)."""
    return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", T: Optional[int] = None, num_seqs: Optional[int] = None,
                lengths=None) -> dict:
    """Draw the workload's inputs on the CPU, then move them to ``device``.

    ``T`` overrides the token count (for reduced-size parity runs), ``lengths``
    forces explicit varlen lengths.  Returns a dict with q, k, v (bf16), g,
    beta (fp32), initial_state (fp32 or None), cu_seqlens (int32 CPU tensor or
    None), scale, and dO / dht when the workload has gradients.
    """
    T = w.T if T is None else int(T)
    ns = w.num_seqs if num_seqs is None else int(num_seqs)
    cu = None
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
    elif ns > 0:
        rng = np.random.default_rng(w.seed)
        lo = min(w.len_lo, T // ns)
        hi = max(min(w.len_hi, T), -(-T // ns))
        lens = varlen_lengths(rng, ns, T, lo, hi)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    B = 1 if cu is not None else w.B
    N = (len(cu) - 1) if cu is not None else B
    gen = torch.Generator().manual_seed(w.seed)
    q = _unit_bf16(torch.randn(B, T, w.H_qk, w.K, generator=gen))
    k = _unit_bf16(torch.randn(B, T, w.H_qk, w.K, generator=gen))
    v = torch.randn(B, T, w.H_v, w.V, generator=gen).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(torch.randn(B, T, w.H_v, generator=gen) + w.g_mu)
    beta = torch.sigmoid(torch.randn(B, T, w.H_v, generator=gen))
    h0 = None
    if w.h0_std is not None:
        h0 = torch.randn(N, w.H_v, w.K, w.V, generator=gen) * w.h0_std
    out = dict(q=q, k=k, v=v, g=g.float(), beta=beta.float(), initial_state=h0,
               cu_seqlens=None if cu is None else torch.from_numpy(cu), scale=w.scale)
    if w.with_grads:
        out["dO"] = torch.randn(B, T, w.H_v, w.V, generator=gen).to(torch.bfloat16)
        out["dht"] = torch.randn(N, w.H_v, w.K, w.V, generator=gen) * 0.01
    if device != "cpu":
        for key, val in list(out.items()):
            if isinstance(val, torch.Tensor) and key != "cu_seqlens":
                out[key] = val.to(device)
    return out


def random_inputs(B, T, H_qk, H_v, K=128, V=128, seed=0, g_mu=2.0, h0_std=None, lengths=None,
                  device="cpu") -> dict:
    """Same recipe at arbitrary shapes (parity sweeps, edge cases)."""
    w = Workload(f"custom_{seed}", seed, B=B, T=T, H_qk=H_qk, H_v=H_v, K=K, V=V, g_mu=g_mu,
                 h0_std=h0_std)
    return make_inputs(w, device=device, lengths=lengths)


def to_f32_numpy(x):
    """Exact float32 copy of a (bf16 or fp32) tensor for the oracle."""
    if x is None:
        return None
    return x.detach().to("cpu", torch.float32).numpy()


def reduced(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def device_inputs(B, T, H_qk, H_v, K=128, V=128, seed=0, g_mu=2.0, h0_std=0.1, device="cuda:0") -> dict:
    """The same recipe drawn directly on the device (timing sweeps over large
    shapes, where a CPU draw would dominate the run; values differ from
    make_inputs' CPU draw)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    q = _unit_bf16(torch.randn(B, T, H_qk, K, generator=gen, device=device))
    k = _unit_bf16(torch.randn(B, T, H_qk, K, generator=gen, device=device))
    v = torch.randn(B, T, H_v, V, generator=gen, device=device).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(torch.randn(B, T, H_v, generator=gen, device=device) + g_mu)
    beta = torch.sigmoid(torch.randn(B, T, H_v, generator=gen, device=device))
    h0 = None if h0_std is None else torch.randn(B, H_v, K, V, generator=gen, device=device) * h0_std
    return dict(q=q, k=k, v=v, g=g.float(), beta=beta.float(), initial_state=h0, cu_seqlens=None, scale=K ** -0.5)
