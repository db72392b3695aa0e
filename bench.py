#!/usr/bin/env python3
"""Benchmark: GDN chunked-prefill forward on one MI355X.

One step = one gdn_fwd call (the whole forward: every chunk of every v-head,
o and final_state) over the 1 x 32768-token, 16 qk / 16 v-head workload, with
inputs resident in HBM.  Prints ONE JSON line on stdout:

  value        tokens per second: tokens per step over ms_per_step
  ms_per_step  mean duration of one forward (HIP events on the launch stream
               around each call); before every timed call the bench writes a
               1 GiB buffer (four times the 256 MB Infinity Cache), so each
               call reads its inputs from HBM, as a call inside a model would
  roofline     the forward kernel's algorithmic HBM bytes per launch over its
               mean launch duration, against the 8 TB/s HBM peak; `traffic` =
               measured HBM bytes per launch from rocprofv3 FETCH_SIZE +
               WRITE_SIZE (scaled by a copy-kernel calibration) when the stored
               counters match the current kernel source, else null
  mfma         the forward's algorithmic MFMA flops over the same duration,
               against the published 2.5 PFLOP/s bf16 peak and against the
               rate a probe kernel of the same MFMA instruction sustains on this GPU
  cpu_baseline the fp64 oracle on a bounded prefix of the same workload, timed
               on this host's cores
Before the warm-up steps the bench writes the flush buffer for about 0.3 s,
which brings the GPU's clocks out of idle (untimed).

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload NAME]
       [--cp auto|warmup|off] [--no-cpu-baseline] [--cpu-seconds 10]
       python bench.py --sweep [--steps 200] [--warmup 100] [--cp auto]   (head-setting sweep)
       python bench.py --sweep-bwd [--steps 200] [--warmup 100]   (training step against total tokens)
       python bench.py --workload gdn_fwdbwd_1x32768_h4x16   (training step: forward keeping h and A,
              then the backward; roofline of the backward against the bf16 MFMA peak)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 1 << 30
SETTLE_S = 0.3
# Pages' FlashQLA forward latency for this exact workload (1 x 32768, h_qk=16, h_v=16)
# on an NVIDIA H200 (agentlenshq.com FlashQLA blog, benchmark table): context only.
PAGES_MS = {"gdn_fwd_1x32768_h16x16": 0.493, "gdn_fwd_1x32768_h2x8": 0.310}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_deltanet_chunked_chunk_amd", "csrc", f)
                  for f in ("gdn_fwd.hip", "gdn_internal.h", "gdn_window.h")] + [
                  os.path.join(ROOT, "gated_deltanet_chunked_chunk_amd", "build.py")]  # its code-generation options


# the training step's kernels: the forward (keeping h, A, v') and the backward
BWD_SOURCES = KERNEL_SOURCES + [os.path.join(ROOT, "gated_deltanet_chunked_chunk_amd", "csrc", "gdn_bwd.hip")]
# (role, kernel name) of each kernel of one training step whose HBM bytes are stored
TRAINING_KERNELS = (("forward", "gdn_fwd_main_kernel"), ("reverse", "gdn_bwd_dh_kernel"),
                    ("local", "gdn_bwd_local_kernel"))


def is_training(workload: str) -> bool:
    return workload.startswith("gdn_fwdbwd")


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in (sources or KERNEL_SOURCES):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def workload_source_hash(workload: str) -> str:
    return kernel_source_hash(BWD_SOURCES if is_training(workload) else None)


def algorithmic_bytes(x) -> int:
    """HBM bytes the forward must move at minimum: read q, k, v (bf16), g, beta
    (fp32), initial_state (fp32) once; write o (bf16) and final_state (fp32) once."""
    q, v, g = x["q"], x["v"], x["g"]
    n = q.numel() * 2 * 2 + v.numel() * 2 * 2 + g.numel() * 4 * 2
    if x["initial_state"] is not None:
        n += x["initial_state"].numel() * 4 * 2  # h0 read + final_state write
    return int(n)


def bwd_algorithmic(x) -> tuple:
    """Backward bytes and flops at minimum.  Bytes: read q, k, v, dO (bf16), g,
    beta (fp32), initial_state and d final_state (fp32) once; write dq, dk, dv
    (bf16), dg, dbeta, d initial_state (fp32) once.  Flops: every distinct
    product of the chunked backward once per (chunk, v-head), counted as 2 m n k
    (reverse pass: P^T dO, K dh', Q~^T dO, W^T dv'; chunk-local: W, Q K^T,
    T diag(beta) V, W h, dO v'^T, dPm K, dO h^T, dPm^T Q, v' dh'^T, dv' h^T,
    dW K^T, dv' V^T, T^T dW, T^T dv', T^T dT, (T^T dT) T^T, K K^T, M K, M^T K),
    no hi/lo split terms; the forward's h and A are inputs, not recomputed."""
    q, v, g = x["q"], x["v"], x["g"]
    n = q.numel() * 2 * 2 * 2 + v.numel() * 2 * 3 + g.numel() * 4 * 4  # q, k, dq, dk; v, dO, dv; g, beta, dg, dbeta
    if x["initial_state"] is not None:
        n += x["initial_state"].numel() * 4 * 2
    if x.get("dht") is not None:
        n += x["dht"].numel() * 4
    B, T, Hv, V = v.shape
    K = q.shape[-1]
    C = 64
    chunk_heads = B * (-(-T // C)) * Hv
    mm = lambda m, nn, k: 2 * m * nn * k  # noqa: E731
    reverse = mm(C, V, C) + mm(C, V, K) + mm(K, V, C) + mm(K, V, C)
    local = (mm(C, K, C) + mm(C, C, K) + mm(C, V, C) + mm(C, V, K) + mm(C, C, V) + mm(C, K, C) + mm(C, K, V)
             + mm(C, K, C) + mm(C, K, V) + mm(C, K, V) + mm(C, C, K) + mm(C, C, V) + mm(C, K, C) + mm(C, V, C)
             + mm(C, C, C) + mm(C, C, C) + mm(C, C, K) + mm(C, K, C) + mm(C, K, C))
    return int(n), int(chunk_heads * (reverse + local))


def traffic_key(workload: str, cp: str) -> str:
    return workload if cp == "auto" else f"{workload}:{cp}"


def stored_traffic_entry(workload: str, cp: str = "auto"):
    """The stored counter entry of a workload, or None once its kernels changed."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = d.get(traffic_key(workload, cp))
    if not e or e.get("kernel_source_sha") != workload_source_hash(workload):
        return None
    return e


def stored_traffic(workload: str, cp: str = "auto"):
    e = stored_traffic_entry(workload, cp)
    return None if e is None else e.get("bytes_per_launch")


def _counter_mean(csv_path: str, counter: str, kernel_substr: str) -> float:
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} rows for '{kernel_substr}' in {csv_path}")
    return sum(vals) / len(vals)


def ingest_counters(workload: str, cp: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of the
    forward and of the 1 GiB copy calibration into HBM bytes per launch, and
    store them with the hash of the kernel source they were taken on."""
    gib = float(1 << 30)
    f_fac = gib / (_counter_mean(copy_fetch_csv, "FETCH_SIZE", "copyBuffer") * 1024.0)
    w_fac = gib / (_counter_mean(copy_write_csv, "WRITE_SIZE", "copyBuffer") * 1024.0)
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        d = {}
    key = traffic_key(workload, cp)
    if is_training(workload):
        # per kernel of the step; bytes_per_launch is one backward call (reverse
        # pass + chunk-local gradients), the forward with saved tensors apart
        kern = {}
        for role, name in TRAINING_KERNELS:
            fetch = _counter_mean(fetch_csv, "FETCH_SIZE", name) * 1024.0 * f_fac
            write = _counter_mean(write_csv, "WRITE_SIZE", name) * 1024.0 * w_fac
            kern[role] = {"kernel": name, "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write))}
        bwd = sum(kern[r]["fetch_bytes"] + kern[r]["write_bytes"] for r in ("reverse", "local"))
        d[key] = {"bytes_per_launch": int(bwd), "kernels": kern, "fetch_scale": round(f_fac, 4),
                  "write_scale": round(w_fac, 4), "kernel_source_sha": workload_source_hash(workload)}
    else:
        fetch = _counter_mean(fetch_csv, "FETCH_SIZE", "gdn_fwd_main_kernel") * 1024.0 * f_fac
        write = _counter_mean(write_csv, "WRITE_SIZE", "gdn_fwd_main_kernel") * 1024.0 * w_fac
        d[key] = {"bytes_per_launch": int(round(fetch + write)), "fetch_bytes": int(round(fetch)),
                  "write_bytes": int(round(write)), "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4),
                  "kernel_source_sha": workload_source_hash(workload)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(d, open(TRAFFIC_FILE, "w"), indent=2, sort_keys=True)
    print(json.dumps(d[key]))


class Flusher:
    """A 1 GiB device buffer, rewritten before every timed call so that no input
    of the call is still in the 256 MB Infinity Cache (or the L2)."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n & 7))

    def settle(self, work=None, seconds: float = SETTLE_S):
        """Untimed, before the warm-up steps: run `work` (the measured call
        itself), each time after a flush, for `seconds`, so that the clocks
        reach the state they hold under this load.  Measured: after a settle
        that only writes the flush buffer, the first 20 timed calls of the
        16/16-head forward averaged 0.234 ms against 0.220 ms at steady state;
        after a settle on the call itself, 0.220 ms from the first call."""
        import torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                self()
                if work is not None:
                    work()
            torch.cuda.synchronize()


def time_steps(fns, steps: int, flush, stream):
    """Run `steps` steps; each step flushes the caches, then runs the callables
    in `fns` in order, each bracketed by HIP events on `stream`.  Returns the
    per-step durations of each callable (ms) and the wall time of the whole
    timed region (flushes included), bracketed by device synchronisation."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        flush()
        e[0].record(stream)
        for i, fn in enumerate(fns):
            fn()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[e[i].elapsed_time(e[i + 1]) for e in ev] for i in range(len(fns))]
    return per, wall


MFMA_BF16_PEAK_TFLOPS = 2500.0
PROBE_LIB = os.path.join(ROOT, "gated_deltanet_chunked_chunk_amd", "libgdn_probe.so")


def measured_mfma_peak(dev) -> float:
    """bf16 MFMA rate (TFLOP/s) the probe kernel sustains: v_mfma_f32_16x16x32_bf16
    in eight independent chains per wave, four waves per block, 1024 blocks;
    the best of ten launches after three untimed ones."""
    import ctypes
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_mfma_bf16.restype = ctypes.c_int
    lib.probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    blocks, iters = 1024, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for i in range(13):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), blocks, iters, ctypes.c_void_p(stream.cuda_stream))
        b.record(stream)
        if rc != 0:
            raise RuntimeError(f"MFMA probe launch failed ({rc})")
        torch.cuda.synchronize()
        if i >= 3:
            best = max(best, lib.probe_mfma_bf16_flops(blocks, iters) / (a.elapsed_time(b) * 1e-3) / 1e12)
    return best


def measured_gemm_rate(dev) -> float:
    """bf16 rate (TFLOP/s) of a large library GEMM (torch.matmul, 8192^3, on
    hipBLASLt): what a plain dense product reaches on this GPU; the best of five
    calls after two untimed ones."""
    import torch
    n = 8192
    gen = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, generator=gen).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=gen).to(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for i in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        c = torch.matmul(a, b)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            best = max(best, 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    del a, b, c
    return best


def fwd_flops(x) -> int:
    """Algorithmic MFMA flops of the forward: 2 (3 C K + 2 C V + 3 K V) per token
    and v-head (K K^T, W, Q K^T; U, P v'; W h, K^T v', Q h at chunk C = 64)."""
    v, q = x["v"], x["q"]
    K, V, C = q.shape[-1], v.shape[-1], 64
    tokens = v.shape[0] * v.shape[1]
    return int(2 * (3 * C * K + 2 * C * V + 3 * K * V) * tokens * v.shape[2])


def cpu_baseline(x, w, target_s: float):
    import numpy as np  # noqa: F401
    import oracle
    from gated_deltanet_chunked_chunk_amd import workloads as W
    threads = min(16, oracle.default_threads())
    host = {k: W.to_f32_numpy(x[k]) for k in ("q", "k", "v", "g", "beta", "initial_state")}

    def run(T):
        t0 = time.perf_counter()
        oracle.fwd(host["q"][:, :T], host["k"][:, :T], host["v"][:, :T], host["g"][:, :T], host["beta"][:, :T],
                   scale=x["scale"], initial_state=host["initial_state"], n_threads=threads)
        return time.perf_counter() - t0

    t_cal = run(256)
    T = int(min(w.T, max(256, 256 * target_s / max(t_cal, 1e-6))))
    T = max(256, T // 64 * 64)
    dt = run(T)
    return {"value": T * w.B / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {T} of {w.T} tokens, all {w.H_v} v-heads, fp64 per-token recurrence, {dt:.1f} s"}


# The pages' head settings at their tensor-parallel shares (blog, benchmark
# table; wiki, benchmarks: h in {64, 48, 32, 24, 16, 8} over TP1..TP8): per-GPU
# (H_qk, H_v) and the full layer's heads / TP degree they stand for.
SWEEP_HEADS = [((2, 8), "16/64 heads, TP8"), ((4, 16), "16/64 heads, TP4"), ((8, 32), "16/64 heads, TP2"),
               ((16, 64), "16/64 heads, TP1"), ((8, 24), "16/48 heads, TP2"), ((16, 48), "16/48 heads, TP1"),
               ((16, 16), "16/16 heads, TP1")]
SWEEP_SHAPES = [(1, 8192), (1, 32768), (4, 32768), (1, 131072)]
# pages' H200 FlashQLA forward latency at 1 x 32768 (blog, benchmark table): context only
PAGES_H200_MS = {(2, 8): 0.310, (4, 16): 0.486, (8, 24): 0.659, (16, 16): 0.493}


def sweep(steps: int, warmup: int, cp: str):
    """Forward latency over the pages' head settings and several batch lengths:
    one JSON line per case, then a markdown table on stderr."""
    import torch
    from gated_deltanet_chunked_chunk_amd import PreparedForward
    from gated_deltanet_chunked_chunk_amd import workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = Flusher(dev)
    flush.settle()
    rows = []
    for (hqk, hv), model in SWEEP_HEADS:
        for B, T in SWEEP_SHAPES:
            x = W.device_inputs(B, T, hqk, hv, seed=1000 + hqk * 100 + hv, device=dev)
            call = PreparedForward(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                   initial_state=x["initial_state"], output_final_state=True, cp=cp)
            flush.settle(call, seconds=0.1)  # the clocks under this case's load
            for _ in range(warmup):
                flush()
                call()
            stream = torch.cuda.current_stream(dev)
            (per,), _ = time_steps([call], steps, flush, stream)
            ms = sum(per) / len(per)
            alg = algorithmic_bytes(x)
            frac = alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
            ref = PAGES_H200_MS.get((hqk, hv)) if (B, T) == (1, 32768) else None
            line = {"model": model, "H_qk": hqk, "H_v": hv, "B": B, "T": T, "cp": call.info["cp"],
                    "segment_chunks": call.info["segment_chunks"], "workgroups": call.info["workgroups"],
                    "ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                    "hbm_roofline_frac": round(frac, 4), "pages_h200_ms": ref}
            print(json.dumps(line), flush=True)
            rows.append(line)
            del call, x
            torch.cuda.empty_cache()
    print("| layer heads / TP | H_qk | H_v | B x T | CP (L, workgroups) | ms | M tokens/s | HBM roofline | pages H200 ms |",
          file=sys.stderr)
    print("|---|---|---|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {r['model']} | {r['H_qk']} | {r['H_v']} | {r['B']} x {r['T']} | {r['cp']} ({r['segment_chunks']}, "
              f"{r['workgroups']}) | {r['ms']:.3f} | {r['tokens_per_s'] / 1e6:.1f} | {r['hbm_roofline_frac']:.3f} | "
              f"{r['pages_h200_ms'] if r['pages_h200_ms'] else ''} |", file=sys.stderr)


def cpu_baseline_bwd(x, w, target_s: float):
    """The oracle's forward + reverse-mode backward on a prefix of the workload."""
    import oracle
    from gated_deltanet_chunked_chunk_amd import workloads as W
    threads = min(16, oracle.default_threads())
    host = {k: W.to_f32_numpy(x[k]) for k in ("q", "k", "v", "g", "beta", "initial_state", "dO", "dht")}

    def run(T):
        t0 = time.perf_counter()
        args = [host[n][:, :T] for n in ("q", "k", "v", "g", "beta")]
        oracle.fwd(*args, scale=x["scale"], initial_state=host["initial_state"], n_threads=threads)
        oracle.bwd(*args, host["dO"][:, :T], host["dht"], scale=x["scale"], initial_state=host["initial_state"],
                   n_threads=threads)
        return time.perf_counter() - t0

    t_cal = run(256)
    T = int(min(w.T, max(256, 256 * target_s / max(t_cal, 1e-6))))
    T = max(256, T // 64 * 64)
    dt = run(T)
    return {"value": T * w.B / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {T} of {w.T} tokens, all {w.H_v} v-heads, fp64 per-token forward + reverse-mode "
                      f"backward, {dt:.1f} s"}


SWEEP_BWD_TOKENS = [(1, 8192), (1, 32768), (4, 32768), (1, 131072)]


def sweep_bwd(steps: int, warmup: int, cp: str):
    """Training-step latency (the forward keeping h, A and v', then the
    backward) against total tokens over the pages' head settings: one JSON line
    per case, then a markdown table on stderr.  Inputs: the forward's sweep
    inputs plus dO N(0, 1) rounded to bfloat16 and d final_state N(0, 0.01^2),
    drawn on the device from a seeded generator."""
    import torch
    from gated_deltanet_chunked_chunk_amd import PreparedForwardBackward
    from gated_deltanet_chunked_chunk_amd import workloads as W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = Flusher(dev)
    flush.settle()
    rows = []
    for (hqk, hv), model in SWEEP_HEADS:
        for B, T in SWEEP_BWD_TOKENS:
            seed = 2000 + hqk * 100 + hv
            x = W.device_inputs(B, T, hqk, hv, seed=seed, device=dev)
            gen = torch.Generator(device=dev).manual_seed(seed)
            V, K = x["v"].shape[-1], x["q"].shape[-1]
            x["dO"] = torch.randn(B, T, hv, V, generator=gen, device=dev).to(torch.bfloat16)
            x["dht"] = torch.randn(B, hv, K, V, generator=gen, device=dev) * 0.01
            call = PreparedForwardBackward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["dO"], scale=x["scale"],
                                           initial_state=x["initial_state"], d_final_state=x["dht"], cp=cp)
            flush.settle(call, seconds=0.1)  # the clocks under this case's load
            for _ in range(warmup):
                flush()
                call()
            stream = torch.cuda.current_stream(dev)
            (pf, pb), _ = time_steps([call.forward, call.backward], steps, flush, stream)
            fwd_ms = sum(pf) / steps
            bwd_ms = sum(pb) / steps
            _, flops = bwd_algorithmic(x)
            frac = flops / (bwd_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
            line = {"model": model, "H_qk": hqk, "H_v": hv, "B": B, "T": T, "total_tokens": B * T,
                    "bwd_cp": call.binfo["cp"], "bwd_segment_chunks": call.binfo["segment_chunks"],
                    "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "step_ms": round(fwd_ms + bwd_ms, 4),
                    "step_tokens_per_s": round(B * T / ((fwd_ms + bwd_ms) * 1e-3), 1),
                    "bwd_mfma_frac": round(frac, 4)}
            print(json.dumps(line), flush=True)
            rows.append(line)
            del call, x
            torch.cuda.empty_cache()
    print("| layer heads / TP | H_qk | H_v | B x T | reverse-pass CP (L) | forward ms | backward ms | step ms | "
          "M tokens/s | backward MFMA frac |", file=sys.stderr)
    print("|---|---|---|---|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {r['model']} | {r['H_qk']} | {r['H_v']} | {r['B']} x {r['T']} | {r['bwd_cp']} "
              f"({r['bwd_segment_chunks']}) | {r['fwd_ms']:.3f} | {r['bwd_ms']:.3f} | {r['step_ms']:.3f} | "
              f"{r['step_tokens_per_s'] / 1e6:.1f} | {r['bwd_mfma_frac']:.3f} |", file=sys.stderr)


def fwd_bwd(args, w, x, dev):
    """One step = the forward keeping h and A, then the backward on them."""
    import torch
    from gated_deltanet_chunked_chunk_amd import PreparedForwardBackward
    call = PreparedForwardBackward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["dO"], scale=x["scale"],
                                   initial_state=x["initial_state"], d_final_state=x["dht"], cp=args.cp)
    tokens = w.B * w.T
    flush = Flusher(dev)
    flush.settle(call, seconds=args.settle_seconds)
    for _ in range(args.warmup):
        flush()
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    (pf, pb), wall = time_steps([call.forward, call.backward], args.steps, flush, stream)
    fwd_ms = sum(pf) / len(pf)
    bwd_ms = sum(pb) / len(pb)
    ms_per_step = fwd_ms + bwd_ms
    value = tokens / (ms_per_step * 1e-3)
    bwd_bytes, bwd_flops = bwd_algorithmic(x)
    achieved = bwd_flops / (bwd_ms * 1e-3) / 1e12
    tr = stored_traffic_entry(args.workload, args.cp)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None if tr is None else tr["bytes_per_launch"],
                "kernel": "gdn_bwd (reverse pass + chunk-local gradients, key-head sums fused)",
                "algorithmic_flops_per_launch": bwd_flops, "algorithmic_bytes_per_launch": bwd_bytes,
                "mean_launch_ms": round(bwd_ms, 4), "forward_mean_launch_ms": round(fwd_ms, 4)}
    if tr is not None:
        # HBM bytes per call of each kernel of the step (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled)
        roofline["traffic_by_kernel"] = {r: e["fetch_bytes"] + e["write_bytes"] for r, e in tr["kernels"].items()}
        roofline["traffic_over_algorithmic"] = round(tr["bytes_per_launch"] / bwd_bytes, 2)
    cpu = None if args.no_cpu_baseline else cpu_baseline_bwd(x, w, args.cpu_seconds)
    line = {
        "metric": "GDN fwd+bwd latency (ms) & tokens/s at 1x32768, 4/16 heads; % of MFMA roofline (backward)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "wall_ms_per_step_with_flush": round(wall * 1e3 / args.steps, 4),
        "dtype": "bf16", "data": "synthetic (seeded random q,k,v,g,beta,initial_state,dO,d_final_state)",
        "config": {"workload": args.workload, "B": w.B, "T": w.T, "H_qk": w.H_qk, "H_v": w.H_v, "K": w.K,
                   "V": w.V, "cp": call.finfo["cp"], "bwd_cp": call.binfo["cp"],
                   "bwd_segment_chunks": call.binfo["segment_chunks"], "grad_dtype": "bf16"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~100 launches (~30 ms) bring the clocks to their steady state; fewer
    # time part of the ramp (the first launches run up to 15 % slower)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gdn_fwd_1x32768_h16x16")
    ap.add_argument("--cp", default="auto")
    ap.add_argument("--o-dtype", default="bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA probe and the library GEMM (short profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-seconds", type=float, default=SETTLE_S,
                    help="untimed run of the measured call before the warm-up steps (clock settle)")
    ap.add_argument("--sweep", action="store_true",
                    help="forward latency over the pages' head settings and batch lengths (one JSON line each)")
    ap.add_argument("--sweep-bwd", action="store_true",
                    help="training-step latency against total tokens over the pages' head settings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="store HBM bytes per launch from rocprofv3 counter CSVs (no GPU needed)")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.workload, args.cp, *args.ingest_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the forward shards over (sequence, head-group) "
              "with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args.steps, args.warmup, args.cp)
        return
    if args.sweep_bwd:
        sweep_bwd(args.steps, args.warmup, args.cp)
        return

    import torch
    from gated_deltanet_chunked_chunk_amd import PreparedForward
    from gated_deltanet_chunked_chunk_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return

    w = W.WORKLOADS[args.workload]
    x = W.make_inputs(w, device=dev)
    if w.with_grads:
        fwd_bwd(args, w, x, dev)
        return
    call = PreparedForward(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                           initial_state=x["initial_state"], output_final_state=w.want_ht,
                           cu_seqlens=x["cu_seqlens"], cp=args.cp, o_dtype=args.o_dtype)
    info = call.info
    tokens = w.B * w.T if x["cu_seqlens"] is None else int(x["cu_seqlens"][-1])

    flush = Flusher(dev)
    flush.settle(call, seconds=args.settle_seconds)
    for _ in range(args.warmup):
        flush()
        call()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    (per_launch_ms,), wall = time_steps([call], args.steps, flush, stream)
    kern_ms = sum(per_launch_ms) / len(per_launch_ms)
    ms_per_step = kern_ms
    value = tokens / (ms_per_step * 1e-3)

    alg = algorithmic_bytes(x)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(args.workload, args.cp),
                "kernel": "gdn_fwd_main_kernel", "algorithmic_bytes_per_launch": alg,
                "mean_launch_ms": round(kern_ms, 4)}
    flops = fwd_flops(x)
    tflops = flops / (kern_ms * 1e-3) / 1e12
    peak_meas = None if args.no_mfma_probe else measured_mfma_peak(dev)
    gemm = None if args.no_mfma_probe else measured_gemm_rate(dev)
    mfma = {"achieved": round(tflops, 1), "unit": "TFLOP/s", "algorithmic_flops_per_launch": flops,
            "peak_published": MFMA_BF16_PEAK_TFLOPS, "frac_published": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_measured": round(peak_meas, 1) if peak_meas else None,
            "frac_measured": round(tflops / peak_meas, 4) if peak_meas else None,
            "library_gemm_8192": round(gemm, 1) if gemm else None}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, args.cpu_seconds)

    line = {
        "metric": "GDN fwd latency (ms) & tokens/s at 1x32768; % of HBM/MFMA roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "wall_ms_per_step_with_flush": round(wall * 1e3 / args.steps, 4),
        "pages_h200_ms_context": PAGES_MS.get(args.workload),
        "dtype": "bf16", "data": "synthetic (seeded random q,k,v,g,beta,initial_state of the workload's shapes)",
        "config": {"workload": args.workload, "B": w.B, "T": w.T, "H_qk": w.H_qk, "H_v": w.H_v, "K": w.K,
                   "V": w.V, "cp": info["cp"], "segment_chunks": info["segment_chunks"],
                   "workgroups": info["workgroups"], "o_dtype": args.o_dtype},
        "roofline": roofline,
        "mfma": mfma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
