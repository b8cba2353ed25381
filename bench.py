#!/usr/bin/env python3
"""Throughput of the DARKFormer PRF-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one dark_prf_fwd call over one batch (every kernel of the path:
operand preparation, key-side state, state prefix, query-side output), on
seeded synthetic inputs already resident in HBM.  The timed region replays a
HIP graph of back-to-back forwards that rotate over enough input copies to
touch more memory than the 256 MB Infinity Cache holds; the step time is the
median over several timed replays.  Prints one JSON line.  Its headline is the
causal L=2048 attention core (B=2, H=8, d_h=64, m=256, r=64); the other
workloads are measured in the same run and reported under "workloads": the
L=64K non-causal one (B=1, H=8, d_h=64, m=1024, r=16), the L=8192 GQA prefill
(B=4, 8 query heads on 1 K/V head, d_h=256, m=512, r=256), the decode step
(256 sequences x 8 heads) and the tiny fp32 call (as a latency).  Each carries
the roofline of its dominant kernel and the fp64 oracle timed on a bounded
sample.  `--workload NAME` prints the line of one workload only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "fwd tokens/sec (all heads) at L=2048 and L=64K; % bf16 MFMA/HBM roofline"
MALL_BYTES = 256 << 20


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work per kernel (method steps only; no recomputation counted)
# ---------------------------------------------------------------------------
CHUNK_ALG = 64   # causal chunk length of the algorithmic count (fixed; not the implementation's)


def folded_queries(w) -> bool:
    """Whether the query feature map counts as the folded product x W_h^T
    (W_h = Omega M_h, m x d_h): when m d_h < r d_h + m r."""
    return w.m * w.d_h < w.r * w.d_h + w.m * w.r


def alg_flops_per_token_head(w) -> dict:
    """Algorithmic flops per (token, query head) of each side of the forward:
    key feature map 2 r (d_h + m); query feature map 2 m d_h when folded, else
    2 r (d_h + m); each feature-space contraction 2 m (d_h + 1); causal adds the
    masked C x C block 2 C (m + d_h + 1) with C = 64."""
    fmap = 2 * w.r * (w.d_h + w.m)
    qmap = 2 * w.m * w.d_h if folded_queries(w) else fmap
    contr = 2 * w.m * (w.d_h + 1)
    intra = 2 * CHUNK_ALG * (w.m + w.d_h + 1) if w.causal else 0
    return {"kstate": fmap + contr, "qout": qmap + contr + intra}


def kernel_flops(w) -> dict:
    """Algorithmic flops per launch of the key-side and query-side kernels."""
    th = w.B * w.H * w.L
    return {k: th * v for k, v in alg_flops_per_token_head(w).items()}


def alg_flops(w) -> int:
    return sum(kernel_flops(w).values())


def io_bytes(w) -> int:
    e = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.L * w.d_h * e
    return tok * (2 * w.H + 2 * w.hkv)


def nominal_flops(w) -> int:
    return 8 * w.B * w.H * w.L * w.m * w.d_h


def source_digest() -> str:
    """Digest of the sources the forward, cross-attention and decode kernels
    are built and planned from (the kernels whose HBM bytes are recorded)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "random_feature_linear_amd")
    # the kernel sources, the host planner and the generator of the instantiation units
    for f in ("csrc/common.h", "csrc/prf_kernels.h", "csrc/decode_kernels.h", "csrc/api.hip", "build.py"):
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        ent = rec.get(workload, {}).get(kernel)
        if ent and ent.get("source_digest") == source_digest():
            return ent.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


# ---------------------------------------------------------------------------
# device-side forward
# ---------------------------------------------------------------------------
class Forward:
    """Device inputs (several copies), output and workspace for one workload."""

    def __init__(self, w, copies: int):
        import torch

        from random_feature_linear_amd import binding as bd
        from random_feature_linear_amd.workloads import make_inputs
        self.bd, self.w = bd, w
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
        inp = make_inputs(w)
        self.M = torch.from_numpy(inp["M"]).to("cuda:0")
        self.omega = torch.from_numpy(bd.dark_prf_omega(w.seed, w.m, w.r, w.orthogonal)).to("cuda:0")
        base = {n: torch.from_numpy(inp[n]).to(dt).to("cuda:0") for n in ("q", "k", "v")}
        mask = torch.from_numpy(inp["mask"]).to("cuda:0") if inp["mask"] is not None else None
        self.copies = []
        for _ in range(copies):
            c = {n: base[n].clone() for n in base}
            c["mask"] = mask.clone() if mask is not None else None
            c["out"] = torch.empty_like(c["q"])
            self.copies.append(c)
        self.tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
        c0 = self.copies[0]
        self.desc = bd.make_desc(c0["q"], c0["k"], c0["v"], c0["out"], self.M, self.omega, w.causal, self.tag)
        self.ws_bytes = bd.dark_prf_workspace_bytes(self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
        self.args = [(c["q"].data_ptr(), c["k"].data_ptr(), c["v"].data_ptr(),
                      c["mask"].data_ptr() if c["mask"] is not None else 0, c["out"].data_ptr())
                     for c in self.copies]

    def __call__(self, i: int) -> None:
        import torch
        q, k, v, mk, out = self.args[i % len(self.args)]
        st = self.bd.dark_prf_fwd(self.desc, q, k, v, self.M.data_ptr(), self.omega.data_ptr(), mk,
                                  out, 0, 0, self.ws.data_ptr(), self.ws_bytes,
                                  torch.cuda.current_stream().cuda_stream)
        if st != self.bd.DARK_OK:
            raise self.bd.DarkPrfError(st, "dark_prf_fwd")


def timed_replays(g, replays: int) -> list:
    """Milliseconds of each of `replays` replays of graph g, timed with events on the
    current stream (one untimed replay first)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    return times


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def measure(w, steps: int, warmup: int, eager: bool = False, replays: int = 5) -> dict:
    import torch
    per_copy = io_bytes(w)
    copies = max(2, min(32, -(-(MALL_BYTES + (64 << 20)) // per_copy)))
    fwd = Forward(w, copies)
    log(f"[bench] {w.name}: {copies} input copies of {per_copy / 1e6:.1f} MB, workspace "
        f"{fwd.ws_bytes / 1e6:.1f} MB")
    for i in range(warmup):
        fwd(i)
    torch.cuda.synchronize()
    if eager:   # plain launches (for profilers that follow kernel dispatches)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            fwd(i)
        t1.record()
        torch.cuda.synchronize()
        return {"ms": t0.elapsed_time(t1) / steps, "n_fwd": steps, "copies": copies, "kernels": {},
                "launch": "eager"}
    # Timed region: one HIP graph of `steps` forwards that rotate over the input
    # copies; the per-forward time is the median over `replays` timed replays.
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fwd(i)
    torch.cuda.synchronize()
    reps = timed_replays(g, replays)
    # Per-kernel times: the same `steps` forwards launched one by one right behind
    # the replays (the GPU stays busy), with the library's HIP events recorded
    # around every kernel launch on the stream the kernel runs on.
    g.replay()
    fwd.bd.dark_prf_timing_begin()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fwd(i)
    e1.record()
    per = fwd.bd.dark_prf_timing_end()
    torch.cuda.synchronize()
    ms = median(reps) / steps
    ms_eager = e0.elapsed_time(e1) / steps
    del g
    kern = {k: {"avg_us": 1e3 * v[0] / v[1], "launches": v[1]} for k, v in per.items() if v[1] > 0}
    return {"ms": ms, "ms_eager": ms_eager, "n_fwd": steps, "copies": copies, "kernels": kern,
            "replay_ms": [round(t / steps, 6) for t in reps]}


def roofline(w, res: dict) -> dict:
    """Roofline of the dominant kernel (largest average live duration): its
    algorithmic flops per launch over that duration, against the dense MFMA peak
    of the input type."""
    flops = kernel_flops(w)
    dom = max(res["kernels"], key=lambda k: res["kernels"][k]["avg_us"])
    avg_s = res["kernels"][dom]["avg_us"] * 1e-6
    traffic = traffic_from_profiles(dom, w.name)
    if dom in flops:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        ach = flops[dom] / avg_s / 1e12
        return {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                "flops_per_launch": flops[dom],
                "flops_per_token_head": alg_flops_per_token_head(w)[dom],
                "avg_launch_us": round(res["kernels"][dom]["avg_us"], 3)}
    return {"bound": "hbm", "kernel": dom, "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": None, "traffic": traffic, "avg_launch_us": round(res["kernels"][dom]["avg_us"], 3)}


def cpu_baseline(w, max_heads=None, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle on the host cores, on a bounded sample of the same workload:
    `max_heads` (batch, head) slices at full length, repeated until at least
    `min_seconds` of wall time have passed."""
    from threadpoolctl import threadpool_info

    import oracle
    from random_feature_linear_amd.workloads import make_inputs
    inp = make_inputs(w)
    om = oracle.omega(w.seed, w.m, w.r, w.orthogonal)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    if max_heads is not None:
        pairs = pairs[:max_heads]
    reps, t = 0, time.perf_counter()
    while True:
        oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], om, mask=inp["mask"],
                         causal=w.causal, heads=pairs)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    frac = len(pairs) / (w.B * w.H)
    tok_s = reps * w.B * w.L * frac / dt
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") in
                   ("openblas", "mkl", "blis")] or [1])
    return {"value": round(tok_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(pairs)} of {w.B * w.H} (batch, head) slices at full length, fp64, "
                      f"{reps} repetitions in {dt:.1f} s", "blas": "openblas",
            "host_cpus": len(os.sched_getaffinity(0))}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 4) -> None:
    """Plain device-to-device copies of `nbytes` (for scaling HBM byte counters)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def line_for(w, res: dict) -> dict:
    tokens = w.B * w.L
    sec = res["ms"] * 1e-3
    value = tokens / sec
    nom = nominal_flops(w) / sec / 1e12
    alg = alg_flops(w) / sec / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    return {
        "value": round(value, 1), "unit": "tokens/s", "ms_per_step": round(res["ms"], 6),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.hkv, "L": w.L, "d_h": w.d_h,
                   "m": w.m, "r": w.r, "causal": w.causal, "mask": w.mask_kind,
                   "launch": "one hipGraph of %d forwards over %d rotating input copies, median of %d replays"
                             % (res["n_fwd"], res["copies"], len(res["replay_ms"]))},
        "roofline": roofline(w, res),
        "forward_frac": {"alg_tflops": round(alg, 2), "alg_frac": round(alg / peak, 4),
                         "nominal_tflops": round(nom, 2), "nominal_frac": round(nom / peak, 4),
                         "io_GBps": round(io_bytes(w) / sec / 1e9, 1),
                         "io_frac_hbm": round(io_bytes(w) / sec / 1e9 / PEAK_HBM_GBS, 4)},
        "replay_ms_per_step": res["replay_ms"],
        "kernels_us": {k: round(v["avg_us"], 3) for k, v in res["kernels"].items()},
        "kernel_timing": "HIP events around each launch, eager pass of the same forwards "
                         "right behind the timed replays (%.4f ms per forward)" % res["ms_eager"],
    }


def decode_line(steps: int, replays: int = 3) -> dict:
    """Workload 5: `steps` one-token steps over 256 sequences x 8 heads (fp32
    state, updated in place), captured in one HIP graph; median of `replays`
    replays.  The state holds seeded random values of the shape a 4096-token
    prefill leaves (a step's work and bytes do not depend on the values)."""
    import torch

    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import CONFIGS, make_decode_tokens, make_inputs
    w = CONFIGS["c5_decode"]
    g = torch.Generator(device="cuda:0").manual_seed(w.seed)
    dt = torch.bfloat16
    S = torch.randn((w.B, w.H, w.m, w.d_h), generator=g, device="cuda:0", dtype=torch.float32)
    z = torch.rand((w.B, w.H, w.m), generator=g, device="cuda:0", dtype=torch.float32) * 4096
    tok = make_decode_tokens(w, steps)
    tq, tk, tv = (torch.from_numpy(tok[n]).to(dt).to("cuda:0") for n in ("q", "k", "v"))
    M = torch.from_numpy(make_inputs(w.with_(B=1, L=1))["M"]).to("cuda:0")
    om = torch.from_numpy(bd.dark_prf_omega(w.seed, w.m, w.r, w.orthogonal)).to("cuda:0")
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    out = torch.empty_like(tq[0])
    for t in range(4):
        bd.decode_step(tq[t], tk[t], tv[t], M, om, S, z, tag, tag, out=out)
    torch.cuda.synchronize()
    sm = torch.cuda.Stream()
    sm.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(sm):
        with torch.cuda.graph(gr, stream=sm):
            for t in range(steps):
                bd.decode_step(tq[t], tk[t], tv[t], M, om, S, z, tag, tag, out=out)
    torch.cuda.synchronize()
    reps = timed_replays(gr, replays)
    ms = median(reps) / steps
    del gr
    bd.dark_prf_timing_begin()
    for t in range(min(steps, 64)):
        bd.decode_step(tq[t], tk[t], tv[t], M, om, S, z, tag, tag, out=out)
    per = bd.dark_prf_timing_end()
    avg_us = 1e3 * per["decode"][0] / per["decode"][1]
    # algorithmic bytes of one step: S and z read and written once (fp32), plus
    # q, k, v and out (bf16)
    state_bytes = 2 * (w.B * w.H * w.m * (w.d_h + 1) * 4)
    tok_bytes = 2 * w.d_h * (2 * w.B * w.H + 2 * w.B * w.hkv)
    ach = (state_bytes + tok_bytes) / (avg_us * 1e-6) / 1e9
    return {"value": round(w.B / (ms * 1e-3), 1), "ms_per_step": round(ms, 6), "unit": "tokens/s",
            "config": {"workload": w.name, "N": w.B, "H": w.H, "d_h": w.d_h, "m": w.m, "r": w.r,
                       "steps": steps, "state": "seeded random fp32 of the prefilled state's shape",
                       "launch": "one hipGraph of %d decode steps, median of %d replays" % (steps, replays)},
            "replay_ms_per_step": [round(t / steps, 6) for t in reps],
            "roofline": {"bound": "hbm", "kernel": "decode", "achieved": round(ach, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": traffic_from_profiles("decode", w.name),
                         "bytes_per_launch": state_bytes + tok_bytes, "avg_launch_us": round(avg_us, 3)}}


def cpu_baseline_decode(w, seqs: int = 16, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle's recurrence (oracle.decode_step, vectorised over sequences
    and heads) on `seqs` of the 256 sequences, one token per step, repeated until
    `min_seconds` have passed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from random_feature_linear_amd.workloads import make_decode_tokens, make_inputs
    om = oracle.omega(w.seed, w.m, w.r, w.orthogonal)
    M = make_inputs(w.with_(B=1, L=1))["M"]
    rng = np.random.default_rng(w.seed)
    S = rng.standard_normal((seqs, w.H, w.m, w.d_h))
    z = rng.random((seqs, w.H, w.m)) * 4096
    tok = make_decode_tokens(w.with_(B=seqs), 64)
    steps, t = 0, time.perf_counter()
    while True:
        i = steps % 64
        _, S, z = oracle.decode_step(S, z, tok["q"][i], tok["k"][i], tok["v"][i], M, om)
        steps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") in
                   ("openblas", "mkl", "blis")] or [1])
    return {"value": round(seqs * steps / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{seqs} of {w.B} sequences x {w.H} heads, {steps} one-token steps in {dt:.1f} s, fp64",
            "host_cpus": len(os.sched_getaffinity(0))}


def cross_line(steps: int, eager: bool = False) -> dict:
    """Cross-attention at the pages' example shape: queries B=2 x L_q=256 against
    a context of L_k=1024 (8 heads of 64, m=256), with a padded context.  One
    step = the context summary (dark_prf_context_state) and the queries against
    it (dark_prf_cross_fwd); both run in one HIP graph of `steps` steps."""
    import torch

    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import Workload, make_inputs
    Lq, Lk = 256, 1024
    wk = Workload(name="cross_example", B=2, H=8, L=Lk, d_h=64, m=256, r=64, dtype="bf16", causal=False,
                  seed=1010, mask_kind="tail", max_pad=256)
    wq = wk.with_(L=Lq, mask_kind="none")
    ctx, qry = make_inputs(wk), make_inputs(wq)
    dt = torch.bfloat16
    dev = lambda a, t=None: torch.from_numpy(a).to(t).to("cuda:0") if t else torch.from_numpy(a).to("cuda:0")
    k, v, q = dev(ctx["k"], dt), dev(ctx["v"], dt), dev(qry["q"], dt)
    cmask = dev(ctx["mask"])
    M = dev(ctx["M"])
    om = torch.from_numpy(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal)).to("cuda:0")
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    S = torch.empty((wk.B, wk.H, wk.m, wk.d_h), dtype=torch.float32, device="cuda:0")
    z = torch.empty((wk.B, wk.H, wk.m), dtype=torch.float32, device="cuda:0")
    out = torch.empty_like(q)
    dk = bd.make_desc(k, k, v, k, M, om, False, tag)
    dk.H = wk.H
    dq = bd.make_desc(q, q, q, out, M, om, False, tag)
    dq.H_kv = wk.H
    nb = max(bd.dark_prf_workspace_bytes(dk), bd.dark_prf_workspace_bytes(dq))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")

    def step():
        st = torch.cuda.current_stream().cuda_stream
        r1 = bd.dark_prf_context_state(dk, k.data_ptr(), v.data_ptr(), M.data_ptr(), om.data_ptr(),
                                       cmask.data_ptr(), S.data_ptr(), z.data_ptr(), ws.data_ptr(), nb, st)
        r2 = bd.dark_prf_cross_fwd(dq, q.data_ptr(), M.data_ptr(), om.data_ptr(), S.data_ptr(), z.data_ptr(),
                                   tag, 0, out.data_ptr(), ws.data_ptr(), nb, st)
        if r1 != bd.DARK_OK or r2 != bd.DARK_OK:
            raise bd.DarkPrfError(r1 or r2, "cross-attention")

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    if eager:   # plain launches (for profilers that follow kernel dispatches)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        return {"workload": "cross_example", "ms_per_step": t0.elapsed_time(t1) / steps, "steps": steps,
                "launch": "eager"}
    sm = torch.cuda.Stream()
    sm.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(sm):
        with torch.cuda.graph(g, stream=sm):
            for _ in range(steps):
                step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g
    bd.dark_prf_timing_begin()
    for _ in range(steps):
        step()
    per = bd.dark_prf_timing_end()
    torch.cuda.synchronize()
    kern = {kk: 1e3 * vv[0] / vv[1] for kk, vv in per.items() if vv[1] > 0}
    # key side: projection, exponent and state per context token and head; query
    # side: projection, exponent and output per query token and head
    per_tok = 2 * wk.r * wk.d_h + 2 * wk.r * wk.m + 2 * wk.m * (wk.d_h + 1)
    flops = {"kstate": wk.B * wk.H * Lk * per_tok, "qout": wk.B * wk.H * Lq * per_tok}
    dom = max(("kstate", "qout"), key=lambda kk: kern.get(kk, 0.0))
    ach = flops[dom] / (kern[dom] * 1e-6) / 1e12
    return {"value": round(wk.B * Lq / (ms * 1e-3), 1), "unit": "query tokens/s", "ms_per_step": round(ms, 6),
            "config": {"workload": "cross_example", "B": wk.B, "H": wk.H, "L_q": Lq, "L_k": Lk, "d_h": wk.d_h,
                       "m": wk.m, "r": wk.r, "context_mask": "tail", "query_mask": "none",
                       "step": "dark_prf_context_state + dark_prf_cross_fwd",
                       "launch": "one hipGraph of %d steps" % steps},
            "kernels_us": {kk: round(vv, 3) for kk, vv in kern.items()},
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profiles(dom, "cross_example"),
                         "flops_per_launch": flops[dom], "avg_launch_us": round(kern[dom], 3)}}


def cross_step_line(steps: int) -> dict:
    """Cross-attention in generation: 256 sequences x 8 heads, each with a context
    summary of 1024 tokens (made once, untimed); every step is one query token per
    sequence against its summary (dark_prf_cross_fwd with L_q = 1)."""
    import torch

    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import Workload, make_inputs
    wk = Workload(name="cross_step", B=256, H=8, L=1024, d_h=64, m=256, r=64, dtype="bf16", causal=False,
                  seed=1011, mask_kind="tail", max_pad=256)
    ctx = make_inputs(wk)
    dt = torch.bfloat16
    k = torch.from_numpy(ctx["k"]).to(dt).to("cuda:0")
    v = torch.from_numpy(ctx["v"]).to(dt).to("cuda:0")
    cmask = torch.from_numpy(ctx["mask"]).to("cuda:0")
    M = torch.from_numpy(ctx["M"]).to("cuda:0")
    om = torch.from_numpy(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal)).to("cuda:0")
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    S, z = bd.context_state(k, v, M, om, wk.H, context_mask=cmask, proj_tag=tag)
    del k, v
    g = torch.Generator(device="cuda:0").manual_seed(wk.seed)
    tq = torch.randn((steps, wk.B, wk.H, 1, wk.d_h), generator=g, device="cuda:0").to(dt)
    out = torch.empty_like(tq[0])
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda:0")
    for t in range(4):
        bd.cross_attention(tq[t], M, om, S, z, tag, tag, H_kv=wk.H, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for t in range(steps):
        bd.cross_attention(tq[t], M, om, S, z, tag, tag, H_kv=wk.H, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    bd.dark_prf_timing_begin()
    for t in range(min(steps, 64)):
        bd.cross_attention(tq[t], M, om, S, z, tag, tag, H_kv=wk.H, out=out, workspace=ws)
    per = bd.dark_prf_timing_end()
    avg_us = 1e3 * per["decode"][0] / per["decode"][1]
    state_bytes = wk.B * wk.H * wk.m * (wk.d_h + 1) * 4   # the summary, read once
    ach = state_bytes / (avg_us * 1e-6) / 1e9
    return {"value": round(wk.B / (ms * 1e-3), 1), "ms_per_step": round(ms, 6), "unit": "query tokens/s",
            "config": {"workload": "cross_step", "N": wk.B, "H": wk.H, "L_q": 1, "L_k": wk.L, "d_h": wk.d_h,
                       "m": wk.m, "r": wk.r, "steps": steps, "launch": "eager, one launch per step"},
            "roofline": {"bound": "hbm", "kernel": "decode_kernel (read-only form)", "achieved": round(ach, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": None, "bytes_per_launch": state_bytes, "avg_launch_us": round(avg_us, 3)}}


def exact_line(w, steps: int) -> dict:
    """The exact learned-kernel path (dark_prf_exact_fwd) on a workload's inputs,
    timed like the linear forward (one HIP graph over rotating input copies).
    Algorithmic flops: 2 r (score) + 2 d_h (weighted sum) per visible
    (query, key) pair; the projections 2 r d_h per row of q and k."""
    import torch

    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import make_inputs
    inp = make_inputs(w)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    copies = max(2, min(32, -(-(MALL_BYTES + (64 << 20)) // io_bytes(w))))
    base = {n: torch.from_numpy(inp[n]).to(dt).to("cuda:0") for n in ("q", "k", "v")}
    M = torch.from_numpy(inp["M"]).to("cuda:0")
    mask = torch.from_numpy(inp["mask"]).to("cuda:0") if inp["mask"] is not None else None
    sets = [{n: base[n].clone() for n in base} for _ in range(copies)]
    outs = [torch.empty_like(base["q"]) for _ in range(copies)]
    c0 = sets[0]
    d = bd.make_desc(c0["q"], c0["k"], c0["v"], outs[0], M, torch.empty((16, w.r)), w.causal, 0)
    nb = bd.dark_prf_exact_workspace_bytes(d)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    mptr = mask.data_ptr() if mask is not None else 0

    def step(i):
        c, o = sets[i % copies], outs[i % copies]
        st = bd.dark_prf_exact_fwd(d, c["q"].data_ptr(), c["k"].data_ptr(), c["v"].data_ptr(), M.data_ptr(), mptr,
                                   o.data_ptr(), ws.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
        if st != bd.DARK_OK:
            raise bd.DarkPrfError(st, "dark_prf_exact_fwd")

    for i in range(10):
        step(i)
    torch.cuda.synchronize()
    sm = torch.cuda.Stream()
    sm.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(sm):
        with torch.cuda.graph(g, stream=sm):
            for i in range(steps):
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g
    bd.dark_prf_timing_begin()
    for i in range(steps):
        step(i)
    per = bd.dark_prf_timing_end()
    torch.cuda.synchronize()
    kern = {{"prep": "mfrag", "shift": "project", "qout": "attention"}.get(kk, kk): 1e3 * vv[0] / vv[1]
            for kk, vv in per.items() if vv[1] > 0}
    pairs = w.L * (w.L + 1) // 2 if w.causal else w.L * w.L
    flops = w.B * w.H * pairs * 2 * (w.r + w.d_h)
    ach = flops / (kern["attention"] * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    return {"value": round(w.B * w.L / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 6),
            "config": {"workload": w.name, "path": "exact (dark_prf_exact_fwd)", "B": w.B, "H": w.H,
                       "H_kv": w.hkv, "L": w.L, "d_h": w.d_h, "r": w.r, "causal": w.causal,
                       "launch": "one hipGraph of %d forwards over %d rotating input copies" % (steps, copies)},
            "kernels_us": {kk: round(vv, 3) for kk, vv in kern.items()},
            "roofline": {"bound": "mfma", "kernel": "attention", "achieved": round(ach, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None,
                         "flops_per_launch": flops, "avg_launch_us": round(kern["attention"], 3)}}


def bwd_flops_per_token_head(w, chunk: int = 64) -> int:
    """Algorithmic flops of the backward's matrix products per (token, head):
    projections of q and k (2 * 2 r d_h), their features (2 * 2 r m), the key
    and query chunk states (2 * 2 m (d_h+1)), [N, D] from the states
    (2 m (d_h+1)), dPhi(Q) and dPhi(K) from the states (2 * 2 m (d_h+1)), dV
    from the state (2 m d_h), dU (2 * 2 m r), dX (2 * 2 r d_h) and dM
    (2 * 2 r d_h); causal adds the intra-chunk blocks over C = 64 tokens:
    Phi(Q)Phi(K)^T (2 C m), Gd [V,1]^T (2 C (d_h+1)) and their products with
    [V,1], Phi(K), Phi(Q) and dN (2 C (d_h+1) + 2 * 2 C m + 2 C d_h)."""
    d, m, r, C = w.d_h, w.m, w.r, chunk
    f = 4 * r * d + 4 * r * m + 4 * m * (d + 1) + 2 * m * (d + 1) + 4 * m * (d + 1) + 2 * m * d \
        + 4 * m * r + 4 * r * d + 4 * r * d
    if w.causal:
        f += 2 * C * m + 2 * C * (d + 1) + 2 * C * (d + 1) + 4 * C * m + 2 * C * d
    return f


def bwd_line(w, steps: int) -> dict:
    """The backward pass (dark_prf_bwd) on a workload's inputs with a seeded
    upstream gradient: one HIP graph of `steps` backward calls, then one eager
    pass with per-kernel HIP-event timing for the matrix-product roofline."""
    import numpy as np
    import torch

    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import make_inputs
    inp = make_inputs(w)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    dev = {n: torch.from_numpy(inp[n]).to(dt).to("cuda:0") for n in ("q", "k", "v")}
    rng = np.random.default_rng(w.seed + 7)
    dout = torch.from_numpy(rng.standard_normal(inp["q"].shape).astype(np.float32)).to(dt).to("cuda:0")
    M = torch.from_numpy(inp["M"]).to("cuda:0")
    om = torch.from_numpy(bd.dark_prf_omega(w.seed, w.m, w.r, w.orthogonal)).to("cuda:0")
    mask = torch.from_numpy(inp["mask"]).to("cuda:0") if inp["mask"] is not None else None
    grads = [torch.empty_like(dev[n]) for n in ("q", "k", "v")] + [torch.empty_like(M)]
    d = bd.make_desc(dev["q"], dev["k"], dev["v"], dout, M, om, w.causal)
    nb = bd.dark_prf_bwd_workspace_bytes(d)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    mptr = mask.data_ptr() if mask is not None else 0

    def step():
        st = bd.dark_prf_bwd(d, dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), M.data_ptr(),
                             om.data_ptr(), mptr, dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                             grads[2].data_ptr(), grads[3].data_ptr(), ws.data_ptr(), nb,
                             torch.cuda.current_stream().cuda_stream)
        if st != bd.DARK_OK:
            raise bd.DarkPrfError(st, "dark_prf_bwd")

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    sm = torch.cuda.Stream()
    sm.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(sm):
        with torch.cuda.graph(g, stream=sm):
            for _ in range(steps):
                step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g
    bd.dark_prf_timing_begin()
    for _ in range(steps):
        step()
    per = bd.dark_prf_timing_end()
    torch.cuda.synchronize()
    gemm_ms, gemm_n = per["bwd_gemm"]
    aux_ms, aux_n = per["bwd_aux"]
    flops = w.B * w.H * w.L * bwd_flops_per_token_head(w)
    gemm_per_call_us = 1e3 * gemm_ms / steps
    ach = flops / (gemm_per_call_us * 1e-6) / 1e12
    return {"value": round(w.B * w.L / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 6),
            "config": {"workload": w.name, "path": "backward (dark_prf_bwd)", "B": w.B, "H": w.H,
                       "H_kv": w.hkv, "L": w.L, "d_h": w.d_h, "m": w.m, "r": w.r, "causal": w.causal,
                       "launch": "one hipGraph of %d backward calls" % steps},
            "kernels_us": {"gemm_per_call": round(gemm_per_call_us, 3), "gemm_launches_per_call": gemm_n // steps,
                           "aux_per_call": round(1e3 * aux_ms / steps, 3), "aux_launches_per_call": aux_n // steps},
            "roofline": {"bound": "mfma", "kernel": "bgemm (all matrix products of one call)",
                         "achieved": round(ach, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_F32_TFLOPS, 4), "traffic": None, "flops_per_launch": flops,
                         "avg_launch_us": round(gemm_per_call_us, 3)}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_causal_L2048")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-secondary", action="store_true",
                    help="measure only the chosen workload (no other workloads, no cross-attention)")
    ap.add_argument("--no-cross", action="store_true",
                    help="skip the cross-attention, exact-path and backward measurements")
    ap.add_argument("--eager", action="store_true",
                    help="plain launches instead of a HIP graph, no per-kernel timing (for profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path, so --gpus must be 1",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from random_feature_linear_amd import binding as bd
    from random_feature_linear_amd.workloads import CONFIGS
    if args.copy_calibration:
        copy_calibration()
        return 0
    bd.lib()
    torch.cuda.synchronize()
    if args.workload == "c5_decode":
        rec = decode_line(min(args.steps, 512))
        rec.update({"metric": "decode tokens/sec (256 sequences x 8 heads, one token each)",
                    "n_gpus": 1, "steps": min(args.steps, 512), "warmup": 4, "higher_is_better": True,
                    "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return 0
    if args.workload == "cross_step":
        rec = cross_step_line(min(args.steps, 512))
        rec.update({"metric": "cross-attention decoder-step query tokens/sec (one token per sequence)",
                    "n_gpus": 1, "steps": min(args.steps, 512), "warmup": 4, "higher_is_better": True,
                    "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return 0
    if args.workload == "cross_example":
        rec = cross_line(min(args.steps, 400), eager=args.eager)
        if not args.eager:
            rec.update({"metric": "cross-attention query tokens/sec (context summary + queries)", "n_gpus": 1,
                        "steps": min(args.steps, 400), "warmup": 10, "higher_is_better": True,
                        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return 0
    if args.workload.startswith("bwd:"):   # the backward pass on one of the workloads' inputs
        wb = CONFIGS[args.workload.split(":", 1)[1]]
        nsteps = max(2, min(args.steps, 50))
        rec = bwd_line(wb, nsteps)
        rec.update({"metric": "backward tokens/sec", "n_gpus": 1, "steps": nsteps, "warmup": 3,
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                    "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return 0
    if args.workload.startswith("exact:"):   # the exact path on one of the workloads' inputs
        we = CONFIGS[args.workload.split(":", 1)[1]]
        rec = exact_line(we, min(args.steps, 200))
        rec.update({"metric": "exact-path fwd tokens/sec", "n_gpus": 1, "steps": min(args.steps, 200),
                    "warmup": 10, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                    "dtype": we.dtype, "data": "synthetic"})
        print(json.dumps(rec), flush=True)
        return 0
    w = CONFIGS[args.workload]
    if args.eager:
        res = measure(w, args.steps, args.warmup, eager=True)
        print(json.dumps({"workload": w.name, "ms_per_step": res["ms"], "steps": res["n_fwd"],
                          "launch": "eager"}), flush=True)
        return 0
    res = measure(w, args.steps, args.warmup)
    main_line = line_for(w, res)
    rec = {"metric": METRIC, "value": main_line["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": res["n_fwd"], "warmup": args.warmup, "ms_per_step": main_line["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic (seeded Gaussian inputs of the workload's shape)"}
    rec.update({k: v for k, v in main_line.items() if k not in ("value", "ms_per_step")})
    if not args.no_cpu and torch.cuda.current_device() == 0:
        log("[bench] timing the fp64 oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(w, max_heads=1 if w.L * w.B * w.H > 1 << 17 else None)
    if args.workload != "c2_causal_L2048" or args.no_secondary:
        print(json.dumps(rec), flush=True)
        return 0
    # the other workloads, measured in the same run
    others = {}
    w3 = CONFIGS["c3_long_L64K"]
    res3 = measure(w3, max(10, args.steps // 2), min(args.warmup, 5))
    others[w3.name] = line_for(w3, res3)
    w4 = CONFIGS["c4_gqa_L8192"]
    res4 = measure(w4, max(5, args.steps // 4), min(args.warmup, 3))
    others[w4.name] = line_for(w4, res4)
    log("[bench] decode steps")
    others["c5_decode"] = decode_line(512)
    w1 = CONFIGS["c1_tiny_f32"]
    res1 = measure(w1, max(100, args.steps * 5), args.warmup)
    l1 = line_for(w1, res1)
    l1["latency_us"] = round(1e3 * res1["ms"], 3)
    l1["note"] = "launch-bound (36 KB of data, 0.6 MFLOP): reported as an absolute latency per forward"
    others[w1.name] = l1
    if not args.no_cpu:
        log("[bench] timing the fp64 oracle on samples of the other workloads")
        others[w3.name]["cpu_baseline"] = cpu_baseline(w3, max_heads=1)
        others[w4.name]["cpu_baseline"] = cpu_baseline(w4, max_heads=1)
        others["c5_decode"]["cpu_baseline"] = cpu_baseline_decode(CONFIGS["c5_decode"])
        others[w1.name]["cpu_baseline"] = cpu_baseline(w1, min_seconds=3.0)
    rec["workloads"] = others
    if not args.no_cross:
        log("[bench] cross-attention, exact path and backward")
        rec["cross"] = cross_line(max(20, args.steps // 4))
        rec["cross_step"] = cross_step_line(256)
        rec["exact"] = exact_line(w, max(20, args.steps // 4))
        rec["backward"] = bwd_line(w, 20)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
