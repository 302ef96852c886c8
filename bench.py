#!/usr/bin/env python3
"""Benchmark of the PaTH attention hot path on one MI355X.

A step is one causal PaTH forward pass (prep + scan kernels) over the
B32 H32 L4096 d64 bf16 workload; K steps are timed after W warm-up steps.
Alongside it the decode step (B16 H32 d64, 32768 cached rows, bf16, 64 steps
with fresh q, w, beta each), the prefill -> decode cache build on the
forward's workspace, and the other forward workloads (L 1024 - 8192 at
d64, L4096 at d128, B8 H16 L4096, PaTH-FoX B4 H16 L16384) and the backward
pass on the forward workload are timed, and the fp64 CPU oracle is timed on
bounded samples of the forward, decode and backward workloads.  Prints one
JSON line.

Work units (fixed, declared):
  forward  F = 4 B H L^2 d flop: per causal pair of 64-token blocks the query-
           key logits, the probability-value product and the rank-64 query
           transform (2 + 2 + 4) * 64^2 d; the in-block (diagonal) work is not
           counted.
  decode   bytes = 3 B H n d * 2: read every cached key, write it back
           updated, read every cached value.
  backward Fb = 8 B H L^2 d flop: per causal pair of 64-token blocks eight
           64 x 64 x d contractions (logits, dO V^T, dV, dk^, dS k^, the
           adjoint's and the query's transition products, the transition
           gradient) at 2 * 64^2 d each; the key-major walk's recomputation
           of the logits and dO V^T and the in-block work are not counted.
           Its walks run on bf16 matrix cores for bf16 inputs, so it is
           priced against the bf16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 matrix peak (published)
METRIC = "PaTH fwd TFLOP/s + % MFMA peak (B32 H32 d64 L4096); decode-step HBM GB/s"
FWD_WORKLOAD = "sweep_L4096_d64_bf16"
DEC_WORKLOAD = "decode_N32768_bf16"
SWEEP_WORKLOADS = ["sweep_L1024_d64_bf16", "sweep_L2048_d64_bf16", "sweep_L8192_d64_bf16", "sweep_L4096_d128_bf16",
                   "lm760m_L4096_bf16", "fox_L16384_bf16"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_B32H32L4096_decode_N32768.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_fwd_B32H32L4096_decode_N32768.txt")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_B32H32L4096.txt")
COPY_BYTES = 1 << 30        # calibration copy of the counter run
KERNEL_SOURCES = {
    "path_fwd_kernel": ["attention_fwd_amd/csrc/path_fwd.hip", "attention_fwd_amd/csrc/path_common.h",
                        "attention_fwd_amd/csrc/path_layout.h"],
    "path_decode_kernel": ["attention_fwd_amd/csrc/path_decode.hip", "attention_fwd_amd/csrc/path_common.h"],
    "path_cache_kernel": ["attention_fwd_amd/csrc/path_cache.hip", "attention_fwd_amd/csrc/path_common.h",
                          "attention_fwd_amd/csrc/path_layout.h"],
    "path_bwd": ["attention_fwd_amd/csrc/path_bwd.hip", "attention_fwd_amd/csrc/path_bwd.h",
                 "attention_fwd_amd/csrc/path_common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(kernel):
    h = hashlib.sha256()
    for s in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, path=TRAFFIC_FILE):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    the counters were taken on the current kernel source (else None)."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get(kernel + ".source_sha256_16") != kernel_hash(kernel):
            return None
        return float(kv[kernel + ".hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def read_mfma_flop(kernel="path_fwd_kernel", path=MFMA_FILE):
    """Matrix-core flop one launch of `kernel` executes, from the committed counter summary
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), if the counters were taken on the current kernel source."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get(kernel + ".source_sha256_16") != kernel_hash(kernel):
            return None
        return float(kv[kernel + ".mfma_flop_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_forward(steps, warmup, name=FWD_WORKLOAD):
    import torch

    import attention_fwd_amd as pa
    import pathgen

    c = pathgen.WORKLOADS[name]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    x = pathgen.fwd_inputs(B, H, L, d, c["dtype"], seed=0, fox=c["fox"], clip=c["clip"], device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty((B, H, L), device="cuda", dtype=torch.float32)
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        pa.fwd_prep(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, ws)
        if ev:
            ev[1].record(stream)
        pa.fwd_scan(out, lse, x["logf"] is not None, ws)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    per_step = sorted(e[0].elapsed_time(e[2]) for e in evs)
    flops = 4.0 * B * H * L * L * d
    return dict(B=B, H=H, L=L, d=d, flops=flops, wall_s=wall, ms_per_step=wall * 1e3 / steps,
                prep_ms=prep_ms, scan_ms=scan_ms, x=x, ms_median=per_step[len(per_step) // 2], ms_min=per_step[0])


def bench_copy(reps=10, nbytes=1 << 31):
    """Plain device streams in the same run, for the HBM rates the memory-bound kernels can be
    compared with: a copy (torch copy_ of nbytes of bf16; GB/s counts read + write), a write-only
    fill of the same buffer, a read-only sum over three times as many bytes, and an in-place add
    b += a (two reads and one write per element: the decode step's mix)."""
    import torch

    a = torch.ones(nbytes // 2, device="cuda", dtype=torch.bfloat16)
    b = torch.empty_like(a)
    big = torch.ones(3 * nbytes // 2, device="cuda", dtype=torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: b.copy_(a))
    ms_fill = timed(lambda: b.fill_(1.0))
    ms_sum = timed(lambda: torch.sum(big, dtype=torch.float32))
    ms_add = timed(lambda: b.add_(a))
    del a, b, big
    torch.cuda.empty_cache()
    gbs = lambda nb, t: round(nb / (t * 1e-3) / 1e9, 1)
    return {"bytes_moved": 2 * nbytes, "ms": round(ms, 4), "GB_per_s": gbs(2 * nbytes, ms),
            "frac_of_hbm_peak": round(2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "fill_GB_per_s": gbs(nbytes, ms_fill), "read_sum_GB_per_s": gbs(3 * nbytes, ms_sum),
            "add_2r1w_GB_per_s": gbs(3 * nbytes, ms_add)}


def bench_sweep(steps, warmup):
    """The other forward workloads, timed the same way (not the headline line)."""
    import torch

    res = {}
    for name in SWEEP_WORKLOADS:
        f = bench_forward(steps, warmup, name)
        del f["x"]
        torch.cuda.empty_cache()
        tf = f["flops"] / (f["ms_per_step"] * 1e-3) / 1e12
        res[name] = {"ms_per_step": round(f["ms_per_step"], 4), "prep_ms": round(f["prep_ms"], 4),
                     "scan_ms": round(f["scan_ms"], 4), "TFLOP_per_s": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "tokens_per_s": round(f["B"] * f["L"] / (f["ms_per_step"] * 1e-3))}
        log("sweep %s: %.3f ms/step (prep %.3f, scan %.3f) %.1f TFLOP/s" %
            (name, f["ms_per_step"], f["prep_ms"], f["scan_ms"], tf))
    return res


def bench_fox_skip(steps, warmup, name="fox_L16384_bf16"):
    """The forget-gate workload with PATH_FWD_SKIP_NEGLIGIBLE (whole forward,
    prep + scan): time and tokens/s only -- the skipped blocks are not work
    done, so no FLOP rate is claimed for it."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    c = pathgen.WORKLOADS[name]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    x = pathgen.fwd_inputs(B, H, L, d, c["dtype"], seed=0, fox=True, clip=c["clip"], device="cuda")
    out = torch.empty_like(x["q"])
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    res = {}
    for skip in (False, True):
        for _ in range(warmup):
            pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out=out, workspace=ws, skip_negligible=skip)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out=out, workspace=ws, skip_negligible=skip)
        e1.record(stream)
        torch.cuda.synchronize()
        res[skip] = e0.elapsed_time(e1) / steps
    del x, out, ws
    torch.cuda.empty_cache()
    return {"workload": name, "ms_per_step": round(res[True], 4), "full_walk_ms_per_step": round(res[False], 4),
            "tokens_per_s": round(B * L / (res[True] * 1e-3)), "speedup_vs_full_walk": round(res[False] / res[True], 2)}


def bench_fused(steps, warmup, name=FWD_WORKLOAD):
    """The headline forward shape with the producer of w and beta fused in
    (path_attn_fwd_fused: width-3 causal convolution + L2 normalisation of w,
    beta = 2 sigmoid(z) capped at 1.98), timed as a whole call next to the plain
    forward on ready-made (w, beta) of the same shape."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    c = pathgen.WORKLOADS[name]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    x = pathgen.fused_inputs(B, H, L, d, c["dtype"], seed=0, device="cuda")
    y = pathgen.fwd_inputs(B, H, L, d, c["dtype"], seed=0, clip=c["clip"], device="cuda")
    out = torch.empty_like(x["q"])
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    calls = {
        "fused": lambda: pa.fwd_fused(x["q"], x["k"], x["v"], x["wraw"], x["conv_w"], x["zbeta"], c["clip"],
                                      out=out, workspace=ws),
        "plain": lambda: pa.fwd(y["q"], y["k"], y["v"], y["w"], y["beta"], out=out, workspace=ws),
    }
    res = {}
    for key, call in calls.items():
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        res[key] = e0.elapsed_time(e1) / steps
    del x, y, out, ws
    torch.cuda.empty_cache()
    flops = 4.0 * B * H * L * L * d
    return {"workload": name + "+producer", "ms_per_step": round(res["fused"], 4),
            "TFLOP_per_s": round(flops / (res["fused"] * 1e-3) / 1e12, 1),
            "plain_forward_ms_per_step": round(res["plain"], 4),
            "tokens_per_s": round(B * L / (res["fused"] * 1e-3))}


def bench_decode(steps, gate=False):
    """Decode steps of the decode workload; with gate, PaTH-FoX decode: a gate cache of
    prefix sums c_j (fp32, read once per step like the keys) and log f_t per step
    (logsigmoid(N(3, 1)), the forget-gate workload's distribution)."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    c = pathgen.WORKLOADS[DEC_WORKLOAD]
    B, H, n, d = c["B"], c["H"], c["n"], c["d"]
    x = pathgen.decode_inputs(B, H, n, d, steps=steps, dtype=c["dtype"], seed=0, clip=c["clip"], device="cuda")
    fc = lf = None
    if gate:
        g = torch.Generator(device="cuda")
        g.manual_seed(1)
        lf = torch.nn.functional.logsigmoid(3.0 + torch.randn((steps + 3, B, H), generator=g, device="cuda"))
        fc = torch.cumsum(torch.nn.functional.logsigmoid(
            3.0 + torch.randn((B, H, n), generator=g, device="cuda")), dim=-1).contiguous()
    out = torch.empty((B, H, d), device="cuda", dtype=x["kcache"].dtype)
    ws = torch.empty(max(pa.decode_workspace_size(B, H, n, d, x["kcache"].dtype), 16), device="cuda",
                     dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    kc, vc = x["kcache"], x["vcache"]
    gk = (lambda t: dict(logf=lf[t].contiguous(), fcache=fc)) if gate else (lambda t: {})
    for t in range(3):  # warm-up on the same cache (the update is an ordinary step)
        pa.decode_step(kc, vc, n, x["q"][t], x["w"][t], x["beta"][t], out=out, workspace=ws, **gk(t))
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for t in range(steps):
        evs[t][0].record(stream)
        pa.decode_step(kc, vc, n, x["q"][t], x["w"][t], x["beta"][t], out=out, workspace=ws, **gk(t))
        evs[t][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in evs)
    step_ms = sum(per) / steps
    nbytes = 3.0 * B * H * n * d * kc.element_size() + (4.0 * B * H * n if gate else 0.0)
    del x, kc, vc, fc, lf, ws
    torch.cuda.empty_cache()
    return dict(B=B, H=H, n=n, d=d, steps=steps, step_ms=step_ms, wall_s=wall, bytes=nbytes,
                ms_median=per[len(per) // 2], ms_min=per[0])


def bench_cache(steps, f):
    """Prefill -> decode cache (path_decode_cache_from_fwd) on the forward workload's workspace.

    Algorithmic bytes per launch: read the key blocks khat (B H Lp d) and the
    block transitions (B H nb d^2) from the forward's records, write the key
    cache (B H L d), read and write the values (2 B H L d), all in bf16."""
    import torch

    import attention_fwd_amd as pa

    x = f["x"]
    B, H, L, d = f["B"], f["H"], f["L"], f["d"]
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], workspace=ws)
    kc = torch.empty((B, H, L, d), device="cuda", dtype=x["q"].dtype)
    vc = torch.empty_like(kc)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        pa.decode_cache_from_fwd(ws, x["v"], kc, vc)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        pa.decode_cache_from_fwd(ws, x["v"], kc, vc)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nb = (L + 63) // 64
    es = kc.element_size()
    nbytes = float(B * H * (nb * 64 * d + nb * d * d + L * d + 2 * L * d) * es)
    del ws, kc, vc
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB_per_s": round(gbs, 1), "bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": read_traffic("path_cache_kernel")}}


def bench_backward(steps, warmup, name=FWD_WORKLOAD):
    """Backward pass (path_attn_bwd) on a forward workload: gradients of q, k, v, w, beta
    for a random upstream gradient, fed the forward's own out and lse."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    c = pathgen.WORKLOADS[name]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    x = pathgen.fwd_inputs(B, H, L, d, c["dtype"], seed=0, fox=c["fox"], clip=c["clip"], device="cuda")
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], return_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(x["q"].dtype)
    ws = torch.empty(pa.bwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["q"]), torch.empty_like(x["q"]), torch.empty_like(x["q"]),
             torch.empty_like(x["beta"]), torch.empty_like(x["beta"]) if x["logf"] is not None else None)
    call = lambda: pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, workspace=ws,
                          grads=grads)
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    heads_per_pass = ws.numel() // pa.bwd_workspace_size(1, 1, L, d, x["q"].dtype)
    del x, out, lse, dout, ws, grads
    torch.cuda.empty_cache()
    flops = 8.0 * B * H * L * L * d
    tf = flops / (ms * 1e-3) / 1e12
    traffic = read_traffic("path_bwd", BWD_TRAFFIC_FILE) if name == FWD_WORKLOAD else None
    res = {"workload": name + " backward", "ms_per_step": round(ms, 3), "flop_per_step": flops,
           "traffic_note": "HBM bytes of one whole backward pass (all kernels, all passes over the workspace)",
           "TFLOP_per_s": round(tf, 2), "steps": steps,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
           "heads_per_workspace_pass": int(heads_per_pass),
           "tokens_per_s": round(B * L / (ms * 1e-3))}
    if traffic:
        # the measured HBM bytes of the pass (counters, while their source hash matches) over its time:
        # the walks materialise per-pair state, so this rate is the other bound to read the time against
        gbs = traffic / (ms * 1e-3) / 1e9
        res["hbm_measured"] = {"GB_per_s": round(gbs, 1), "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def counter_run(fwd_steps=2, dec_steps=2):
    """No timing: the kernels a hardware-counter pass reads.  First a plain
    device copy of COPY_BYTES (read and written once each, the calibration of
    FETCH_SIZE / WRITE_SIZE), then forward steps of the headline workload and
    decode steps of the decode workload."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    src = torch.ones(COPY_BYTES // 2, device="cuda", dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    c = pathgen.WORKLOADS[FWD_WORKLOAD]
    x = pathgen.fwd_inputs(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed=0, fox=c["fox"], clip=c["clip"],
                           device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty(x["beta"].shape, device="cuda", dtype=torch.float32)
    ws = torch.empty(pa.fwd_workspace_size(c["B"], c["H"], c["L"], c["d"], x["q"].dtype), device="cuda",
                     dtype=torch.uint8)
    for _ in range(fwd_steps):
        pa.fwd_prep(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, ws)
        pa.fwd_scan(out, lse, x["logf"] is not None, ws)
    kc = torch.empty_like(x["k"])
    vc = torch.empty_like(x["v"])
    for _ in range(fwd_steps):
        pa.decode_cache_from_fwd(ws, x["v"], kc, vc)
    torch.cuda.synchronize()
    del x, out, lse, ws, kc, vc
    torch.cuda.empty_cache()
    c = pathgen.WORKLOADS[DEC_WORKLOAD]
    x = pathgen.decode_inputs(c["B"], c["H"], c["n"], c["d"], steps=dec_steps, dtype=c["dtype"], seed=0,
                              clip=c["clip"], device="cuda")
    ws = torch.empty(max(pa.decode_workspace_size(c["B"], c["H"], c["n"], c["d"], x["kcache"].dtype), 16),
                     device="cuda", dtype=torch.uint8)
    for t in range(dec_steps):
        pa.decode_step(x["kcache"], x["vcache"], c["n"], x["q"][t], x["w"][t], x["beta"][t], workspace=ws)
    torch.cuda.synchronize()
    log("counter run done: copy %d bytes, %d forward steps + cache builds, %d decode steps" %
        (COPY_BYTES, fwd_steps, dec_steps))


def counter_run_sweep():
    """No timing: the calibration copy (as in counter_run), then one forward (prep + scan) of
    each other forward workload in SWEEP_WORKLOADS order, then one fused-producer forward of the
    headline shape, for rocprofv3 --pmc beyond the headline shape (three dispatches per forward:
    prep, bounded walk, redo)."""
    import torch

    import attention_fwd_amd as pa
    import pathgen

    src = torch.ones(COPY_BYTES // 2, device="cuda", dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for name in SWEEP_WORKLOADS:
        c = pathgen.WORKLOADS[name]
        x = pathgen.fwd_inputs(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed=0, fox=c["fox"], clip=c["clip"],
                               device="cuda")
        out = torch.empty_like(x["q"])
        lse = torch.empty(x["beta"].shape, device="cuda", dtype=torch.float32)
        ws = torch.empty(pa.fwd_workspace_size(c["B"], c["H"], c["L"], c["d"], x["q"].dtype), device="cuda",
                         dtype=torch.uint8)
        pa.fwd_prep(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, ws)
        pa.fwd_scan(out, lse, x["logf"] is not None, ws)
        torch.cuda.synchronize()
        del x, out, lse, ws
        torch.cuda.empty_cache()
        log("counter run: forward %s" % name)
    c = pathgen.WORKLOADS[FWD_WORKLOAD]
    x = pathgen.fused_inputs(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed=0, device="cuda")
    pa.fwd_fused(x["q"], x["k"], x["v"], x["wraw"], x["conv_w"], x["zbeta"], c["clip"])
    torch.cuda.synchronize()
    log("counter run: fused-producer forward %s" % FWD_WORKLOAD)


def counter_run_backward():
    """No timing: the calibration copy (as in counter_run), then one forward and one backward
    pass of the forward workload, for rocprofv3 --pmc over the backward kernels."""
    import torch

    src = torch.ones(COPY_BYTES // 2, device="cuda", dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    bench_backward(1, 0)


def cpu_baseline(x, target_s):
    """The fp64 oracle, as it stands, on whole heads of the forward workload."""
    import oracle

    B, H, L, d = x["q"].shape
    G = B * H
    flat = {k: (v.reshape(G, L, -1) if v.dim() == 4 else v.reshape(G, L)) for k, v in x.items() if v is not None}
    threads = oracle.default_threads()

    def run(nh):
        sel = {k: v[:nh].cpu() for k, v in flat.items()}
        t0 = time.perf_counter()
        oracle.fwd(sel["q"], sel["k"], sel["v"], sel["w"], sel["beta"], nthreads=threads)
        return time.perf_counter() - t0

    nh = 1
    t = run(nh)
    if t < target_s:
        nh = int(min(G, max(1, round(nh * target_s / max(t, 1e-3)))))
        t = run(nh)
    tflops = 4.0 * nh * L * L * d / t / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d heads of the B%d H%d L%d d%d workload, every row, %.1f s" % (nh, G, B, H, L, d, t)}


def cpu_baseline_backward(target_s, name=FWD_WORKLOAD):
    """The fp64 oracle's backward, as it stands, on whole heads of the backward workload (same seeds)."""
    import torch

    import oracle
    import pathgen

    c = pathgen.WORKLOADS[name]
    L, d = c["L"], c["d"]
    threads = oracle.default_threads()

    def run(nh):
        x = pathgen.fwd_inputs(1, nh, L, d, c["dtype"], seed=0, fox=c["fox"], clip=c["clip"], device="cpu")
        dout = torch.randn((1, nh, L, d), generator=torch.Generator().manual_seed(1)).to(x["q"].dtype)
        t0 = time.perf_counter()
        oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], dout, nthreads=threads)
        return time.perf_counter() - t0

    nh = 1
    t = run(nh)
    if t < target_s:
        nh = int(max(1, round(nh * target_s / max(t, 1e-3))))
        t = run(nh)
    tflops = 8.0 * nh * L * L * d / t / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d heads of L%d d%d, every row, %.1f s (work unit 8 L^2 d per head)" % (nh, L, d, t)}


def cpu_baseline_decode(target_s):
    """The fp64 oracle's decode step, as it stands, on whole heads of the decode workload's cache."""
    import oracle
    import pathgen

    c = pathgen.WORKLOADS[DEC_WORKLOAD]
    n, d = c["n"], c["d"]
    threads = oracle.default_threads()

    def run(nh):
        x = pathgen.decode_inputs(1, nh, n, d, steps=1, dtype=c["dtype"], seed=0, clip=c["clip"], device="cpu")
        t0 = time.perf_counter()
        oracle.decode(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], nthreads=threads)
        return time.perf_counter() - t0

    nh = 8
    t = run(nh)
    if t < target_s:
        nh = int(min(c["B"] * c["H"], max(1, round(nh * target_s / max(t, 1e-3)))))
        t = run(nh)
    gbs = 3.0 * nh * n * d * 2 / t / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of the %d heads of the n%d d%d decode workload, one step, %.1f s (bytes counted as on the GPU, bf16)" % (
                nh, c["B"] * c["H"], n, d, t)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline budget; 0 skips it")
    ap.add_argument("--sweep-steps", type=int, default=5, help="timed steps per other forward workload; 0 skips them")
    ap.add_argument("--backward-steps", type=int, default=3, help="timed backward passes; 0 skips them")
    ap.add_argument("--backward-only", action="store_true", help="only the backward leg (for kernel traces)")
    ap.add_argument("--counter-run-backward", action="store_true",
                    help="no timing: a calibration copy plus one backward pass, for rocprofv3 --pmc")
    ap.add_argument("--counter-run-sweep", action="store_true",
                    help="no timing: one forward of each other workload, for rocprofv3 --pmc")
    ap.add_argument("--counter-run", action="store_true",
                    help="no timing: a calibration copy plus a few forward and decode steps, for rocprofv3 --pmc")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the PaTH hot path here has no multi-GPU mode "
              "(heads would shard with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_fwd_amd as pa

    pa.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.counter_run:
        counter_run()
        return
    if args.counter_run_backward:
        counter_run_backward()
        return
    if args.counter_run_sweep:
        counter_run_sweep()
        return
    if args.backward_only:
        print(json.dumps({"backward": bench_backward(max(1, args.backward_steps), 1),
                          "backward_d128": bench_backward(max(1, args.backward_steps), 1, "sweep_L4096_d128_bf16")}),
              flush=True)
        return
    log("forward: %s, %d warm-up + %d timed steps" % (FWD_WORKLOAD, args.warmup, args.steps))
    f = bench_forward(args.steps, args.warmup)
    log("forward: %.3f ms/step (prep %.3f ms, scan %.3f ms)" % (f["ms_per_step"], f["prep_ms"], f["scan_ms"]))
    cache = bench_cache(10, f)
    log("prefill -> decode cache: %.3f ms, %.1f GB/s" % (cache["ms"], cache["GB_per_s"]))
    copy = bench_copy()
    log("device copy: %.1f GB/s (read + write); fill %.1f GB/s (write); sum %.1f GB/s (read); add %.1f GB/s (2 reads + 1 write)"
        % (copy["GB_per_s"], copy["fill_GB_per_s"], copy["read_sum_GB_per_s"], copy["add_2r1w_GB_per_s"]))
    log("decode: %s, %d steps" % (DEC_WORKLOAD, args.decode_steps))
    dres = bench_decode(args.decode_steps)
    log("decode: %.3f ms/step" % dres["step_ms"])
    gres = bench_decode(args.decode_steps, gate=True)
    log("decode with the forget gate: %.3f ms/step" % gres["step_ms"])
    sweep = fox_skip = fused = None
    if args.sweep_steps > 0:
        sweep = bench_sweep(args.sweep_steps, 2)
        fox_skip = bench_fox_skip(args.sweep_steps, 2)
        fused = bench_fused(args.sweep_steps, 2)
        log("fused producer, %s: %.3f ms/step (plain forward %.3f ms)" %
            (fused["workload"], fused["ms_per_step"], fused["plain_forward_ms_per_step"]))
        log("fox workload, skipping negligible blocks: %.3f ms/step (full walk %.3f ms)" %
            (fox_skip["ms_per_step"], fox_skip["full_walk_ms_per_step"]))
    bwd = bwd128 = None
    if args.backward_steps > 0:
        bwd = bench_backward(args.backward_steps, 1)
        log("backward: %.2f ms/step, %.1f TFLOP/s (%.1f%% of the bf16 matrix peak)" %
            (bwd["ms_per_step"], bwd["TFLOP_per_s"], 100 * bwd["roofline"]["frac"]))
        bwd128 = bench_backward(args.backward_steps, 1, "sweep_L4096_d128_bf16")
        log("backward d128: %.2f ms/step, %.1f TFLOP/s" % (bwd128["ms_per_step"], bwd128["TFLOP_per_s"]))
    cpu = dec_cpu = None
    if args.cpu_seconds > 0:
        log("cpu baseline: oracle, ~%.0f s" % args.cpu_seconds)
        cpu = cpu_baseline(f["x"], args.cpu_seconds)
        log("cpu baseline: %s" % cpu["sample"])
        dec_cpu = cpu_baseline_decode(args.cpu_seconds / 3)
        log("cpu baseline, decode: %s" % dec_cpu["sample"])
        if bwd is not None:
            bwd["cpu_baseline"] = cpu_baseline_backward(args.cpu_seconds / 3)
            log("cpu baseline, backward: %s" % bwd["cpu_baseline"]["sample"])

    value = f["flops"] / (f["ms_per_step"] * 1e-3) / 1e12
    scan_tflops = f["flops"] / (f["scan_ms"] * 1e-3) / 1e12
    traffic = read_traffic("path_fwd_kernel")
    mfma_flop = read_mfma_flop("path_fwd_kernel")
    dec_gbs = dres["bytes"] / (dres["step_ms"] * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": FWD_WORKLOAD, "B": f["B"], "H": f["H"], "L": f["L"], "d": f["d"], "causal": True,
                   "decode_workload": DEC_WORKLOAD},
        "roofline": {"bound": "mfma", "kernel": "path_fwd_kernel (scan stage: bounded walk + redo launch)",
                     "achieved": round(scan_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(scan_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "whole_pass_frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "declared_flop_per_launch": f["flops"],
                     "mfma_flop_executed_per_launch": mfma_flop,
                     "executed_over_declared": round(mfma_flop / f["flops"], 4) if mfma_flop else None},
        "forward": {"ms_per_step": round(f["ms_per_step"], 4), "ms_median": round(f["ms_median"], 4),
                    "ms_min": round(f["ms_min"], 4),
                    "TFLOP_per_s_fa_convention": round(2.0 * f["B"] * f["H"] * f["L"] ** 2 * f["d"] /
                                                       (f["ms_per_step"] * 1e-3) / 1e12, 1),
                    "prep_ms": round(f["prep_ms"], 4),
                    "scan_ms": round(f["scan_ms"], 4), "frac_of_peak_whole_pass": round(value / PEAK_BF16_TFLOPS, 4),
                    "tokens_per_s": round(f["B"] * f["L"] / (f["ms_per_step"] * 1e-3)),
                    "flop_per_step": f["flops"]},
        "decode": {"ms_per_step": round(dres["step_ms"], 4), "ms_median": round(dres["ms_median"], 4),
                   "ms_min": round(dres["ms_min"], 4), "GB_per_s": round(dec_gbs, 1),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "traffic": read_traffic("path_decode_kernel")},
                   "tokens_per_s": round(dres["B"] / (dres["step_ms"] * 1e-3)), "bytes_per_step": dres["bytes"],
                   "steps": dres["steps"], "cpu_baseline": dec_cpu},
        "decode_forget_gate": {"ms_per_step": round(gres["step_ms"], 4), "bytes_per_step": gres["bytes"],
                               "GB_per_s": round(gres["bytes"] / (gres["step_ms"] * 1e-3) / 1e9, 1),
                               "frac_of_hbm_peak": round(gres["bytes"] / (gres["step_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "decode_cache_from_fwd": cache,
        "device_copy": copy,
        "other_workloads": sweep,
        "fox_skip_negligible": fox_skip,
        "fused_producer": fused,
        "backward": bwd,
        "backward_d128": bwd128,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
