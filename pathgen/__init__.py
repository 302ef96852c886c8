"""Seeded synthetic inputs for PaTH attention workloads.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, and both the HIP path's tests/benchmark and the oracle
take their inputs from here.

Distributions (the pages train on real text; these stand-ins have the
shapes and value ranges the method expects):
  q, k, v ~ N(0, 1)
  w_s = z / ||z||, z ~ N(0, I_d)          (unit direction of H_s = I - beta w w^T)
  beta_s = 2 * sigmoid(N(0, 1))           (range (0, 2)), optionally clipped
                                          to <= 1.98 for bf16 inputs, where the
                                          pages advise clipping beta near 2
  log f_s = logsigmoid(N(3, 1))           (forget gate for PaTH-FoX)
Draw order is fixed: q, k, v, w, z_beta, z_f (all fp32, then cast with
round-to-nearest-even to the target dtype).  beta and log f stay fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# Named workloads.  Forward: B, H, L, d; decode: B, H, n (cache rows), d, steps.
WORKLOADS = {
    "tiny_fp32": dict(kind="fwd", B=1, H=2, L=64, d=64, dtype="f32", fox=False, clip=None),
    "lm760m_L4096_bf16": dict(kind="fwd", B=8, H=16, L=4096, d=64, dtype="bf16", fox=False, clip=1.98),
    "sweep_L1024_d64_bf16": dict(kind="fwd", B=32, H=32, L=1024, d=64, dtype="bf16", fox=False, clip=1.98),
    "sweep_L2048_d64_bf16": dict(kind="fwd", B=32, H=32, L=2048, d=64, dtype="bf16", fox=False, clip=1.98),
    "sweep_L4096_d64_bf16": dict(kind="fwd", B=32, H=32, L=4096, d=64, dtype="bf16", fox=False, clip=1.98),
    "sweep_L8192_d64_bf16": dict(kind="fwd", B=32, H=32, L=8192, d=64, dtype="bf16", fox=False, clip=1.98),
    "sweep_L4096_d128_bf16": dict(kind="fwd", B=32, H=32, L=4096, d=128, dtype="bf16", fox=False, clip=1.98),
    "fox_L16384_bf16": dict(kind="fwd", B=4, H=16, L=16384, d=64, dtype="bf16", fox=True, clip=1.98),
    "decode_N32768_bf16": dict(kind="decode", B=16, H=32, n=32768, d=64, dtype="bf16", steps=64, clip=1.98),
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(z):
    return z / torch.linalg.vector_norm(z, dim=-1, keepdim=True)


def fwd_inputs(B, H, L, d, dtype="bf16", seed=0, fox=False, clip=None, device="cpu", fox_mean=3.0):
    """Inputs of one forward pass: dict(q, k, v, w [B,H,L,d] dtype; beta, logf [B,H,L] fp32).

    With fox, logf = logsigmoid(fox_mean + N(0, 1)) (the workloads use fox_mean 3)."""
    tdt = TORCH_DTYPES[dtype]
    g = _gen(device, seed)
    shape = (B, H, L, d)
    f32 = torch.float32
    q = torch.randn(shape, generator=g, device=device, dtype=f32)
    k = torch.randn(shape, generator=g, device=device, dtype=f32)
    v = torch.randn(shape, generator=g, device=device, dtype=f32)
    w = _unit_rows(torch.randn(shape, generator=g, device=device, dtype=f32))
    beta = 2.0 * torch.sigmoid(torch.randn((B, H, L), generator=g, device=device, dtype=f32))
    if clip is not None:
        beta = beta.clamp(max=float(clip))
    logf = None
    if fox:
        logf = torch.nn.functional.logsigmoid(
            float(fox_mean) + torch.randn((B, H, L), generator=g, device=device, dtype=f32))
    out = dict(q=q.to(tdt), k=k.to(tdt), v=v.to(tdt), w=w.to(tdt), beta=beta.contiguous(), logf=logf)
    return out


def fused_inputs(B, H, L, d, dtype="bf16", seed=0, fox=False, device="cpu", fox_mean=3.0):
    """Inputs of a forward pass with the producer of w and beta fused in: dict(q, k, v,
    wraw [B,H,L,d] dtype (all N(0, 1)); zbeta [B,H,L] fp32 N(0, 1) (so beta = 2 sigmoid(z)
    has the workloads' distribution); logf as in fwd_inputs; conv_w [H,d,3] fp32
    N(0, 1/3), a random initialisation of a width-3 depthwise convolution)."""
    tdt = TORCH_DTYPES[dtype]
    g = _gen(device, seed)
    shape = (B, H, L, d)
    f32 = torch.float32
    q = torch.randn(shape, generator=g, device=device, dtype=f32)
    k = torch.randn(shape, generator=g, device=device, dtype=f32)
    v = torch.randn(shape, generator=g, device=device, dtype=f32)
    wraw = torch.randn(shape, generator=g, device=device, dtype=f32)
    zbeta = torch.randn((B, H, L), generator=g, device=device, dtype=f32)
    logf = None
    if fox:
        logf = torch.nn.functional.logsigmoid(
            float(fox_mean) + torch.randn((B, H, L), generator=g, device=device, dtype=f32))
    conv_w = torch.randn((H, d, 3), generator=g, device=device, dtype=f32) / 3.0 ** 0.5
    return dict(q=q.to(tdt), k=k.to(tdt), v=v.to(tdt), wraw=wraw.to(tdt), zbeta=zbeta, logf=logf,
                conv_w=conv_w.contiguous())


def decode_inputs(B, H, n, d, steps, dtype="bf16", seed=0, clip=None, device="cpu", rowcap=None):
    """Inputs of a decode run: cache K, V [B,H,rowcap,d] (rows >= n are zero),
    and per step q, w [steps,B,H,d] dtype, beta [steps,B,H] fp32."""
    tdt = TORCH_DTYPES[dtype]
    g = _gen(device, seed)
    f32 = torch.float32
    rowcap = n if rowcap is None else rowcap
    kc = torch.zeros((B, H, rowcap, d), device=device, dtype=tdt)
    vc = torch.zeros((B, H, rowcap, d), device=device, dtype=tdt)
    kc[:, :, :n] = torch.randn((B, H, n, d), generator=g, device=device, dtype=f32).to(tdt)
    vc[:, :, :n] = torch.randn((B, H, n, d), generator=g, device=device, dtype=f32).to(tdt)
    q = torch.randn((steps, B, H, d), generator=g, device=device, dtype=f32)
    w = _unit_rows(torch.randn((steps, B, H, d), generator=g, device=device, dtype=f32))
    beta = 2.0 * torch.sigmoid(torch.randn((steps, B, H), generator=g, device=device, dtype=f32))
    if clip is not None:
        beta = beta.clamp(max=float(clip))
    return dict(kcache=kc, vcache=vc, q=q.to(tdt), w=w.to(tdt), beta=beta.contiguous())


def workload_inputs(name, seed=0, device="cpu", **over):
    """Inputs of a named workload (optionally overriding any size field)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(over)
    if cfg["kind"] == "fwd":
        return fwd_inputs(cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["dtype"], seed, cfg["fox"], cfg["clip"],
                          device)
    return decode_inputs(cfg["B"], cfg["H"], cfg["n"], cfg["d"], cfg["steps"], cfg["dtype"], seed, cfg["clip"],
                         device)
