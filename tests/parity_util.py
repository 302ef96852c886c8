"""Helpers shared by the GPU parity tests (comparison only; no method arithmetic)."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def max_abs(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    if np.isnan(d).any():
        return float("inf")
    return float(d.max())


def bf16_ulp_distance(a, b):
    """Max distance in bf16 units-in-the-last-place between two bf16 tensors."""
    ia = a.detach().contiguous().view(torch.int16).to(torch.int32)
    ib = b.detach().contiguous().view(torch.int16).to(torch.int32)
    # map sign-magnitude to a monotone integer line
    ia = torch.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = torch.where(ib < 0, -(ib & 0x7FFF), ib)
    return int((ia - ib).abs().max().item()) if ia.numel() else 0


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (float64 array); subnormal spacing near 0."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def cache_update_bound(k_before, w, beta, ref):
    """Allowed |gpu - exact| for k' = k - beta (w.k) w evaluated in fp32 and
    rounded to bf16: one bf16 ulp of the exact value plus the fp32 forward-error
    bound of the evaluation (Higham: |fl(w.k) - w.k| <= gamma_d sum|w_c k_c|,
    gamma_d = d u / (1 - d u), u = 2^-24; then the scale by beta and the
    subtraction add two more roundings)."""
    u = 2.0 ** -24
    d = k_before.shape[-1]
    gamma = d * u / (1 - d * u)
    absdot = np.abs(k_before * w[:, None, :]).sum(-1, keepdims=True)        # [G, n, 1]
    dot = (k_before * w[:, None, :]).sum(-1, keepdims=True)
    bw = np.abs(beta)[:, None, None] * np.abs(w)[:, None, :]               # [G, 1, d]
    e32 = bw * (gamma * absdot + 2 * u * np.abs(dot)) + 2 * u * (np.abs(k_before) + bw * np.abs(dot))
    return bf16_ulp(ref) + e32
