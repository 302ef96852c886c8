"""GPU parity of path_attn_fwd_fused (producer of w and beta fused into the forward)
against the fp64 oracle's producer + forward, through the C ABI.

Bars: max-abs 1e-4 on out and lse for fp32 inputs, 2e-2 for bf16 inputs (in bf16
the kernel also rounds the convolution output to bf16, inside that budget).
Also: the fused call equals the plain forward fed with the oracle's (w, beta)
rounded to the element type, within the same bars; rows whose convolution window
is all zero (w = 0, H = I); the beta cap.
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_fused(B, H, L, d, dtype, fox, seed, clip, rows=None, prep=None):
    say("case fused B%d H%d L%d d%d %s fox=%s clip=%s seed=%d" % (B, H, L, d, dtype, fox, clip, seed))
    x = pathgen.fused_inputs(B, H, L, d, dtype, seed=seed, fox=fox, device="cuda")
    if prep:
        prep(x)
    out, lse = pa.fwd_fused(x["q"], x["k"], x["v"], x["wraw"], x["conv_w"], x["zbeta"], clip, x["logf"],
                            return_lse=True)
    torch.cuda.synchronize()
    c = {k: (v.cpu() if v is not None else None) for k, v in x.items()}
    if rows is None:
        ro, rl = oracle.fwd_fused(c["q"], c["k"], c["v"], c["wraw"], c["conv_w"], c["zbeta"], clip, c["logf"])
        eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    else:
        r = np.asarray(rows, dtype=np.int64)
        ro, rl = oracle.fwd_fused(c["q"], c["k"], c["v"], c["wraw"], c["conv_w"], c["zbeta"], clip, c["logf"], rows=r)
        G = B * H
        og, lg = to_np(out).reshape(G, L, d), to_np(lse).reshape(G, L)
        eo, el = max_abs(og[r[:, 0], r[:, 1]], ro), max_abs(lg[r[:, 0], r[:, 1]], rl)
    say("  max-abs out %.3e  lse %.3e" % (eo, el))
    assert np.isfinite(to_np(out)).all()
    assert eo <= TOL[dtype] and el <= TOL[dtype], (eo, el)
    return x, out, lse


@gpu
@pytest.mark.parametrize("L", [1, 2, 3, 64, 65, 200, 700])
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_fp32(L, fox, d):
    run_fused(1, 2, L, d, "f32", fox, seed=500 + L, clip=0.0)


@gpu
@pytest.mark.parametrize("L", [64, 333, 2048])
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_bf16(L, fox, d):
    run_fused(2, 2, L, d, "bf16", fox, seed=600 + L, clip=1.98)


@gpu
def test_fused_zero_window_and_cap():
    """Tokens whose convolution window is all zero get w = 0 (identity transition);
    large z drives beta to the cap."""
    def prep(x):
        x["wraw"][0, 1, 100:140] = 0
        x["zbeta"][0, 0, :300] = 9.0
    run_fused(1, 2, 300, 64, "f32", False, seed=7, clip=1.5, prep=prep)


@gpu
def test_fused_equals_plain_forward_on_produced_inputs():
    """The fused call against the plain forward fed with the oracle's (w, beta) rounded
    to the element type (fp32: identical transitions up to fp32 rounding)."""
    B, H, L, d = 1, 2, 260, 64
    x = pathgen.fused_inputs(B, H, L, d, "f32", seed=9, device="cuda")
    w, b = oracle.produce(x["wraw"].cpu(), x["conv_w"].cpu(), x["zbeta"].cpu(), 0.0)
    o1 = pa.fwd_fused(x["q"], x["k"], x["v"], x["wraw"], x["conv_w"], x["zbeta"], 0.0)
    o2 = pa.fwd(x["q"], x["k"], x["v"], torch.from_numpy(w).float().cuda(), torch.from_numpy(b).float().cuda())
    torch.cuda.synchronize()
    e = float((o1 - o2).abs().max())
    say("  fused vs plain on produced inputs: %.3e" % e)
    assert e <= 1e-4


@gpu
def test_fused_headline_shape_sampled_rows():
    """B32 H32 L4096 d64 bf16 with the producer fused: 256 random rows plus the last 64
    rows of two heads against the oracle."""
    B, H, L, d = 32, 32, 4096, 64
    rng = np.random.default_rng(3)
    rows = [(int(g), int(i)) for g, i in zip(rng.integers(0, B * H, 256), rng.integers(0, L, 256))]
    rows += [(g, i) for g in (5, B * H - 1) for i in range(L - 64, L)]
    run_fused(B, H, L, d, "bf16", False, seed=0, clip=1.98, rows=rows)
