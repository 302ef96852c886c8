"""GPU parity of path_attn_fwd against the fp64 oracle (through the C ABI).

Tolerances (max-abs, fp32 accumulation in both paths): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs, on the output and on the log-sum-exp.
"""
import math

import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_and_compare(B, H, L, d, dtype, fox, seed, rows=None, heads=None, clip=None, scale=None):
    say("case B%d H%d L%d d%d %s fox=%s seed=%d" % (B, H, L, d, dtype, fox, seed))
    if clip is None and dtype == "bf16":
        clip = 1.98
    x = pathgen.fwd_inputs(B, H, L, d, dtype, seed=seed, fox=fox, clip=clip, device="cuda")
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], scale=scale, return_lse=True)
    torch.cuda.synchronize()
    G = B * H
    flat = {k: (v.reshape(G, L, -1) if v is not None and v.dim() == 4 else (v.reshape(G, L) if v is not None else None))
            for k, v in x.items()}
    heads = list(range(G)) if heads is None else list(heads)
    sel = {k: (v[heads].cpu() if v is not None else None) for k, v in flat.items()}
    o_gpu = out.reshape(G, L, d)[heads].cpu()
    l_gpu = lse.reshape(G, L)[heads].cpu()
    tol = TOL[dtype]
    if rows is None:
        ro, rl = oracle.fwd(sel["q"], sel["k"], sel["v"], sel["w"], sel["beta"], sel["logf"], scale=scale)
        eo, el = max_abs(to_np(o_gpu), ro), max_abs(to_np(l_gpu), rl)
    else:
        r = np.asarray(rows, dtype=np.int64)
        ro, rl = oracle.fwd(sel["q"], sel["k"], sel["v"], sel["w"], sel["beta"], sel["logf"], scale=scale, rows=r)
        og, lg = to_np(o_gpu), to_np(l_gpu)
        eo = max_abs(og[r[:, 0], r[:, 1]], ro)
        el = max_abs(lg[r[:, 0], r[:, 1]], rl)
    say("  max-abs out %.3e  lse %.3e  (tol %.0e)" % (eo, el, tol))
    assert eo <= tol, "output error %.3e > %.0e" % (eo, tol)
    assert el <= tol, "lse error %.3e > %.0e" % (el, tol)
    return out, lse


FP32_CASES = [(1, 2, 64), (1, 1, 1), (1, 1, 2), (1, 2, 63), (1, 1, 65), (2, 1, 128), (1, 2, 200), (1, 1, 257),
              (1, 2, 512), (1, 1, 700)]


@gpu
@pytest.mark.parametrize("B,H,L", FP32_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
def test_fwd_fp32(B, H, L, fox):
    run_and_compare(B, H, L, 64, "f32", fox, seed=1000 + L)


@gpu
def test_fwd_fp32_tiny_workload():
    """The tiny fp32 workload exactly as specified: B1 H2 L64 d64, scale 1/sqrt(d), seed 0, no clip."""
    cfg = pathgen.WORKLOADS["tiny_fp32"]
    run_and_compare(cfg["B"], cfg["H"], cfg["L"], cfg["d"], "f32", False, seed=0, clip=None, scale=0.125)


@gpu
@pytest.mark.parametrize("B,H,L", [(1, 2, 64), (2, 2, 200), (1, 2, 1000), (1, 1, 1), (1, 1, 333), (1, 1, 2048)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
def test_fwd_bf16_small(B, H, L, fox):
    run_and_compare(B, H, L, 64, "bf16", fox, seed=2000 + L)


D128_FP32_CASES = [(1, 2, 64), (1, 1, 1), (1, 1, 65), (1, 2, 200), (2, 1, 257), (1, 1, 700)]


@gpu
@pytest.mark.parametrize("B,H,L", D128_FP32_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
def test_fwd_fp32_d128(B, H, L, fox):
    run_and_compare(B, H, L, 128, "f32", fox, seed=3000 + L)


@gpu
@pytest.mark.parametrize("B,H,L", [(1, 2, 64), (2, 2, 200), (1, 2, 1000), (1, 1, 1), (1, 1, 333), (1, 1, 2048)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
def test_fwd_bf16_d128_small(B, H, L, fox):
    run_and_compare(B, H, L, 128, "bf16", fox, seed=4000 + L)


@gpu
def test_fwd_fp32_beta_extremes():
    """fp32 inputs with beta at the ends of its range: 0 (plain attention), exactly 2 (reflections) and 1
    (projections)."""
    B, H, L, d = 1, 2, 300, 64
    for bval in (0.0, 2.0, 1.0):
        x = pathgen.fwd_inputs(B, H, L, d, "f32", seed=7, device="cuda")
        beta = torch.full((B, H, L), bval, device="cuda")
        say("case beta=%g" % bval)
        out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], beta, return_lse=True)
        ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), beta.cpu())
        assert max_abs(to_np(out), ro) <= 1e-4
        assert max_abs(to_np(lse), rl) <= 1e-4


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bval", [0.0, 1.98], ids=["beta0", "beta1.98"])
@pytest.mark.parametrize("fox", [False, True], ids=["path", "fox"])
def test_fwd_bf16_beta_edges_long(d, bval, fox):
    """bf16 inputs over a long sequence (L = 2048, 32 key blocks) with beta held at an end of the range the
    bf16 workloads use: 0 (every transition is the identity: plain causal attention) and the 1.98 clip
    (near-reflections, where the pages warn that bf16 products of transitions lose accuracy).  Flat bars."""
    B, H, L = 1, 2, 2048
    say("case bf16 beta=%g d%d L%d fox=%s" % (bval, d, L, fox))
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=8 + d, fox=fox, clip=1.98, device="cuda")
    beta = torch.full((B, H, L), bval, device="cuda")
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], beta, x["logf"], return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), beta.cpu(),
                        x["logf"].cpu() if fox else None)
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  max-abs out %.3e  lse %.3e" % (eo, el))
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]


@gpu
@pytest.mark.parametrize("name", ["lm760m_L4096_bf16", "sweep_L1024_d64_bf16", "sweep_L2048_d64_bf16",
                                  "sweep_L4096_d64_bf16", "sweep_L4096_d128_bf16"])
def test_fwd_workload_full_heads(name):
    """Full-size workload; two whole heads (first and last) compared row by row."""
    c = pathgen.WORKLOADS[name]
    G = c["B"] * c["H"]
    run_and_compare(c["B"], c["H"], c["L"], c["d"], c["dtype"], c["fox"], seed=0, heads=[0, G - 1])


@gpu
@pytest.mark.parametrize("name", ["sweep_L8192_d64_bf16", "fox_L16384_bf16"])
def test_fwd_workload_sampled_rows(name):
    """Long workloads: 256 random rows of two heads plus the last 64 rows of each."""
    c = pathgen.WORKLOADS[name]
    G, L = c["B"] * c["H"], c["L"]
    rng = np.random.default_rng(5)
    heads = [int(rng.integers(G)), G - 1]
    rows = [(int(rng.integers(2)), int(rng.integers(L))) for _ in range(256)]
    rows += [(g, L - 1 - t) for g in (0, 1) for t in range(64)]
    run_and_compare(c["B"], c["H"], L, c["d"], c["dtype"], c["fox"], seed=0, heads=heads, rows=rows)


def offset_inputs(L, d, dtype, seed, fox=False):
    """Four heads; in heads 1-3 every logit carries a large common offset while
    the softmax stays well conditioned: the last coordinate of each key is 8
    and of each query is alpha, and every w is orthogonal to that axis, so the
    transitions leave it alone and s_ij = scale (8 alpha + the usual term).
    (The last coordinate is summed last by the matrix cores: the offset then
    costs one rounding of the logit, where earlier it would cost one per added
    term, about sqrt(d) 2^-24 |s| in fp32.)
    With scale = ln(2) / 8 the logits in log2 units are s_ij / 8, and the offset
    8 alpha / 8 = alpha is exact in bf16 after that scaling too (the bf16
    pipeline keeps the scaled queries in bf16; an offset it had to round would
    move the off-diagonal logits against the diagonal block's by 2^-9 of it).
    Head 1: alpha = +150 (2^150 overflows fp32), head 2: alpha = -150 (every
    probability underflows), head 3: alpha = +150 for the queries of the last
    block only.  Head 0 is the plain workload."""
    x = pathgen.fwd_inputs(1, 4, L, d, dtype, seed=seed, fox=fox, clip=1.98 if dtype == "bf16" else None,
                           device="cuda")
    q, k, w = x["q"].float(), x["k"].float(), x["w"].float()
    for hh, alpha, first in ((1, 150.0, 0), (2, -150.0, 0), (3, 150.0, 64 * ((L - 1) // 64))):
        w[0, hh, :, -1] = 0.0
        w[0, hh] = w[0, hh] / w[0, hh].norm(dim=-1, keepdim=True)
        k[0, hh, :, -1] = 8.0
        q[0, hh, :, -1] = 0.0
        q[0, hh, first:, -1] = alpha
    dt = x["q"].dtype
    x["q"], x["k"], x["w"] = q.to(dt).contiguous(), k.to(dt).contiguous(), w.to(dt).contiguous()
    return x


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", ["none", "fox", "fox_skip"])
def test_fwd_large_common_offset(dtype, d, gate):
    """Logits far above or below 0 (overflow / underflow of a walk referenced to
    0) and a head where only one query tile is affected: same bars as any input,
    also under the forget gate, with and without skipping negligible blocks."""
    L = 300
    fox = gate != "none"
    say("case large common logit offset %s d%d L%d gate=%s" % (dtype, d, L, gate))
    x = offset_inputs(L, d, dtype, seed=77 + d, fox=fox)
    scale = math.log(2.0) / 8
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], scale=scale, return_lse=True,
                      skip_negligible=gate == "fox_skip")
    torch.cuda.synchronize()
    G = 4
    ro, rl = oracle.fwd(*(x[n].cpu() for n in ("q", "k", "v", "w", "beta")), x["logf"].cpu() if fox else None,
                        scale=scale)
    eo = max_abs(to_np(out), ro)
    el = max_abs(to_np(lse), rl)
    say("  max-abs out %.3e  lse %.3e  (lse range %.1f .. %.1f)" % (eo, el, float(rl.min()), float(rl.max())))
    assert np.isfinite(to_np(out)).all() and np.isfinite(to_np(lse)).all()
    assert eo <= TOL[dtype], "output error %.3e" % eo
    assert el <= TOL[dtype], "lse error %.3e" % el
    assert G == out.shape[1]


@gpu
def test_fwd_deterministic_and_guarded():
    """Two runs are bitwise equal; nothing is written outside out / lse."""
    B, H, L, d = 2, 3, 777, 64
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=3, fox=True, clip=1.98, device="cuda")
    n = B * H * L * d
    big = torch.full((n + 4096,), 7.0, device="cuda", dtype=torch.bfloat16)
    bigl = torch.full((B * H * L + 1024,), 7.0, device="cuda")
    outs = []
    for _ in range(2):
        out = big[:n].view(B, H, L, d)
        lse = bigl[:B * H * L].view(B, H, L)
        pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out=out, lse=lse)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone()))
        assert torch.all(big[n:] == 7.0) and torch.all(bigl[B * H * L:] == 7.0), "write past the end"
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@gpu
def test_fwd_rejects_bad_arguments_on_device():
    x = pathgen.fwd_inputs(1, 1, 64, 64, "bf16", device="cuda")
    with pytest.raises(pa.PathError):
        pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], workspace=torch.empty(16, device="cuda",
                                                                                  dtype=torch.uint8))
