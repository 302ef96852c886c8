"""GPU parity of path_attn_bwd (the backward pass) against the fp64 oracle's reverse mode.

The GPU backward is fed the GPU forward's own out and lse (as a training step
would); the oracle recomputes its forward exactly.  Bars, per gradient tensor,
relative to the tensor's largest reference magnitude (gradients are not
normalised the way attention outputs are): max|g - ref| <= tol * max(1, max|ref|)
with tol 1e-4 for fp32 inputs (fp32 arithmetic throughout) and 2e-2 for bf16
inputs (the backward computes in fp32, but its inputs out/lse carry the bf16
forward's rounding and dq, dk, dv, dw are rounded to bf16 on output).
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import say, to_np

gpu = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")


def run_case(B, H, L, dtype, seed, fox, beta=None, with_dlse=True, scale=None, workspace=None, d=64):
    x = pathgen.fwd_inputs(B, H, L, d, dtype, seed=seed, fox=fox, clip=1.98 if dtype == "bf16" else None,
                           device="cuda")
    if beta is not None:
        x["beta"] = torch.full((B, H, L), float(beta), device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 500)
    dout = torch.randn((B, H, L, d), generator=g, device="cuda").to(x["q"].dtype)
    dlse = torch.randn((B, H, L), generator=g, device="cuda") if with_dlse else None
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], scale=scale, return_lse=True)
    grads = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse, scale=scale,
                   workspace=workspace)
    torch.cuda.synchronize()
    return x, dout, dlse, out, lse, grads


def compare(x, dout, dlse, grads, dtype, scale=None, what=""):
    ref = oracle.bwd(*(x[n].cpu() for n in ("q", "k", "v", "w", "beta")), x["logf"].cpu() if x["logf"] is not None
                     else None, dout.cpu(), dlse.cpu() if dlse is not None else None, scale=scale)
    worst = {}
    for n, t in zip(NAMES, grads):
        if t is None:
            assert ref[n] is None
            continue
        r = ref[n]
        e = float(np.abs(to_np(t) - r).max())
        bar = TOL[dtype] * max(1.0, float(np.abs(r).max()))
        worst[n] = e / bar
        assert e <= bar, "%s %s: max-abs %.3e > bar %.3e (max|ref| %.3e)" % (what, n, e, bar, np.abs(r).max())
    say("  %s error / bar: %s" % (what, " ".join("%s %.3f" % kv for kv in worst.items())))


@gpu
@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 130, 200, 333])
def test_bwd_fp32(L, fox):
    say("case bwd fp32 L%d fox=%s" % (L, fox))
    x, dout, dlse, _, _, grads = run_case(1, 2, L, "f32", seed=L, fox=fox)
    compare(x, dout, dlse, grads, "f32", what="L%d" % L)


@gpu
@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("L", [64, 300, 700])
def test_bwd_bf16(L, fox):
    say("case bwd bf16 L%d fox=%s" % (L, fox))
    x, dout, dlse, _, _, grads = run_case(2, 2, L, "bf16", seed=10 + L, fox=fox)
    compare(x, dout, dlse, grads, "bf16", what="L%d" % L)


@gpu
@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_bwd_beta_regimes(beta):
    """beta = 0 (plain softmax attention), 1 (projectors) and 2 (reflections), fp32, without dlse."""
    say("case bwd beta=%g" % beta)
    x, dout, dlse, _, _, grads = run_case(1, 2, 150, "f32", seed=77, fox=True, beta=beta, with_dlse=False)
    compare(x, dout, dlse, grads, "f32", what="beta=%g" % beta)
    if beta == 0.0:
        assert float(grads[3].abs().max()) == 0.0, "dw must vanish at beta = 0"


@gpu
def test_bwd_scale():
    say("case bwd scale 0.3")
    x, dout, dlse, _, _, grads = run_case(2, 1, 257, "f32", seed=5, fox=True, scale=0.3)
    compare(x, dout, dlse, grads, "f32", scale=0.3, what="scale 0.3")


@gpu
def test_bwd_chunked_workspace_and_determinism():
    """A workspace of one head's share (heads one at a time) gives the same bits as all heads at once,
    and repeated calls are bitwise identical."""
    say("case bwd chunked workspace")
    B, H, L = 1, 3, 200
    share = pa.bwd_workspace_size(1, 1, L, 64, torch.float32)
    ws1 = torch.empty(share, device="cuda", dtype=torch.uint8)
    x, dout, dlse, out, lse, g_all = run_case(B, H, L, "f32", seed=9, fox=True)
    g_one = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse, workspace=ws1)
    g_rep = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse)
    torch.cuda.synchronize()
    for n, a, b, c in zip(NAMES, g_all, g_one, g_rep):
        assert torch.equal(a, b), "chunked " + n
        assert torch.equal(a, c), "repeat " + n


@gpu
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_many_heads_short_bf16(d):
    """bf16 with the gate, 255 heads of L = 130 (B5 H51): the walks' work order deals heads to the XCDs in
    groups, here with a head count that is no multiple of the 8 XCDs and walks of one or two steps;
    every element of every head against the oracle."""
    say("case bwd many heads short d%d" % d)
    x, dout, dlse, _, _, grads = run_case(5, 51, 130, "bf16", seed=31 + d, fox=True, d=d)
    compare(x, dout, dlse, grads, "bf16", what="B5 H51 L130 d%d" % d)


@gpu
def test_bwd_uneven_passes_bf16():
    """bf16, five heads through workspaces of two and four heads' shares (passes of 2, 2, 1 and of 4, 1
    heads): the same bits as all heads at once."""
    say("case bwd uneven passes bf16")
    B, H, L = 1, 5, 200
    share = pa.bwd_workspace_size(1, 1, L, 64, torch.bfloat16)
    x, dout, dlse, out, lse, g_all = run_case(B, H, L, "bf16", seed=29, fox=True)
    for n_sh in (2, 4):
        ws = torch.empty(n_sh * share, device="cuda", dtype=torch.uint8)
        g_n = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse, workspace=ws)
        torch.cuda.synchronize()
        for n, a, b in zip(NAMES, g_all, g_n):
            assert torch.equal(a, b), "%d shares: %s" % (n_sh, n)


@gpu
def test_bwd_per_head_workload_shape():
    """One head at the per-head shape of the B32 H32 L4096 d64 bf16 workload, every gradient element."""
    say("case bwd bf16 L4096 one head")
    x, dout, dlse, _, _, grads = run_case(1, 1, 4096, "bf16", seed=3, fox=False)
    compare(x, dout, dlse, grads, "bf16", what="L4096")


@gpu
@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("L", [1, 64, 65, 200, 333])
def test_bwd_fp32_d128(L, fox):
    say("case bwd fp32 d128 L%d fox=%s" % (L, fox))
    x, dout, dlse, _, _, grads = run_case(1, 2, L, "f32", seed=400 + L, fox=fox, d=128)
    compare(x, dout, dlse, grads, "f32", what="d128 L%d" % L)


@gpu
@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("L", [64, 300, 700])
def test_bwd_bf16_d128(L, fox):
    say("case bwd bf16 d128 L%d fox=%s" % (L, fox))
    x, dout, dlse, _, _, grads = run_case(2, 2, L, "bf16", seed=500 + L, fox=fox, d=128)
    compare(x, dout, dlse, grads, "bf16", what="d128 L%d" % L)


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [65, 130, 200, 333])
def test_bwd_bf16_partial_tiles(L, d):
    """bf16 with the gate where the walks' groups of four query blocks are partly idle: 1, 2, 3 and 5
    query blocks past the first (the idle waves store to the spare set and must not disturb the rest)."""
    say("case bwd bf16 partial tiles d%d L%d" % (d, L))
    x, dout, dlse, _, _, grads = run_case(1, 2, L, "bf16", seed=600 + L + d, fox=True, d=d)
    compare(x, dout, dlse, grads, "bf16", what="partial d%d L%d" % (d, L))


@gpu
@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_bwd_beta_regimes_d128(beta):
    """beta = 0, 1 and 2 at head dimension 128, fp32, with the gate."""
    say("case bwd d128 beta=%g" % beta)
    x, dout, dlse, _, _, grads = run_case(1, 1, 150, "f32", seed=78, fox=True, beta=beta, d=128)
    compare(x, dout, dlse, grads, "f32", what="d128 beta=%g" % beta)
    if beta == 0.0:
        assert float(grads[3].abs().max()) == 0.0, "dw must vanish at beta = 0"


@gpu
def test_bwd_per_head_workload_shape_d128():
    """One head at the per-head shape of the B32 H32 L4096 d128 bf16 workload, every gradient element."""
    say("case bwd bf16 d128 L4096 one head")
    x, dout, dlse, _, _, grads = run_case(1, 1, 4096, "bf16", seed=4, fox=False, d=128)
    compare(x, dout, dlse, grads, "bf16", what="d128 L4096")


@gpu
def test_bwd_chunked_workspace_d128():
    """d = 128: a workspace of one head's share gives the same bits as all heads at once."""
    say("case bwd chunked workspace d128")
    B, H, L = 1, 3, 130
    share = pa.bwd_workspace_size(1, 1, L, 128, torch.bfloat16)
    ws1 = torch.empty(share, device="cuda", dtype=torch.uint8)
    x, dout, dlse, out, lse, g_all = run_case(B, H, L, "bf16", seed=19, fox=True, d=128)
    g_one = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse, workspace=ws1)
    torch.cuda.synchronize()
    for n, a, b in zip(NAMES, g_all, g_one):
        assert torch.equal(a, b), "chunked " + n


@gpu
def test_bwd_full_workload_sampled_heads():
    """The whole B32 H32 L4096 d64 bf16 workload through the default workspace (heads in passes over 32 GiB,
    the launch configuration the benchmark times); heads are independent, so the first and the last head
    are checked element by element against the oracle run on that head's inputs alone."""
    c = pathgen.WORKLOADS["sweep_L4096_d64_bf16"]
    B, H, L = c["B"], c["H"], c["L"]
    say("case bwd full workload B%d H%d L%d bf16" % (B, H, L))
    x = pathgen.fwd_inputs(B, H, L, 64, "bf16", seed=0, clip=1.98, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    dout = torch.randn((B, H, L, 64), generator=g, device="cuda").to(torch.bfloat16)
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, return_lse=True)
    grads = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, out, lse, dout)
    torch.cuda.synchronize()
    assert pa.bwd_workspace_size(B, H, L, 64, torch.bfloat16) < B * H * pa.bwd_workspace_size(1, 1, L, 64, torch.bfloat16)
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        ref = oracle.bwd(*(sl(x[n]) for n in ("q", "k", "v", "w", "beta")), None, sl(dout), None)
        for n, t in zip(NAMES, grads):
            if t is None:
                continue
            r = ref[n]
            e = float(np.abs(to_np(t[b:b + 1, h:h + 1]) - r).max())
            bar = TOL["bf16"] * max(1.0, float(np.abs(r).max()))
            assert e <= bar, "head (%d, %d) %s: %.3e > %.3e" % (b, h, n, e, bar)
        say("  head (%d, %d) ok" % (b, h))


@gpu
def test_bwd_full_workload_sampled_heads_d128():
    """The whole B32 H32 L4096 d128 bf16 workload through the default workspace (344 heads per pass over
    32 GiB, as the benchmark times it); the first head, one at a pass boundary and the last head are
    checked element by element against the oracle run on that head's inputs alone."""
    c = pathgen.WORKLOADS["sweep_L4096_d128_bf16"]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    say("case bwd full workload B%d H%d L%d d%d bf16" % (B, H, L, d))
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=0, clip=1.98, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    dout = torch.randn((B, H, L, d), generator=g, device="cuda").to(torch.bfloat16)
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, return_lse=True)
    grads = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, out, lse, dout)
    torch.cuda.synchronize()
    share = pa.bwd_workspace_size(1, 1, L, d, torch.bfloat16)
    per_pass = pa.bwd_workspace_size(B, H, L, d, torch.bfloat16) // share
    assert 1 <= per_pass < B * H
    for flat in (0, per_pass, B * H - 1):
        b, h = divmod(flat, H)
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        ref = oracle.bwd(*(sl(x[n]) for n in ("q", "k", "v", "w", "beta")), None, sl(dout), None)
        for n, t in zip(NAMES, grads):
            if t is None:
                continue
            r = ref[n]
            e = float(np.abs(to_np(t[b:b + 1, h:h + 1]) - r).max())
            bar = TOL["bf16"] * max(1.0, float(np.abs(r).max()))
            assert e <= bar, "head (%d, %d) %s: %.3e > %.3e" % (b, h, n, e, bar)
        say("  head (%d, %d) ok" % (b, h))


@gpu
def test_bwd_long_sequence_fox():
    """One head at the shape of the B4 H16 L16384 d64 bf16 forget-gate workload (256 blocks, 32640 block
    pairs), every gradient element against the oracle."""
    say("case bwd bf16 L16384 fox one head")
    x, dout, dlse, _, _, grads = run_case(1, 1, 16384, "bf16", seed=21, fox=True)
    compare(x, dout, dlse, grads, "bf16", what="L16384 fox")


@gpu
def test_bwd_fp32_many_levels():
    """fp32 with the gate at L = 1500 (24 blocks): the carried queries and the adjoint run 23 levels."""
    say("case bwd fp32 L1500 fox")
    x, dout, dlse, _, _, grads = run_case(1, 1, 1500, "f32", seed=22, fox=True)
    compare(x, dout, dlse, grads, "f32", what="L1500")
