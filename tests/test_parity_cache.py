"""GPU parity of path_decode_cache_from_fwd (prefill -> decode) against the fp64 oracle.

Checks, through the C ABI:
  * the key cache against the oracle's cache after the prefix (row j =
    H_{L-1} ... H_{j+1} k_j): fp32 max-abs <= 1e-4 (the fp32 bar); bf16 per
    row within the error budget of the bf16 key blocks the forward pass left
    in its workspace (see bf16_cache_bound);
  * the value cache equal to v bit for bit, and rows >= L untouched;
  * end to end: forward over L tokens, the cache, then decode steps for tokens
    L, L+1, ... reproduce the oracle's forward rows (1e-4 fp32, 2e-2 bf16).
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu


def build_cache(x, ncap, fox=False):
    B, H, L, d = x["q"].shape
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, x["q"].dtype), device="cuda", dtype=torch.uint8)
    pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"] if fox else None, workspace=ws)
    sentinel = 7.0
    kc = torch.full((B, H, ncap, d), sentinel, device="cuda", dtype=x["q"].dtype)
    vc = torch.full((B, H, ncap, d), sentinel, device="cuda", dtype=x["q"].dtype)
    pa.decode_cache_from_fwd(ws, x["v"], kc, vc)
    torch.cuda.synchronize()
    assert bool((kc[:, :, L:] == sentinel).all()) and bool((vc[:, :, L:] == sentinel).all()), "rows >= L touched"
    assert torch.equal(vc[:, :, :L], x["v"]), "value cache must equal v"
    return kc, vc


def bf16_cache_bound(k):
    """Allowed per-row 2-norm error of a bf16 cache row against the exact fp64 row.

    The forward pass stores the boundary-adjusted keys khat (and the block
    transitions) in bf16, each element rounded to nearest: a relative error of
    at most 2^-9 per element, so at most 2^-9 ||khat_j|| in 2-norm, and the
    products of transitions that carry a row to the end of the prefix have
    spectral norm <= 1 for beta in [0, 2] (each H is then a contraction), so
    the cached row inherits at most that much.  khat itself comes out of bf16
    matrix-core products with fp32 accumulation (its operands -A^T W and the
    masked K W^T are rounded to bf16 first): a few more relative roundings of
    the same size.  The cache row is finally rounded to bf16 (2^-9 relative).
    With ||khat_j|| <= ||k_j||, 8 units of 2^-9 ||k_j|| cover these terms.
    """
    return 8.0 * 2.0 ** -9 * np.linalg.norm(k, axis=-1)


def check_keys(kc, x, dtype):
    B, H, L, d = x["q"].shape
    G = B * H
    ref = oracle.decode_cache(x["k"].cpu(), x["w"].cpu(), x["beta"].cpu()).reshape(G, L, d)
    got = to_np(kc[:, :, :L].reshape(G, L, d))
    if dtype == "f32":
        e = max_abs(got, ref)
        say("  fp32 key cache max-abs %.2e" % e)
        assert e <= 1e-4
    else:
        err = np.linalg.norm(got - ref, axis=-1)
        bound = bf16_cache_bound(to_np(x["k"].reshape(G, L, d)))
        r = float((err / bound).max())
        say("  bf16 key cache row error / bound %.3f (max-abs %.2e)" % (r, max_abs(got, ref)))
        assert r <= 1.0


def continue_decoding(kc, vc, x, L, T, dtype):
    """Decode tokens L .. T-1 on top of the cache and compare with the oracle's forward rows."""
    B, H, _, d = x["q"].shape
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu())
    tol_o, tol_l = (1e-4, 1e-4) if dtype == "f32" else (2e-2, 1e-2)
    worst = 0.0
    for t in range(L, T):
        sl = (slice(None), slice(None), t)
        o, l = pa.decode_step(kc, vc, t, x["q"][sl].contiguous(), x["w"][sl].contiguous(), x["beta"][sl].contiguous(),
                              k_new=x["k"][sl].contiguous(), v_new=x["v"][sl].contiguous(), return_lse=True)
        torch.cuda.synchronize()
        eo, el = max_abs(to_np(o), ro[:, :, t]), max_abs(to_np(l), rl[:, :, t])
        worst = max(worst, eo)
        assert eo <= tol_o and el <= tol_l, "decode step %d after the cache: out %.2e lse %.2e" % (t, eo, el)
    say("  decode after cache, tokens %d..%d: max-abs out %.2e" % (L, T - 1, worst))


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200, 333])
def test_cache_fp32(L, d):
    say("case cache fp32 L%d d%d" % (L, d))
    T = L + 3
    x = pathgen.fwd_inputs(1, 2, T, d, "f32", seed=100 + L, device="cuda")
    xp = {k: (v[:, :, :L].contiguous() if v is not None else None) for k, v in x.items()}
    kc, vc = build_cache(xp, T)
    check_keys(kc, xp, "f32")
    continue_decoding(kc, vc, x, L, T, "f32")


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 64, 130, 700, 2048])
def test_cache_bf16(L, d):
    say("case cache bf16 L%d d%d" % (L, d))
    T = L + 3
    x = pathgen.fwd_inputs(2, 2, T, d, "bf16", seed=200 + L, clip=1.98, device="cuda")
    xp = {k: (v[:, :, :L].contiguous() if v is not None else None) for k, v in x.items()}
    kc, vc = build_cache(xp, T + 5)
    check_keys(kc, xp, "bf16")
    continue_decoding(kc, vc, x, L, T, "bf16")


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [64, 333])
def test_cache_fox_prefill_then_decode(L, dtype):
    """PaTH-FoX prefix: the gate cache holds the prefix sums of log f, and gated decode steps on
    top of the caches reproduce the oracle's PaTH-FoX forward rows."""
    say("case cache fox %s L%d" % (dtype, L))
    T = L + 3
    x = pathgen.fwd_inputs(1, 2, T, 64, dtype, seed=400 + L, fox=True, clip=1.98 if dtype == "bf16" else None,
                           device="cuda")
    xp = {k: v[:, :, :L].contiguous() for k, v in x.items()}
    B, H, _, d = xp["q"].shape
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, xp["q"].dtype), device="cuda", dtype=torch.uint8)
    pa.fwd(xp["q"], xp["k"], xp["v"], xp["w"], xp["beta"], xp["logf"], workspace=ws)
    kc = torch.zeros((B, H, T, d), device="cuda", dtype=xp["q"].dtype)
    vc = torch.zeros_like(kc)
    fc = torch.zeros((B, H, T), device="cuda")
    pa.decode_cache_from_fwd(ws, xp["v"], kc, vc, logf=xp["logf"], fcache=fc)
    torch.cuda.synchronize()
    _, rfc = oracle.decode_cache(xp["k"].cpu(), xp["w"].cpu(), xp["beta"].cpu(), logf=xp["logf"].cpu())
    ef = max_abs(to_np(fc[:, :, :L]), rfc)
    assert ef <= 1e-5 * max(1.0, float(np.abs(rfc).max())), "gate cache %.2e" % ef
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu(), x["logf"].cpu())
    tol = 1e-4 if dtype == "f32" else 2e-2
    for t in range(L, T):
        sl = (slice(None), slice(None), t)
        o, l = pa.decode_step(kc, vc, t, x["q"][sl].contiguous(), x["w"][sl].contiguous(), x["beta"][sl].contiguous(),
                              k_new=x["k"][sl].contiguous(), v_new=x["v"][sl].contiguous(), return_lse=True,
                              logf=x["logf"][sl].contiguous(), fcache=fc)
        torch.cuda.synchronize()
        eo, el = max_abs(to_np(o), ro[:, :, t]), max_abs(to_np(l), rl[:, :, t])
        assert eo <= tol and el <= tol, "gated decode step %d after the cache: %.2e %.2e" % (t, eo, el)
    say("  gate cache %.2e; gated decode after cache ok" % ef)


@gpu
def test_cache_after_fox_forward():
    """The forget gate changes only the logits, not the key blocks: the cache is the same."""
    say("case cache after a PaTH-FoX forward")
    x = pathgen.fwd_inputs(1, 2, 300, 64, "bf16", seed=7, fox=True, clip=1.98, device="cuda")
    kc1, _ = build_cache(x, 300, fox=True)
    kc2, _ = build_cache(x, 300, fox=False)
    assert torch.equal(kc1, kc2)


@gpu
def test_cache_full_workload_sampled_heads():
    """B32 H32 L4096 d64 bf16: build every head's cache, check two heads' keys and one decode step."""
    c = pathgen.WORKLOADS["sweep_L4096_d64_bf16"]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    say("case cache full workload B%d H%d L%d" % (B, H, L))
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=0, clip=1.98, device="cuda")
    kc, vc = build_cache(x, L + 1)
    G = B * H
    for g in (0, G - 1):
        b, hh = divmod(g, H)
        xs = {k: (v[b:b + 1, hh:hh + 1] if v is not None else None) for k, v in x.items()}
        check_keys(kc[b:b + 1, hh:hh + 1], xs, "bf16")
