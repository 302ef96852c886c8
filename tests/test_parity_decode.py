"""GPU parity of path_decode_step against the fp64 oracle (through the C ABI).

Checks: the in-place cache update (fp32: 1e-5; bf16: within one bf16 ulp plus
the fp32 forward-error bound of evaluating k - beta (w.k) w, against the
oracle's fp64 update of the same pre-step cache), the output
(1e-4 fp32 / 2e-2 bf16 max-abs, and 2e-2 relative to max |o| for bf16), the
log-sum-exp (1e-4 fp32 / 1e-2 bf16), and decode reproducing the forward pass.
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import bf16_ulp_distance, cache_update_bound, max_abs, say, to_np

gpu = pytest.mark.gpu


def step_and_check(kc, vc, n, q, w, beta, kn=None, vn=None, heads=None, dtype="bf16", scale=None):
    B, H, ncap, d = kc.shape
    G = B * H
    heads = list(range(G)) if heads is None else heads
    kc_before = kc.reshape(G, ncap, d)[heads].cpu()
    vc_before = vc.reshape(G, ncap, d)[heads].cpu()
    out, lse = pa.decode_step(kc, vc, n, q, w, beta, k_new=kn, v_new=vn, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    qs, ws = q.reshape(G, d)[heads].cpu(), w.reshape(G, d)[heads].cpu()
    bs = beta.reshape(G)[heads].cpu()
    kns = kn.reshape(G, d)[heads].cpu() if kn is not None else None
    vns = vn.reshape(G, d)[heads].cpu() if vn is not None else None
    rk, rv, ro, rl = oracle.decode(kc_before, vc_before, n, qs, ws, bs, k_new=kns, v_new=vns, scale=scale)
    rows = n + (1 if kn is not None else 0)
    kc_after = kc.reshape(G, ncap, d)[heads].cpu()
    og = to_np(out.reshape(G, d)[heads])
    lg = to_np(lse.reshape(G)[heads])
    eo, el = max_abs(og, ro), max_abs(lg, rl)
    if dtype == "f32":
        ek = max_abs(to_np(kc_after[:, :rows]), rk[:, :rows])
        say("  fp32 cache %.2e out %.2e lse %.2e" % (ek, eo, el))
        assert ek <= 1e-5 and eo <= 1e-4 and el <= 1e-4
    else:
        kb = to_np(kc_before[:, :n])
        bound = cache_update_bound(kb, to_np(ws), to_np(bs), rk[:, :n])
        err = np.abs(to_np(kc_after[:, :n]) - rk[:, :n])
        ratio = float((err / bound).max()) if n else 0.0
        ulp = bf16_ulp_distance(kc_after[:, :n], torch.from_numpy(rk[:, :n]).float().to(torch.bfloat16))
        rel = eo / max(float(np.abs(ro).max()), 1e-30)
        say("  bf16 cache err/bound %.3f (max ulp distance %d) out %.2e (rel %.2e) lse %.2e" % (ratio, ulp, eo, rel, el))
        assert ratio <= 1.0, "cache update outside the fp32-evaluation + 1 ulp bound (ratio %.3f)" % ratio
        if kn is not None:
            assert torch.equal(kc_after[:, n], kns.to(kc_after.dtype)), "appended key must be stored as given"
        assert eo <= 2e-2 and rel <= 2e-2 and el <= 1e-2
    # rows past the attended range are untouched
    assert torch.equal(kc_after[:, rows:], kc_before[:, rows:])
    assert torch.equal(vc.reshape(G, ncap, d)[heads].cpu()[:, rows:], vc_before[:, rows:])
    return out, lse


@gpu
@pytest.mark.parametrize("n", [1, 7, 128, 1000, 4097])
@pytest.mark.parametrize("append", [False, True], ids=["cache", "append"])
def test_decode_fp32(n, append):
    B, H, d = 2, 3, 64
    say("case decode fp32 n=%d append=%s" % (n, append))
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="f32", seed=n, device="cuda", rowcap=n + 1)
    kn = vn = None
    if append:
        kn = torch.randn(B, H, d, device="cuda")
        vn = torch.randn(B, H, d, device="cuda")
    step_and_check(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], kn, vn, dtype="f32")


@gpu
@pytest.mark.parametrize("n,append", [(4096, False), (333, True), (70000, False)])
def test_decode_bf16(n, append):
    B, H, d = 2, 4, 64
    say("case decode bf16 n=%d append=%s" % (n, append))
    x = pathgen.decode_inputs(B, H, n, d, steps=3, dtype="bf16", seed=11, clip=1.98, device="cuda",
                              rowcap=n + 3)
    for t in range(3):
        kn = vn = None
        rows = n + (t if append else 0)
        if append:
            kn = torch.randn(B, H, d, device="cuda").to(torch.bfloat16)
            vn = torch.randn(B, H, d, device="cuda").to(torch.bfloat16)
        step_and_check(x["kcache"], x["vcache"], rows, x["q"][t], x["w"][t], x["beta"][t], kn, vn)


@gpu
@pytest.mark.parametrize("n,append", [(1, False), (7, True), (1000, False), (4097, True)])
def test_decode_fp32_d128(n, append):
    B, H, d = 2, 3, 128
    say("case decode fp32 d128 n=%d append=%s" % (n, append))
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="f32", seed=50 + n, device="cuda", rowcap=n + 1)
    kn = vn = None
    if append:
        kn = torch.randn(B, H, d, device="cuda")
        vn = torch.randn(B, H, d, device="cuda")
    step_and_check(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], kn, vn, dtype="f32")


@gpu
@pytest.mark.parametrize("n,append", [(4096, False), (333, True)])
def test_decode_bf16_d128(n, append):
    B, H, d = 2, 4, 128
    say("case decode bf16 d128 n=%d append=%s" % (n, append))
    x = pathgen.decode_inputs(B, H, n, d, steps=2, dtype="bf16", seed=17, clip=1.98, device="cuda", rowcap=n + 2)
    for t in range(2):
        kn = vn = None
        rows = n + (t if append else 0)
        if append:
            kn = torch.randn(B, H, d, device="cuda").to(torch.bfloat16)
            vn = torch.randn(B, H, d, device="cuda").to(torch.bfloat16)
        step_and_check(x["kcache"], x["vcache"], rows, x["q"][t], x["w"][t], x["beta"][t], kn, vn)


@gpu
def test_decode_bf16_peaky():
    """q scaled x8 so attention concentrates and |o| = O(1): a skipped or wrong update shows clearly."""
    B, H, n, d = 2, 2, 4096, 64
    say("case decode bf16 peaky")
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="bf16", seed=12, clip=1.98, device="cuda")
    q = (x["q"][0].float() * 8).to(torch.bfloat16)
    out, _ = step_and_check(x["kcache"], x["vcache"], n, q, x["w"][0], x["beta"][0])
    assert float(out.float().abs().max()) > 0.3


@gpu
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f32")])
def test_decode_many_splits(d, dtype):
    """One head with 100 000 cached rows and one appended token: the split plan gives it hundreds of
    splits (more than the merge kernel's 256 threads take in one pass, so the maximum is folded over
    several passes and each of the summing groups adds about a hundred partials)."""
    B, H, n = 1, 1, 100000
    say("case decode many splits d%d %s" % (d, dtype))
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype=dtype, seed=23, clip=1.98 if dtype == "bf16" else None,
                              device="cuda", rowcap=n + 1)
    tdt = x["kcache"].dtype
    kn = torch.randn(B, H, d, device="cuda").to(tdt)
    vn = torch.randn(B, H, d, device="cuda").to(tdt)
    step_and_check(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], kn, vn, dtype=dtype)


@gpu
def test_decode_workload_full_size():
    """Full decode workload (B16 H32 n=32768 bf16), two steps, four heads checked."""
    c = pathgen.WORKLOADS["decode_N32768_bf16"]
    say("case decode full size")
    x = pathgen.decode_inputs(c["B"], c["H"], c["n"], c["d"], steps=2, dtype="bf16", seed=0, clip=1.98, device="cuda")
    G = c["B"] * c["H"]
    for t in range(2):
        step_and_check(x["kcache"], x["vcache"], c["n"], x["q"][t], x["w"][t], x["beta"][t], heads=[0, 5, 300, G - 1])


@gpu
def test_decode_workload_64_steps_against_carried_oracle():
    """The whole decode workload as timed: B16 H32, 32768 cached bf16 rows, 64 steps with fresh (q, w, beta),
    every key updated in place each step.  On four heads the oracle keeps its OWN fp64 cache, carried from
    the original bf16 rows through the same 64 steps, so the drift the bf16 cache accumulates (each step
    rounds every key) enters the comparison.  Every step: out within 2e-2 absolute and relative to max|o|,
    lse within 1e-2.  After the last step every key row's 2-norm error against the fp64 row is within
    ((1 + u')^64 - 1) times the original row's 2-norm, u' = 2^-8 (1 + 2^-7): a step rounds each element to
    bf16 (relative error at most 2^-8) and evaluates k - beta (w.k) w in fp32 (well inside the extra 2^-7),
    every transition is a contraction (beta ||w||^2 <= 1.98 (1 + 2^-8) < 2), so an error carried from earlier
    steps does not grow, and the row being rounded is at most the exact row plus that error."""
    c = pathgen.WORKLOADS["decode_N32768_bf16"]
    B, H, n, d, T = c["B"], c["H"], c["n"], c["d"], c["steps"]
    G = B * H
    heads = [0, 5, 300, G - 1]
    say("case decode workload, %d steps, oracle cache carried on heads %s" % (T, heads))
    x = pathgen.decode_inputs(B, H, n, d, steps=T, dtype="bf16", seed=0, clip=1.98, device="cuda")
    kc, vc = x["kcache"], x["vcache"]
    k0 = kc.reshape(G, n, d)[heads].cpu()
    rk = to_np(k0)
    rv = to_np(vc.reshape(G, n, d)[heads])
    worst = dict(out=0.0, rel=0.0, lse=0.0)
    for t in range(T):
        out, lse = pa.decode_step(kc, vc, n, x["q"][t], x["w"][t], x["beta"][t], return_lse=True)
        qs = x["q"][t].reshape(G, d)[heads].cpu()
        ws = x["w"][t].reshape(G, d)[heads].cpu()
        bs = x["beta"][t].reshape(G)[heads].cpu()
        rk, _, ro, rl = oracle.decode(rk, rv, n, qs, ws, bs)
        torch.cuda.synchronize()
        og, lg = to_np(out.reshape(G, d)[heads]), to_np(lse.reshape(G)[heads])
        eo, el = max_abs(og, ro), max_abs(lg, rl)
        rel = eo / max(float(np.abs(ro).max()), 1e-30)
        worst = dict(out=max(worst["out"], eo), rel=max(worst["rel"], rel), lse=max(worst["lse"], el))
        if t in (0, 31, T - 1):
            say("  step %d: out %.2e (rel %.2e) lse %.2e" % (t + 1, eo, rel, el))
        assert eo <= 2e-2 and rel <= 2e-2 and el <= 1e-2, "step %d: out %.3e rel %.3e lse %.3e" % (t + 1, eo, rel, el)
    kg = to_np(kc.reshape(G, n, d)[heads])
    row_err = np.linalg.norm(kg - rk, axis=-1)
    bound = ((1 + 2.0 ** -8 * (1 + 2.0 ** -7)) ** T - 1) * np.linalg.norm(to_np(k0), axis=-1)
    say("  worst over %d steps: out %.2e (rel %.2e) lse %.2e; key drift max-abs %.3e, row 2-norm / bound %.3f"
        % (T, worst["out"], worst["rel"], worst["lse"], float(np.abs(kg - rk).max()), float((row_err / bound).max())))
    assert (row_err <= bound).all()


@gpu
@pytest.mark.parametrize("d", [64, 128])
def test_decode_reproduces_forward_fp32(d):
    """Decoding token by token from an empty cache gives the forward pass's rows."""
    B, H, T = 1, 2, 70
    say("case decode vs forward d%d" % d)
    x = pathgen.fwd_inputs(B, H, T, d, "f32", seed=21, device="cuda")
    fo, fl = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], return_lse=True)
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu())
    kc = torch.zeros(B, H, T, d, device="cuda")
    vc = torch.zeros(B, H, T, d, device="cuda")
    for t in range(T):
        o, l = pa.decode_step(kc, vc, t, x["q"][:, :, t].contiguous(), x["w"][:, :, t].contiguous(),
                              x["beta"][:, :, t].contiguous(), k_new=x["k"][:, :, t].contiguous(),
                              v_new=x["v"][:, :, t].contiguous(), return_lse=True)
        torch.cuda.synchronize()
        assert max_abs(to_np(o), ro[:, :, t]) <= 1e-4, "step %d vs oracle" % t
        assert max_abs(to_np(l), rl[:, :, t]) <= 1e-4
        assert max_abs(to_np(o), to_np(fo[:, :, t])) <= 1e-4, "step %d vs forward kernel" % t


@gpu
def test_decode_deterministic():
    B, H, n, d = 2, 3, 5000, 64
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="bf16", seed=13, clip=1.98, device="cuda")
    res = []
    for _ in range(2):
        kc, vc = x["kcache"].clone(), x["vcache"].clone()
        o, l = pa.decode_step(kc, vc, n, x["q"][0], x["w"][0], x["beta"][0], return_lse=True)
        torch.cuda.synchronize()
        res.append((o, l, kc))
    assert all(torch.equal(a, b) for a, b in zip(res[0], res[1]))


@gpu
def test_decode_checkpoint_resume():
    """Eight steps in one go equal four steps, a host round-trip of the cache, then four more."""
    B, H, n, d = 1, 2, 3000, 64
    x = pathgen.decode_inputs(B, H, n, d, steps=8, dtype="bf16", seed=14, clip=1.98, device="cuda")
    kc1, vc1 = x["kcache"].clone(), x["vcache"].clone()
    outs1 = [pa.decode_step(kc1, vc1, n, x["q"][t], x["w"][t], x["beta"][t]) for t in range(8)]
    kc2, vc2 = x["kcache"].clone(), x["vcache"].clone()
    outs2 = [pa.decode_step(kc2, vc2, n, x["q"][t], x["w"][t], x["beta"][t]) for t in range(4)]
    kc2, vc2 = kc2.cpu().cuda(), vc2.cpu().cuda()
    outs2 += [pa.decode_step(kc2, vc2, n, x["q"][t], x["w"][t], x["beta"][t]) for t in range(4, 8)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs1, outs2)) and torch.equal(kc1, kc2)


def gate_state(B, H, ncap, n, seed):
    """Random gate cache (prefix sums of log f = logsigmoid(3 + N(0,1))) and the current log f."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    lf = torch.nn.functional.logsigmoid(3.0 + torch.randn((B, H, ncap + 1), generator=g, device="cuda"))
    fc = torch.zeros((B, H, ncap), device="cuda")
    fc[:, :, :n] = torch.cumsum(lf[:, :, :n].double(), dim=-1).float()
    return fc, lf[:, :, n].contiguous()


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 130, 2000])
@pytest.mark.parametrize("append", [False, True], ids=["cache", "append"])
def test_decode_fox(dtype, n, append):
    """PaTH-FoX decode against the oracle: out, lse, the in-place key update, the gate cache row n."""
    B, H, d = 2, 2, 64
    say("case decode fox %s n%d append=%s" % (dtype, n, append))
    ncap = n + 1
    x = pathgen.decode_inputs(B, H, n, d, steps=2, dtype=dtype, seed=40 + n, clip=1.98 if dtype == "bf16" else None,
                              device="cuda", rowcap=ncap)
    fc, lf = gate_state(B, H, ncap, n, 50 + n)
    kn = x["q"][1].clone() if append else None  # any [B, H, d] tensor serves as the new key/value
    vn = x["w"][1].clone() if append else None
    kc0, vc0, fc0 = x["kcache"].cpu(), x["vcache"].cpu(), fc.cpu()
    out, lse = pa.decode_step(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], k_new=kn, v_new=vn,
                              return_lse=True, logf=lf, fcache=fc)
    torch.cuda.synchronize()
    rk, _, ro, rl, rfc = oracle.decode(kc0, vc0, n, x["q"][0].cpu(), x["w"][0].cpu(), x["beta"][0].cpu(),
                                        k_new=kn.cpu() if append else None, v_new=vn.cpu() if append else None,
                                        logf=lf.cpu(), fcache=fc0)
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    ek = max_abs(to_np(x["kcache"][:, :, :n]), rk[:, :, :n])
    ef = max_abs(to_np(fc), rfc)
    say("  out %.2e lse %.2e cache %.2e gate cache %.2e" % (eo, el, ek, ef))
    tol_o, tol_l = (1e-4, 1e-4) if dtype == "f32" else (2e-2, 1e-2)
    assert eo <= tol_o and el <= tol_l
    assert ek <= (1e-5 if dtype == "f32" else 3e-2)
    assert ef <= 1e-5 * max(1.0, float(np.abs(rfc).max())), "gate cache row n"


@gpu
def test_decode_fox_reproduces_forward_fp32():
    """PaTH-FoX: decoding token by token from an empty cache gives the forward pass's rows."""
    B, H, T, d = 1, 2, 70, 64
    say("case decode fox vs forward")
    x = pathgen.fwd_inputs(B, H, T, d, "f32", seed=22, fox=True, device="cuda")
    fo = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"])
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu(), x["logf"].cpu())
    kc = torch.zeros(B, H, T, d, device="cuda")
    vc = torch.zeros(B, H, T, d, device="cuda")
    fc = torch.zeros(B, H, T, device="cuda")
    for t in range(T):
        sl = (slice(None), slice(None), t)
        o, l = pa.decode_step(kc, vc, t, x["q"][sl].contiguous(), x["w"][sl].contiguous(), x["beta"][sl].contiguous(),
                              k_new=x["k"][sl].contiguous(), v_new=x["v"][sl].contiguous(), return_lse=True,
                              logf=x["logf"][sl].contiguous(), fcache=fc)
        torch.cuda.synchronize()
        assert max_abs(to_np(o), ro[:, :, t]) <= 1e-4, "step %d vs oracle" % t
        assert max_abs(to_np(l), rl[:, :, t]) <= 1e-4
        assert max_abs(to_np(o), to_np(fo[:, :, t])) <= 1e-4, "step %d vs forward kernel" % t
