"""Seeded randomized GPU parity across the C ABI: shapes, dtypes, the forget gate,
skipping, scales and beta regimes drawn at random (fixed seeds), each case against
the fp64 oracle at the usual bars (max-abs 1e-4 for fp32 inputs, 2e-2 for bf16;
decode as in test_parity_decode: fp32 cache 1e-5, bf16 output 2e-2 absolute and
relative to max|o|, lse 1e-2).  For bf16 the forward bar is stated at the default
logit scale 1/sqrt(d): the bf16 rounding of the operands puts an error into each logit
proportional to the scale, so at a scale above the default the bar grows by
scale*sqrt(d).  The backward cases use the backward's bars (relative to each gradient
tensor's largest reference magnitude).  Complements the hand-picked cases of the other
parity tests with combinations nobody chose."""
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


def fwd_case(seed):
    r = np.random.default_rng(1000 + seed)
    return dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), L=int(r.integers(1, 701)),
                d=int(r.choice([64, 128])), dtype=str(r.choice(["f32", "bf16"])), fox=bool(r.integers(0, 2)),
                skip=bool(r.integers(0, 2)), scale=float(r.choice([0.0, r.uniform(0.05, 0.3)])),
                beta=str(r.choice(["sigmoid", "uniform", "zero", "two"])))


@gpu
@pytest.mark.parametrize("seed", range(24))
def test_random_forward(seed):
    c = fwd_case(seed)
    B, H, L, d, dt = c["B"], c["H"], c["L"], c["d"], c["dtype"]
    if dt == "bf16" and c["beta"] == "two":
        c["beta"] = "uniform"  # beta = 2 exactly is the bf16 instability the pages clip against
    say("case random fwd %d: %s" % (seed, c))
    x = pathgen.fwd_inputs(B, H, L, d, dt, seed=seed, fox=c["fox"], clip=1.98 if dt == "bf16" else None,
                           device="cuda")
    if c["beta"] != "sigmoid":
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        hi = 1.98 if dt == "bf16" else 2.0
        x["beta"] = {"uniform": torch.rand((B, H, L), generator=g, device="cuda") * hi,
                     "zero": torch.zeros((B, H, L), device="cuda"),
                     "two": torch.full((B, H, L), 2.0, device="cuda")}[c["beta"]].contiguous()
    scale = c["scale"] if c["scale"] > 0 else None
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], scale=scale, return_lse=True,
                      skip_negligible=c["fox"] and c["skip"])
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(*(x[n].cpu() for n in ("q", "k", "v", "w", "beta")),
                        x["logf"].cpu() if c["fox"] else None, scale=scale)
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    tol = TOL[dt] * (max(1.0, c["scale"] * math.sqrt(d)) if dt == "bf16" else 1.0)
    say("  max-abs out %.3e  lse %.3e  (bar %.3e)" % (eo, el, tol))
    assert eo <= tol and el <= tol


@gpu
@pytest.mark.parametrize("seed", range(8))
def test_random_fused(seed):
    r = np.random.default_rng(2000 + seed)
    B, H, L = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(1, 500))
    d, dt, fox = int(r.choice([64, 128])), str(r.choice(["f32", "bf16"])), bool(r.integers(0, 2))
    clip = 1.98 if dt == "bf16" else float(r.choice([0.0, 1.9]))
    say("case random fused %d: B%d H%d L%d d%d %s fox=%s clip=%g" % (seed, B, H, L, d, dt, fox, clip))
    x = pathgen.fused_inputs(B, H, L, d, dt, seed=seed, fox=fox, device="cuda")
    out, lse = pa.fwd_fused(x["q"], x["k"], x["v"], x["wraw"], x["conv_w"], x["zbeta"], clip, x["logf"],
                            return_lse=True)
    torch.cuda.synchronize()
    c = {k: (v.cpu() if v is not None else None) for k, v in x.items()}
    ro, rl = oracle.fwd_fused(c["q"], c["k"], c["v"], c["wraw"], c["conv_w"], c["zbeta"], clip, c["logf"])
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  max-abs out %.3e  lse %.3e" % (eo, el))
    assert eo <= TOL[dt] and el <= TOL[dt]


@gpu
@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    r = np.random.default_rng(3000 + seed)
    B, H, n, d = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(0, 3000)), int(r.choice([64, 128]))
    dt, append, gate = str(r.choice(["f32", "bf16"])), bool(r.integers(0, 2)), bool(r.integers(0, 2))
    if n == 0:
        append = True  # an empty cache needs the new token to attend to
    ncap = n + 1 + int(r.integers(0, 5))
    say("case random decode %d: B%d H%d n%d ncap%d d%d %s append=%s gate=%s" % (seed, B, H, n, ncap, d, dt, append, gate))
    x = pathgen.decode_inputs(B, H, n, d, steps=2, dtype=dt, seed=seed, clip=1.98 if dt == "bf16" else None,
                              device="cuda", rowcap=ncap)
    fc = lf = None
    if gate:
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        lfs = torch.nn.functional.logsigmoid(3.0 + torch.randn((B, H, ncap + 1), generator=g, device="cuda"))
        fc = torch.zeros((B, H, ncap), device="cuda")
        fc[:, :, :n] = torch.cumsum(lfs[:, :, :n].double(), dim=-1).float()
        lf = lfs[:, :, n].contiguous()
    kn = x["q"][1].clone() if append else None
    vn = x["w"][1].clone() if append else None
    kc0, vc0 = x["kcache"].cpu(), x["vcache"].cpu()
    fc0 = fc.cpu() if gate else None
    out, lse = pa.decode_step(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], k_new=kn, v_new=vn,
                              return_lse=True, logf=lf, fcache=fc)
    torch.cuda.synchronize()
    res = oracle.decode(kc0, vc0, n, x["q"][0].cpu(), x["w"][0].cpu(), x["beta"][0].cpu(),
                        k_new=kn.cpu() if append else None, v_new=vn.cpu() if append else None,
                        logf=lf.cpu() if gate else None, fcache=fc0)
    rk, ro, rl = res[0], res[2], res[3]
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  max-abs out %.3e  lse %.3e" % (eo, el))
    if dt == "f32":
        assert eo <= 1e-4 and el <= 1e-4
        assert max_abs(to_np(x["kcache"][:, :, :n]), rk[:, :, :n]) <= 1e-5
    else:
        assert eo <= 2e-2 and eo <= 2e-2 * max(1.0, float(np.abs(ro).max())) and el <= 1e-2


@gpu
@pytest.mark.parametrize("seed", range(8))
def test_random_decode_fused(seed):
    """path_decode_step_fused on random shapes: the oracle's producer on the raw rows (the state drawn at
    random or zero, as before a sequence's first token) followed by oracle.decode, at the decode bars."""
    r = np.random.default_rng(3500 + seed)
    B, H, n, d = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(0, 3000)), int(r.choice([64, 128]))
    dt, append, gate = str(r.choice(["f32", "bf16"])), bool(r.integers(0, 2)), bool(r.integers(0, 2))
    zero_state, clip = bool(r.integers(0, 2)), float(r.choice([0.0, r.uniform(1.0, 2.0)]))
    if n == 0:
        append = True
    ncap = n + 1 + int(r.integers(0, 5))
    say("case random fused decode %d: B%d H%d n%d d%d %s append=%s gate=%s zero_state=%s clip=%g" % (
        seed, B, H, n, d, dt, append, gate, zero_state, clip))
    tdt = pathgen.TORCH_DTYPES[dt]
    x = pathgen.decode_inputs(B, H, n, d, steps=2, dtype=dt, seed=seed + 40, device="cuda", rowcap=ncap)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 41)
    raw = torch.randn((B, H, 3, d), generator=g, device="cuda").to(tdt)
    if zero_state:
        raw[:, :, :2] = 0
    conv_w = (torch.randn((H, d, 3), generator=g, device="cuda") / 3.0 ** 0.5).contiguous()
    zb = torch.randn((B, H, 3), generator=g, device="cuda")
    state = raw[:, :, :2].clone()  # a copy: the step moves it on in place
    fc = lf = None
    if gate:
        lfs = torch.nn.functional.logsigmoid(3.0 + torch.randn((B, H, ncap + 1), generator=g, device="cuda"))
        fc = torch.zeros((B, H, ncap), device="cuda")
        fc[:, :, :n] = torch.cumsum(lfs[:, :, :n].double(), dim=-1).float()
        lf = lfs[:, :, n].contiguous()
    kn = x["q"][1].clone() if append else None
    vn = x["w"][1].clone() if append else None
    kc0, vc0 = x["kcache"].cpu(), x["vcache"].cpu()
    fc0 = fc.cpu() if gate else None
    out, lse = pa.decode_step_fused(x["kcache"], x["vcache"], n, x["q"][0], raw[:, :, 2].contiguous(), conv_w,
                                    zb[:, :, 2].contiguous(), state, beta_clip=clip, k_new=kn, v_new=vn,
                                    return_lse=True, logf=lf, fcache=fc)
    torch.cuda.synchronize()
    w_ref, b_ref = oracle.produce(raw.cpu(), conv_w.cpu(), zb.cpu(), clip)
    res = oracle.decode(kc0, vc0, n, x["q"][0].cpu(), w_ref[:, :, 2], b_ref[:, :, 2],
                        k_new=kn.cpu() if append else None, v_new=vn.cpu() if append else None,
                        logf=lf.cpu() if gate else None, fcache=fc0)
    ro, rl = res[2], res[3]
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  max-abs out %.3e  lse %.3e" % (eo, el))
    if dt == "f32":
        assert eo <= 1e-4 and el <= 1e-4
    else:
        assert eo <= 2e-2 and eo <= 2e-2 * max(1.0, float(np.abs(ro).max())) and el <= 1e-2
    assert torch.equal(state, raw[:, :, 1:3])


@gpu
@pytest.mark.parametrize("seed", range(6))
def test_random_cache(seed):
    r = np.random.default_rng(4000 + seed)
    B, H, L, d = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 400)), int(r.choice([64, 128]))
    fox = bool(r.integers(0, 2))
    say("case random cache %d: B%d H%d L%d d%d fp32 fox=%s" % (seed, B, H, L, d, fox))
    x = pathgen.fwd_inputs(B, H, L, d, "f32", seed=seed, fox=fox, device="cuda")
    ws = torch.empty(pa.fwd_workspace_size(B, H, L, d, torch.float32), device="cuda", dtype=torch.uint8)
    pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], workspace=ws)
    ncap = L + int(r.integers(0, 4))
    kc = torch.zeros((B, H, ncap, d), device="cuda")
    vc = torch.zeros_like(kc)
    fc = torch.zeros((B, H, ncap), device="cuda") if fox else None
    pa.decode_cache_from_fwd(ws, x["v"], kc, vc, logf=x["logf"], fcache=fc)
    torch.cuda.synchronize()
    ref = oracle.decode_cache(x["k"].cpu(), x["w"].cpu(), x["beta"].cpu(), logf=x["logf"].cpu() if fox else None)
    rk = ref[0] if fox else ref
    e = max_abs(to_np(kc[:, :, :L]), rk)
    say("  key cache max-abs %.3e" % e)
    assert e <= 1e-4
    assert torch.equal(vc[:, :, :L], x["v"])
    if fox:
        assert max_abs(to_np(fc[:, :, :L]), ref[1]) <= 1e-5 * max(1.0, float(np.abs(ref[1]).max()))


@gpu
@pytest.mark.parametrize("seed", range(14))
def test_random_backward(seed):
    """path_attn_bwd on random shapes and regimes (head dimension 64 or 128): every gradient element against
    the oracle's reverse mode, bars as in test_parity_bwd (relative to the tensor's largest magnitude)."""
    r = np.random.default_rng(5000 + seed)
    B, H, L = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 600))
    dt, fox, with_dlse = str(r.choice(["f32", "bf16"])), bool(r.integers(0, 2)), bool(r.integers(0, 2))
    scale = float(r.choice([0.0, r.uniform(0.05, 0.2)]))
    breg = str(r.choice(["sigmoid", "uniform", "zero"]))
    d = int(r.choice([64, 128]))
    say("case random bwd %d: B%d H%d L%d d%d %s fox=%s dlse=%s scale=%g beta=%s" % (seed, B, H, L, d, dt, fox,
                                                                                  with_dlse, scale, breg))
    x = pathgen.fwd_inputs(B, H, L, d, dt, seed=seed, fox=fox, clip=1.98 if dt == "bf16" else None, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 900)
    if breg != "sigmoid":
        x["beta"] = (torch.rand((B, H, L), generator=g, device="cuda") * (1.98 if dt == "bf16" else 2.0)
                     if breg == "uniform" else torch.zeros((B, H, L), device="cuda"))
    dout = torch.randn((B, H, L, d), generator=g, device="cuda").to(x["q"].dtype)
    dlse = torch.randn((B, H, L), generator=g, device="cuda") if with_dlse else None
    sc = scale if scale > 0 else None
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], scale=sc, return_lse=True)
    grads = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], out, lse, dout, dlse, scale=sc)
    torch.cuda.synchronize()
    ref = oracle.bwd(*(x[n].cpu() for n in ("q", "k", "v", "w", "beta")),
                     x["logf"].cpu() if fox else None, dout.cpu(), dlse.cpu() if with_dlse else None, scale=sc)
    tol = TOL[dt] * (max(1.0, scale * math.sqrt(d)) if dt == "bf16" else 1.0)
    worst = []
    for n, t in zip(("dq", "dk", "dv", "dw", "dbeta", "dlogf"), grads):
        if t is None:
            continue
        e = float(np.abs(to_np(t) - ref[n]).max()) / max(1.0, float(np.abs(ref[n]).max()))
        worst.append("%s %.2e" % (n, e))
        assert e <= tol, "%s relative error %.3e > %.1e" % (n, e, tol)
    say("  " + " ".join(worst))
