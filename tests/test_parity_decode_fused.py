"""GPU parity of path_decode_step_fused (the decode step with the producer of w and beta
fused in) against the fp64 oracle, through the C ABI.

The oracle side composes the oracle's producer (oracle.produce: the width-3 causal
convolution over the raw rows, L2 normalisation, beta = 2 sigmoid(z), capped) with
oracle.decode, and carries its own fp64 caches from the original ones across the steps.
Bars as in test_parity_decode: fp32 output and lse 1e-4; bf16 output 2e-2 absolute and
relative to max|o|, lse 1e-2.  The convolution state must move on by exactly one raw row
per step.
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu


@gpu
@pytest.mark.parametrize("gate", [False, True], ids=["nogate", "gate"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_fused_steps(dtype, d, gate):
    """Four fused steps after a 100-row cache, each appending its (k, v), the state starting from
    two raw rows of a prefix; every head's output and lse against the oracle at every step."""
    B, H, n0, T = 2, 3, 100, 4
    tdt = pathgen.TORCH_DTYPES[dtype]
    seed = 70 + d + (1 if gate else 0) + (2 if dtype == "bf16" else 0)
    say("case decode fused %s d%d gate=%s" % (dtype, d, gate))
    x = pathgen.decode_inputs(B, H, n0, d, steps=T, dtype=dtype, seed=seed, device="cuda", rowcap=n0 + T)
    kc, vc, q = x["kcache"], x["vcache"], x["q"]
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1000)
    raw = torch.randn((B, H, T + 2, d), generator=g, device="cuda").to(tdt)  # rows t0-2 .. t0+T-1
    conv_w = (torch.randn((H, d, 3), generator=g, device="cuda") / 3.0 ** 0.5).contiguous()
    zb = torch.randn((B, H, T + 2), generator=g, device="cuda")
    kn = torch.randn((T, B, H, d), generator=g, device="cuda").to(tdt)
    vn = torch.randn((T, B, H, d), generator=g, device="cuda").to(tdt)
    clip = 1.98 if dtype == "bf16" else 0.0
    w_ref, b_ref = oracle.produce(raw.cpu(), conv_w.cpu(), zb.cpu(), clip)  # positions 2.. are the steps'
    state = raw[:, :, :2].clone()  # a copy: the step moves it on in place
    logf = fcache = fc_ref = None
    if gate:
        logf = torch.nn.functional.logsigmoid(torch.randn((T, B, H), generator=g, device="cuda") + 3.0)
        fcache = torch.zeros((B, H, n0 + T), device="cuda")
        fcache[:, :, :n0] = torch.cumsum(torch.nn.functional.logsigmoid(
            torch.randn((B, H, n0), generator=g, device="cuda") + 3.0), dim=-1)
        fc_ref = fcache.cpu()
    ok, ov = kc.cpu(), vc.cpu()
    worst = 0.0
    for t in range(T):
        n = n0 + t
        zt = zb[:, :, t + 2].contiguous()
        out, lse = pa.decode_step_fused(kc, vc, n, q[t], raw[:, :, t + 2].contiguous(), conv_w, zt, state,
                                        beta_clip=clip, k_new=kn[t], v_new=vn[t], return_lse=True,
                                        logf=logf[t].contiguous() if gate else None, fcache=fcache)
        torch.cuda.synchronize()
        res = oracle.decode(ok, ov, n, q[t].cpu(), w_ref[:, :, t + 2], b_ref[:, :, t + 2], k_new=kn[t].cpu(),
                            v_new=vn[t].cpu(), logf=logf[t].cpu() if gate else None, fcache=fc_ref)
        ok, ov, ro, rl = res[:4]
        if gate:
            fc_ref = res[4]
        eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
        if dtype == "f32":
            assert eo <= 1e-4 and el <= 1e-4, "step %d: out %.2e lse %.2e" % (t, eo, el)
        else:
            rel = eo / max(float(np.abs(ro).max()), 1e-30)
            assert eo <= 2e-2 and rel <= 2e-2 and el <= 1e-2, "step %d: out %.2e (rel %.2e) lse %.2e" % (t, eo, rel, el)
        worst = max(worst, eo)
        assert torch.equal(state, raw[:, :, t + 1:t + 3]), "the state must hold the last two raw rows"
    say("  worst out error over %d steps %.2e" % (T, worst))


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_fused_zero_rows(dtype):
    """Raw rows and state all zero: y_t = 0, so w_t = 0 and H_t = I; the cache stays bitwise as it was
    and the step is plain attention over it."""
    B, H, n, d = 1, 2, 37, 64
    tdt = pathgen.TORCH_DTYPES[dtype]
    say("case decode fused zero rows %s" % dtype)
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype=dtype, seed=5, device="cuda", rowcap=n)
    kc, vc = x["kcache"], x["vcache"]
    before = kc.clone()
    z = torch.zeros((B, H, d), device="cuda", dtype=tdt)
    state = torch.zeros((B, H, 2, d), device="cuda", dtype=tdt)
    conv_w = torch.ones((H, d, 3), device="cuda")
    zb = torch.zeros((B, H), device="cuda")
    out, lse = pa.decode_step_fused(kc, vc, n, x["q"][0], z, conv_w, zb, state, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(kc, before), "H_t = I must leave the cache as it was"
    _, _, ro, rl = oracle.decode(before.cpu(), vc.cpu(), n, x["q"][0].cpu(), torch.zeros((B, H, d)),
                                 torch.ones((B, H)), scale=None)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert max_abs(to_np(out), ro) <= tol and max_abs(to_np(lse), rl) <= (1e-4 if dtype == "f32" else 1e-2)
