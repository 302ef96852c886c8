"""path_decode_step_noalloc (no workspace; the library's fixed scratch) against
path_decode_step / path_decode_step_ex on identical inputs, through the C ABI:
two calls in a row, the second smaller, so it runs on scratch still holding the
first call's partials.  The two entry points share their kernels and split plan,
so out, lse and the updated caches must be bitwise equal (inside the oracle
bars a fortiori); the first call is also checked against the oracle on a few
heads."""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu


def gate_state(B, H, ncap, n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    lf = torch.nn.functional.logsigmoid(3.0 + torch.randn((B, H, ncap + 1), generator=g, device="cuda"))
    fc = torch.zeros((B, H, ncap), device="cuda")
    fc[:, :, :n] = torch.cumsum(lf[:, :, :n].double(), dim=-1).float()
    return fc, lf[:, :, n].contiguous()


def both(B, H, n, d, dtype, seed, append, gate):
    """Run the same step through the workspace entry point and the no-allocation one."""
    ncap = n + (1 if append else 0)
    x = pathgen.decode_inputs(B, H, n, d, steps=2, dtype=dtype, seed=seed, clip=1.98 if dtype == "bf16" else None,
                              device="cuda", rowcap=ncap)
    kn = x["q"][1].clone() if append else None
    vn = x["w"][1].clone() if append else None
    fc, lf = gate_state(B, H, ncap, n, seed + 1) if gate else (None, None)
    res = {}
    for which in ("workspace", "noalloc"):
        kc, vc = x["kcache"].clone(), x["vcache"].clone()
        f = fc.clone() if gate else None
        out = torch.empty((B, H, d), device="cuda", dtype=kc.dtype)
        lse = torch.empty((B, H), device="cuda")
        torch.cuda.synchronize()
        if which == "workspace":
            pa.decode_step(kc, vc, n, x["q"][0], x["w"][0], x["beta"][0], k_new=kn, v_new=vn, out=out, lse=lse,
                           logf=lf, fcache=f)
        else:
            pa.decode_step_noalloc(kc, vc, n, x["q"][0], x["w"][0], x["beta"][0], out, k_new=kn, v_new=vn, lse=lse,
                                   logf=lf, fcache=f)
        torch.cuda.synchronize()
        res[which] = (out, lse, kc, vc, f)
    return x, res, (kn, vn, fc, lf)


def assert_equal(res):
    a, b = res["workspace"], res["noalloc"]
    for name, s, t in zip(("out", "lse", "kcache", "vcache", "fcache"), a, b):
        if s is None:
            assert t is None
            continue
        assert torch.equal(s, t), "%s differs between the two entry points" % name


@gpu
def test_noalloc_matches_workspace_entry_point():
    # call 1: the decode workload (B16 H32, 32768 cached bf16 rows), forget gate on
    c = pathgen.WORKLOADS["decode_N32768_bf16"]
    B, H, n, d = c["B"], c["H"], c["n"], c["d"]
    say("case noalloc call 1: B%d H%d n%d d%d bf16, gate" % (B, H, n, d))
    x, res, (kn, vn, fc, lf) = both(B, H, n, d, "bf16", seed=60, append=False, gate=True)
    assert_equal(res)
    G = B * H
    heads = [0, 7, G - 1]
    sel = lambda t, shape: t.reshape(shape)[heads].cpu()
    _, _, ro, rl, _ = oracle.decode(sel(x["kcache"], (G, n, d)), sel(x["vcache"], (G, n, d)), n,
                                    sel(x["q"][0], (G, d)), sel(x["w"][0], (G, d)), sel(x["beta"][0], (G,)),
                                    logf=sel(lf, (G,)), fcache=sel(fc, (G, n)))
    out, lse = res["noalloc"][0], res["noalloc"][1]
    eo = max_abs(to_np(out.reshape(G, d)[heads]), ro)
    el = max_abs(to_np(lse.reshape(G)[heads]), rl)
    rel = eo / max(float(np.abs(ro).max()), 1e-30)
    say("  bitwise equal; vs oracle out %.2e (rel %.2e) lse %.2e" % (eo, rel, el))
    assert eo <= 2e-2 and rel <= 2e-2 and el <= 1e-2
    del x, res
    torch.cuda.empty_cache()
    # call 2, smaller, on the scratch the first call left behind: fp32, appending a token, gate on
    say("case noalloc call 2: B2 H3 n1000 d64 fp32, append, gate")
    _, res, _ = both(2, 3, 1000, 64, "f32", seed=61, append=True, gate=True)
    assert_equal(res)
    # and a third without the gate through the plain entry point
    say("case noalloc call 3: B1 H2 n70 d128 bf16")
    _, res, _ = both(1, 2, 70, 128, "bf16", seed=62, append=False, gate=False)
    assert_equal(res)
