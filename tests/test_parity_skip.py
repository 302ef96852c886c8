"""GPU parity of the forward with PATH_FWD_SKIP_NEGLIGIBLE (forget gate): the walk
over key blocks stops once the remaining blocks provably add less than 2^-64 of
the running maximum per key.

Checks: against the fp64 oracle with the usual bars (1e-4 fp32, 2e-2 bf16), and
against the full walk of the same kernel (fp32: 1e-6; bf16: one bf16 ulp of the
largest output), with the workload's forget gate (log f = logsigmoid(3 + N(0,1)))
and a strong one (logsigmoid(N(0,1)), where only a few blocks matter); a head with
a non-contracting transition (beta ||w||^2 > 2) must not skip at all.
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


def run(x, skip):
    out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], return_lse=True, skip_negligible=skip)
    torch.cuda.synchronize()
    return out, lse


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [200, 1000, 3000])
@pytest.mark.parametrize("fox_mean", [3.0, 0.0], ids=["workload_gate", "strong_gate"])
def test_skip_matches_oracle_and_full_walk(L, dtype, fox_mean):
    say("case skip L%d %s fox_mean %g" % (L, dtype, fox_mean))
    x = pathgen.fwd_inputs(1, 2, L, 64, dtype, seed=300 + L, fox=True, clip=1.98 if dtype == "bf16" else None,
                           device="cuda", fox_mean=fox_mean)
    o_s, l_s = run(x, True)
    o_f, l_f = run(x, False)
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu(), x["logf"].cpu())
    eo, el = max_abs(to_np(o_s), ro), max_abs(to_np(l_s), rl)
    do, dl = max_abs(to_np(o_s), to_np(o_f)), max_abs(to_np(l_s), to_np(l_f))
    say("  vs oracle out %.2e lse %.2e; vs full walk out %.2e lse %.2e" % (eo, el, do, dl))
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    if dtype == "f32":
        assert do <= 1e-6 and dl <= 1e-6
    else:
        assert do <= 2.0 ** -8 * float(np.abs(ro).max()) and dl <= 1e-5


@gpu
def test_skip_disabled_by_non_contracting_transition():
    """beta ||w||^2 > 2 in one block: the bound does not hold, nothing may be skipped."""
    x = pathgen.fwd_inputs(1, 1, 1000, 64, "f32", seed=9, fox=True, device="cuda", fox_mean=0.0)
    x["beta"][0, 0, 500] = 2.5
    o_s, l_s = run(x, True)
    o_f, l_f = run(x, False)
    assert torch.equal(o_s, o_f) and torch.equal(l_s, l_f)
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu(), x["logf"].cpu())
    assert max_abs(to_np(o_s), ro) <= 1e-4


@gpu
def test_skip_without_gate_is_the_plain_forward():
    x = pathgen.fwd_inputs(1, 2, 500, 64, "bf16", seed=10, clip=1.98, device="cuda")
    o_s, l_s = run(x, True)
    o_f, l_f = run(x, False)
    assert torch.equal(o_s, o_f) and torch.equal(l_s, l_f)


@gpu
def test_skip_fox_workload_sampled_rows():
    """B4 H16 L16384 bf16 with the workload's forget gate: 256 random rows of two heads plus their last 64 rows."""
    c = pathgen.WORKLOADS["fox_L16384_bf16"]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    say("case skip fox workload")
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=0, fox=True, clip=1.98, device="cuda")
    o_s, l_s = run(x, True)
    G = B * H
    rng = np.random.default_rng(6)
    heads = [int(rng.integers(G)), G - 1]
    rows = np.array([(int(rng.integers(2)), int(rng.integers(L))) for _ in range(256)] +
                    [(g, L - 1 - t) for g in (0, 1) for t in range(64)], dtype=np.int64)
    sel = {k: v.reshape(G, L, -1)[heads].cpu() if v.dim() == 4 else v.reshape(G, L)[heads].cpu() for k, v in x.items()}
    ro, rl = oracle.fwd(sel["q"], sel["k"], sel["v"], sel["w"], sel["beta"], sel["logf"], rows=rows)
    og, lg = to_np(o_s.reshape(G, L, d)[heads]), to_np(l_s.reshape(G, L)[heads])
    eo, el = max_abs(og[rows[:, 0], rows[:, 1]], ro), max_abs(lg[rows[:, 0], rows[:, 1]], rl)
    say("  max-abs out %.2e lse %.2e" % (eo, el))
    assert eo <= 2e-2 and el <= 2e-2
