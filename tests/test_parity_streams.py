"""Calls on a caller-given side stream (through the C ABI).

The binding allocates the workspace (and any output the caller does not pass)
on the current stream but the kernels run on the given stream.  While that
stream is still busy, the caching allocator must not hand the freed workspace
to a new allocation on the current stream; the results must match the oracle.
"""
import numpy as np
import pytest
import torch

import attention_fwd_amd as pa
import oracle
import pathgen
from parity_util import max_abs, say, to_np

gpu = pytest.mark.gpu


class Spy:
    """Wraps one C entry point of the loaded library and records the workspace pointer it received."""

    def __init__(self, name, ws_index):
        self.lib, self.name, self.ws_index, self.ws = pa.lib(), name, ws_index, None

    def __enter__(self):
        self.real = getattr(self.lib, self.name)

        def call(*args):
            self.ws = args[self.ws_index].value
            return self.real(*args)

        setattr(self.lib, self.name, call)
        return self

    def __exit__(self, *exc):
        setattr(self.lib, self.name, self.real)


def busy(stream, cycles=200_000_000):
    with torch.cuda.stream(stream):
        torch.cuda._sleep(cycles)  # keeps the side stream busy (~0.1 s) so its kernels queue behind this


@gpu
def test_fwd_on_side_stream():
    B, H, L, d = 1, 2, 700, 64
    say("case fwd on a side stream")
    x = pathgen.fwd_inputs(B, H, L, d, "bf16", seed=31, fox=True, clip=1.98, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    busy(s)
    with Spy("path_attn_fwd_ex", 14) as spy:
        out, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], return_lse=True, stream=s)
    nbytes = pa.fwd_workspace_size(B, H, L, d, torch.bfloat16)
    junk = torch.full((nbytes,), 0xFF, device="cuda", dtype=torch.uint8)  # current stream, runs at once
    assert junk.data_ptr() != spy.ws, "workspace handed out again while the side stream still uses it"
    s.synchronize()
    ro, rl = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["w"].cpu(), x["beta"].cpu(), x["logf"].cpu())
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  out %.2e lse %.2e" % (eo, el))
    assert eo <= 2e-2 and el <= 2e-2


@gpu
def test_decode_on_side_stream():
    B, H, n, d = 2, 2, 3000, 64
    say("case decode on a side stream")
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="bf16", seed=32, clip=1.98, device="cuda")
    kc0, vc0 = x["kcache"].cpu(), x["vcache"].cpu()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    busy(s)
    with Spy("path_decode_step", 16) as spy:
        out, lse = pa.decode_step(x["kcache"], x["vcache"], n, x["q"][0], x["w"][0], x["beta"][0], return_lse=True,
                                  stream=s)
    nbytes = max(pa.decode_workspace_size(B, H, n, d, torch.bfloat16), 16)
    junk = torch.full((nbytes,), 0xFF, device="cuda", dtype=torch.uint8)
    assert junk.data_ptr() != spy.ws, "workspace handed out again while the side stream still uses it"
    s.synchronize()
    _, _, ro, rl = oracle.decode(kc0, vc0, n, x["q"][0].cpu(), x["w"][0].cpu(), x["beta"][0].cpu())
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    rel = eo / float(np.abs(ro).max())
    say("  out %.2e (rel %.2e) lse %.2e" % (eo, rel, el))
    assert eo <= 2e-2 and rel <= 2e-2 and el <= 1e-2


@gpu
def test_decode_fused_on_side_stream():
    B, H, n, d = 2, 2, 3000, 64
    say("case fused decode on a side stream")
    x = pathgen.decode_inputs(B, H, n, d, steps=1, dtype="bf16", seed=33, clip=1.98, device="cuda")
    kc0, vc0 = x["kcache"].cpu(), x["vcache"].cpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(34)
    raw = torch.randn((B, H, 3, d), generator=g, device="cuda").to(torch.bfloat16)
    conv_w = (torch.randn((H, d, 3), generator=g, device="cuda") / 3.0 ** 0.5).contiguous()
    zb = torch.randn((B, H, 3), generator=g, device="cuda")
    state = raw[:, :, :2].clone()  # a copy: the step moves it on in place
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    busy(s)
    with Spy("path_decode_step_fused", 21) as spy:
        out, lse = pa.decode_step_fused(x["kcache"], x["vcache"], n, x["q"][0], raw[:, :, 2].contiguous(), conv_w,
                                        zb[:, :, 2].contiguous(), state, beta_clip=1.98, return_lse=True, stream=s)
    nbytes = max(pa.decode_fused_workspace_size(B, H, n, d, torch.bfloat16), 16)
    junk = torch.full((nbytes,), 0xFF, device="cuda", dtype=torch.uint8)
    assert junk.data_ptr() != spy.ws, "workspace handed out again while the side stream still uses it"
    s.synchronize()
    w_ref, b_ref = oracle.produce(raw.cpu(), conv_w.cpu(), zb.cpu(), 1.98)
    _, _, ro, rl = oracle.decode(kc0, vc0, n, x["q"][0].cpu(), w_ref[:, :, 2], b_ref[:, :, 2])
    eo, el = max_abs(to_np(out), ro), max_abs(to_np(lse), rl)
    say("  out %.2e lse %.2e" % (eo, el))
    assert eo <= 2e-2 and el <= 1e-2
    assert torch.equal(state, raw[:, :, 1:3])
