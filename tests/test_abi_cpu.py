"""The C-ABI library without a GPU: it loads, exports what the header declares,
sizes workspaces, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import attention_fwd_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "path_attn.h")
BF, F32 = pa.PATH_DTYPE_BF16, pa.PATH_DTYPE_F32


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(path_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pa.lib()
    names = declared_functions()
    assert {"path_attn_fwd", "path_decode_step", "path_attn_fwd_workspace_size", "path_decode_workspace_size",
            "path_status_string", "path_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def declared_params(name):
    """Parameter names of a function declared in the header, in order."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b%s\s*\(([^)]*)\)\s*;" % name, src)
    assert m, name
    return [re.findall(r"(\w+)\s*$", p.strip())[0] for p in m.group(1).split(",")]


def test_entry_points_keep_their_parameter_lists():
    """The two calls of the problem statement keep the frozen parameter lists;
    options come through the _ex variants, which only add parameters."""
    assert declared_params("path_attn_fwd") == [
        "q", "k", "v", "w", "beta", "logf", "out", "lse", "B", "H", "L", "d", "dtype", "scale", "workspace",
        "workspace_bytes", "stream"]
    plain = ["kcache", "vcache", "n", "ncap", "q", "w", "beta", "k_new", "v_new", "out", "lse", "B", "H", "d",
             "dtype", "scale", "workspace", "workspace_bytes", "stream"]
    assert declared_params("path_decode_step") == plain
    assert declared_params("path_decode_step_ex") == plain[:7] + ["logf", "fcache"] + plain[7:]
    assert declared_params("path_attn_fwd_ex") == declared_params("path_attn_fwd")[:-1] + ["flags", "stream"]


def test_version_and_status_strings():
    lib = pa.lib()
    assert lib.path_abi_version() == 1
    for s in range(5):
        assert lib.path_status_string(s) and lib.path_status_string(s) != b"unknown status"
    assert lib.path_status_string(99) == b"unknown status"


def test_workspace_sizes():
    lib = pa.lib()
    assert lib.path_attn_fwd_workspace_size(1, 1, 64, 64, BF) > 0
    assert lib.path_attn_fwd_workspace_size(0, 1, 64, 64, BF) == 0
    assert lib.path_attn_fwd_workspace_size(1, 1, 0, 64, BF) == 0
    assert lib.path_attn_fwd_workspace_size(1, 1, 64, 96, BF) == 0    # unsupported head size
    assert lib.path_attn_fwd_workspace_size(1, 1, 64, 128, BF) > lib.path_attn_fwd_workspace_size(1, 1, 64, 64, BF)
    assert lib.path_attn_fwd_workspace_size(1, 1, 64, 64, 7) == 0     # bad dtype
    a = lib.path_attn_fwd_workspace_size(2, 3, 65, 64, BF)
    b = lib.path_attn_fwd_workspace_size(2, 3, 128, 64, BF)
    assert a == b  # both round up to two 64-token blocks
    assert lib.path_attn_fwd_workspace_size(2, 3, 128, 64, F32) > b
    assert lib.path_decode_workspace_size(16, 32, 32768, 64, BF) > 0
    assert lib.path_decode_workspace_size(16, 32, 0, 64, BF) == 0


# Fake device addresses: the library must reject these calls before any HIP call.
A = 1 << 20


def P(i):
    return ctypes.c_void_p(A * (i + 1))


def fwd_call(**over):
    args = dict(q=P(0), k=P(1), v=P(2), w=P(3), beta=P(4), logf=None, out=P(5), lse=None, B=1, H=1, L=64, d=64,
                dtype=BF, scale=0.0, ws=P(6), wsb=1 << 40, stream=None)
    args.update(over)
    return pa.lib().path_attn_fwd(args["q"], args["k"], args["v"], args["w"], args["beta"], args["logf"],
                                  args["out"], args["lse"], args["B"], args["H"], args["L"], args["d"],
                                  args["dtype"], args["scale"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), pa.PATH_EINVAL),
    (dict(out=None), pa.PATH_EINVAL),
    (dict(ws=None), pa.PATH_EINVAL),
    (dict(beta=None), pa.PATH_EINVAL),
    (dict(B=0), pa.PATH_EINVAL),
    (dict(H=-1), pa.PATH_EINVAL),
    (dict(L=0), pa.PATH_EINVAL),
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(d=32), pa.PATH_EUNSUPPORTED),
    (dict(d=0), pa.PATH_EINVAL),
    (dict(dtype=5), pa.PATH_EINVAL),
    (dict(wsb=16), pa.PATH_EINVAL),
    (dict(q=ctypes.c_void_p(A + 8)), pa.PATH_EINVAL),          # misaligned
    (dict(lse=ctypes.c_void_p(A * 9 + 2)), pa.PATH_EINVAL),    # misaligned fp32 array
    (dict(out=P(0)), pa.PATH_EINVAL),                          # out aliases q
    (dict(ws=P(2)), pa.PATH_EINVAL),                           # workspace overlaps v
    (dict(scale=float("nan")), pa.PATH_EINVAL),
])
def test_fwd_rejects_bad_arguments(over, status):
    assert fwd_call(**over) == status


def dec_call(ex=True, **over):
    args = dict(kc=P(0), vc=ctypes.c_void_p(A * 40), n=100, ncap=100, q=P(80), w=P(81), beta=P(82), lf=None, fc=None,
                kn=None, vn=None,
                out=P(83), lse=None, B=1, H=1, d=64, dtype=BF, scale=0.0, ws=P(84), wsb=1 << 30, stream=None)
    args.update(over)
    a = args
    rest = (a["kn"], a["vn"], a["out"], a["lse"], a["B"], a["H"], a["d"], a["dtype"], a["scale"], a["ws"], a["wsb"],
            a["stream"])
    if ex:
        return pa.lib().path_decode_step_ex(a["kc"], a["vc"], a["n"], a["ncap"], a["q"], a["w"], a["beta"], a["lf"],
                                            a["fc"], *rest)
    assert a["lf"] is None and a["fc"] is None
    return pa.lib().path_decode_step(a["kc"], a["vc"], a["n"], a["ncap"], a["q"], a["w"], a["beta"], *rest)


@pytest.mark.parametrize("over,status", [
    (dict(n=101), pa.PATH_EINVAL),                             # n > ncap
    (dict(n=-1), pa.PATH_EINVAL),
    (dict(n=0), pa.PATH_EINVAL),                               # nothing to attend to
    (dict(kn=P(90)), pa.PATH_EINVAL),                          # k_new without v_new
    (dict(kn=P(90), vn=P(91)), pa.PATH_EINVAL),                # no room for the new row
    (dict(kc=None), pa.PATH_EINVAL),
    (dict(d=32), pa.PATH_EUNSUPPORTED),
    (dict(d=256), pa.PATH_EUNSUPPORTED),
    (dict(wsb=8), pa.PATH_EINVAL),
    (dict(q=ctypes.c_void_p(A * 81 + 4)), pa.PATH_EINVAL),
    (dict(vc=P(0)), pa.PATH_EINVAL),                           # caches alias
    (dict(out=P(0)), pa.PATH_EINVAL),                          # out inside the key cache
    (dict(dtype=3), pa.PATH_EINVAL),
    (dict(lf=P(86)), pa.PATH_EINVAL),                          # gate without its cache
    (dict(lf=P(86), fc=P(0)), pa.PATH_EINVAL),                 # gate cache over the key cache
    (dict(lf=P(86), fc=ctypes.c_void_p(A * 87 + 2)), pa.PATH_EINVAL),  # misaligned gate cache
])
def test_decode_rejects_bad_arguments(over, status):
    assert dec_call(**over) == status
    if "lf" not in over and "fc" not in over:
        assert dec_call(ex=False, **over) == status  # the plain entry point validates the same way


def dec_fused_call(**over):
    args = dict(kc=P(0), vc=P(40), n=100, ncap=101, q=P(80), wraw=P(81), cw=P(82), zb=P(83), clip=0.0, st=P(84),
                lf=None, fc=None, kn=None, vn=None, out=P(85), lse=None, B=1, H=1, d=64, dtype=BF, scale=0.0,
                ws=P(86), wsb=1 << 30, stream=None)
    args.update(over)
    a = args
    return pa.lib().path_decode_step_fused(a["kc"], a["vc"], a["n"], a["ncap"], a["q"], a["wraw"], a["cw"], a["zb"],
                                           a["clip"], a["st"], a["lf"], a["fc"], a["kn"], a["vn"], a["out"], a["lse"],
                                           a["B"], a["H"], a["d"], a["dtype"], a["scale"], a["ws"], a["wsb"],
                                           a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(clip=-0.5), pa.PATH_EINVAL),
    (dict(clip=float("inf")), pa.PATH_EINVAL),
    (dict(clip=float("nan")), pa.PATH_EINVAL),
    (dict(st=None), pa.PATH_EINVAL),
    (dict(wraw=None), pa.PATH_EINVAL),
    (dict(cw=None), pa.PATH_EINVAL),
    (dict(zb=None), pa.PATH_EINVAL),
    (dict(ws=None), pa.PATH_EINVAL),
    (dict(n=102), pa.PATH_EINVAL),                             # n > ncap
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(wsb=64), pa.PATH_EINVAL),                            # workspace below the fused size
    (dict(st=P(0)), pa.PATH_EINVAL),                           # state inside the key cache
    (dict(st=P(81)), pa.PATH_EINVAL),                          # state over the raw row
    (dict(st=P(86)), pa.PATH_EINVAL),                          # state inside the workspace
    (dict(wraw=P(85)), pa.PATH_EINVAL),                        # raw row is the output
    (dict(zb=P(0)), pa.PATH_EINVAL),                           # zbeta inside the key cache
    (dict(cw=P(86)), pa.PATH_EINVAL),                          # taps inside the workspace
    (dict(wraw=ctypes.c_void_p(A * 81 + 8)), pa.PATH_EINVAL),  # misaligned raw row
    (dict(st=ctypes.c_void_p(A * 84 + 8)), pa.PATH_EINVAL),    # misaligned state
    (dict(lf=P(87)), pa.PATH_EINVAL),                          # gate without its cache
])
def test_decode_fused_rejects_bad_arguments(over, status):
    assert dec_fused_call(**over) == status


def test_decode_fused_workspace_size():
    plain = pa.decode_workspace_size(2, 3, 100, 64, pa.torch.bfloat16)
    fused = pa.decode_fused_workspace_size(2, 3, 100, 64, pa.torch.bfloat16)
    assert fused >= plain + 2 * 3 * 64 * 2 + 2 * 3 * 4  # room for the step's w and beta
    assert pa.decode_fused_workspace_size(2, 3, 100, 96, pa.torch.bfloat16) == 0


def noalloc_call(**over):
    G = 1 << 40  # fake device addresses far apart, so large sizes do not overlap
    args = dict(kc=ctypes.c_void_p(G), vc=ctypes.c_void_p(2 * G), n=100, ncap=100, q=ctypes.c_void_p(3 * G),
                w=ctypes.c_void_p(4 * G), beta=ctypes.c_void_p(5 * G), lf=None, fc=None, kn=None, vn=None,
                out=ctypes.c_void_p(6 * G), lse=None, B=1, H=1, d=64, dtype=BF, scale=0.0, stream=None)
    args.update(over)
    a = args
    return pa.lib().path_decode_step_noalloc(a["kc"], a["vc"], a["n"], a["ncap"], a["q"], a["w"], a["beta"], a["lf"],
                                             a["fc"], a["kn"], a["vn"], a["out"], a["lse"], a["B"], a["H"], a["d"],
                                             a["dtype"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(n=101), pa.PATH_EINVAL),                             # n > ncap
    (dict(n=0), pa.PATH_EINVAL),                               # nothing to attend to
    (dict(kc=None), pa.PATH_EINVAL),
    (dict(out=None), pa.PATH_EINVAL),
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(vc=ctypes.c_void_p(1 << 40)), pa.PATH_EINVAL),       # caches alias
    (dict(lf=ctypes.c_void_p(7 << 40)), pa.PATH_EINVAL),       # gate without its cache
    (dict(B=1000, H=100, d=128), pa.PATH_ESCRATCH),            # 100 000 heads: partials beyond the scratch
    (dict(B=1280, H=100, d=64), pa.PATH_ESCRATCH),             # 128 000 heads at d = 64
])
def test_decode_noalloc_rejects_before_launch(over, status):
    """The no-allocation decode entry validates like path_decode_step_ex, and a problem whose split
    partials exceed its fixed scratch is refused with PATH_ESCRATCH before any device call."""
    assert noalloc_call(**over) == status


def test_decode_noalloc_scratch_size():
    lib = pa.lib()
    cap = lib.path_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    # the decode workload (B16 H32, 32768 rows, d 64) and the largest head counts named in the header fit
    assert lib.path_decode_workspace_size(16, 32, 32768, 64, BF) <= cap
    assert lib.path_decode_workspace_size(1, 127100, 32768, 64, BF) <= cap
    assert lib.path_decode_workspace_size(1, 127101, 32768, 64, BF) > cap
    assert lib.path_decode_workspace_size(1, 64527, 32768, 128, BF) <= cap
    assert lib.path_decode_workspace_size(1, 64528, 32768, 128, BF) > cap


def cache_call(**over):
    # the workspace sits above every other buffer, so the baseline call has no overlap
    args = dict(ws=ctypes.c_void_p(A * 1024), wsb=1 << 40, v=ctypes.c_void_p(A * 64), kc=ctypes.c_void_p(A * 128),
                vc=ctypes.c_void_p(A * 192), lf=None, fc=None,
                ncap=256, B=1, H=1, L=200, d=64, dtype=BF, stream=None)
    args.update(over)
    return pa.lib().path_decode_cache_from_fwd(args["ws"], args["wsb"], args["v"], args["lf"], args["kc"], args["vc"],
                                               args["fc"], args["ncap"], args["B"], args["H"], args["L"], args["d"],
                                               args["dtype"], args["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(ws=None), pa.PATH_EINVAL),
    (dict(v=None), pa.PATH_EINVAL),
    (dict(kc=None), pa.PATH_EINVAL),
    (dict(ncap=199), pa.PATH_EINVAL),                          # cache shorter than the prefix
    (dict(L=0), pa.PATH_EINVAL),
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(dtype=4), pa.PATH_EINVAL),
    (dict(wsb=1024), pa.PATH_EINVAL),                          # workspace smaller than the forward's
    (dict(v=ctypes.c_void_p(A * 64 + 8)), pa.PATH_EINVAL),     # misaligned
    (dict(vc=ctypes.c_void_p(A * 128)), pa.PATH_EINVAL),       # caches alias
    (dict(kc=ctypes.c_void_p(A * 1024 + 4096)), pa.PATH_EINVAL),  # key cache inside the used workspace
    (dict(vc=ctypes.c_void_p(A * 64)), pa.PATH_EINVAL),        # value cache over the values
    (dict(lf=ctypes.c_void_p(A * 256)), pa.PATH_EINVAL),       # gate without its cache
    (dict(lf=ctypes.c_void_p(A * 256), fc=ctypes.c_void_p(A * 128)), pa.PATH_EINVAL),  # gate cache over keys
])
def test_cache_from_fwd_rejects_bad_arguments(over, status):
    assert cache_call(**over) == status


def fused_call(**over):
    args = dict(q=P(0), k=P(1), v=P(2), wraw=P(3), cw=P(7), zb=P(4), clip=1.98, logf=None, out=P(5), lse=None, B=1,
                H=1, L=64, d=64, dtype=BF, scale=0.0, ws=P(6), wsb=1 << 40, stream=None)
    args.update(over)
    a = args
    return pa.lib().path_attn_fwd_fused(a["q"], a["k"], a["v"], a["wraw"], a["cw"], a["zb"], a["clip"], a["logf"],
                                        a["out"], a["lse"], a["B"], a["H"], a["L"], a["d"], a["dtype"], a["scale"],
                                        a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(cw=None), pa.PATH_EINVAL),                           # no convolution weights
    (dict(cw=ctypes.c_void_p(A * 8 + 4)), pa.PATH_EINVAL),     # misaligned weights
    (dict(zb=None), pa.PATH_EINVAL),                           # no pre-sigmoid values
    (dict(wraw=None), pa.PATH_EINVAL),                         # no pre-convolution rows
    (dict(clip=-1.0), pa.PATH_EINVAL),                         # negative cap
    (dict(clip=float("nan")), pa.PATH_EINVAL),                 # non-finite cap
    (dict(clip=float("inf")), pa.PATH_EINVAL),
    (dict(cw=P(5)), pa.PATH_EINVAL),                           # weights overlap out
    (dict(cw=P(6)), pa.PATH_EINVAL),                           # weights inside the workspace
    (dict(out=P(3)), pa.PATH_EINVAL),                          # out aliases wraw
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(wsb=16), pa.PATH_EINVAL),                            # workspace too small
])
def test_fwd_fused_rejects_bad_arguments(over, status):
    assert fused_call(**over) == status


def test_fwd_ex_rejects_unknown_flags():
    lib = pa.lib()
    args = [P(0), P(1), P(2), P(3), P(4), None, P(5), None, 1, 1, 64, 64, BF, 0.0, P(6), 1 << 40]
    assert lib.path_attn_fwd_ex(*args, 2, None) == pa.PATH_EINVAL
    assert lib.path_attn_fwd_ex(*args[:1], None, *args[2:], 1, None) == pa.PATH_EINVAL  # k NULL, valid flag


def test_bwd_workspace_sizes():
    lib = pa.lib()
    one = lib.path_attn_bwd_workspace_size(1, 1, 200, 64, BF)
    assert one > 0
    assert lib.path_attn_bwd_workspace_size(2, 3, 200, 64, BF) == 6 * one   # all heads at once
    assert lib.path_attn_bwd_workspace_size(1, 1, 200, 128, BF) > one      # head dimension 128
    assert lib.path_attn_bwd_workspace_size(1, 1, 200, 96, BF) == 0
    assert lib.path_attn_bwd_workspace_size(1, 1, 0, 64, BF) == 0
    assert lib.path_attn_bwd_workspace_size(1, 1, 64, 64, 9) == 0
    share = lib.path_attn_bwd_workspace_size(1, 1, 4096, 64, BF)
    big = lib.path_attn_bwd_workspace_size(32, 32, 4096, 64, BF)
    assert big % share == 0 and share <= big <= 32 << 30                    # capped at whole heads in 32 GiB
    assert lib.path_attn_bwd_workspace_size(1, 1, 65, 64, F32) > lib.path_attn_bwd_workspace_size(1, 1, 64, 64, F32)


def bwd_call(**over):
    share = pa.lib().path_attn_bwd_workspace_size(1, 1, 64, 64, BF)
    args = dict(q=P(0), k=P(1), v=P(2), w=P(3), beta=P(4), logf=None, out=P(5), lse=P(6), dout=P(7), dlse=None,
                dq=P(8), dk=P(9), dv=P(10), dw=P(11), dbeta=P(12), dlogf=None, B=1, H=1, L=64, d=64, dtype=BF,
                scale=0.0, ws=ctypes.c_void_p(A * 64), wsb=share, stream=None)
    args.update(over)
    a = args
    return pa.lib().path_attn_bwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"], a["out"], a["lse"], a["dout"],
                                  a["dlse"], a["dq"], a["dk"], a["dv"], a["dw"], a["dbeta"], a["dlogf"], a["B"],
                                  a["H"], a["L"], a["d"], a["dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(lse=None), pa.PATH_EINVAL),                          # the forward's lse is required
    (dict(out=None), pa.PATH_EINVAL),
    (dict(dout=None), pa.PATH_EINVAL),
    (dict(dbeta=None), pa.PATH_EINVAL),
    (dict(logf=P(13)), pa.PATH_EINVAL),                        # gate without its gradient
    (dict(dlogf=P(13)), pa.PATH_EINVAL),                       # gradient without the gate
    (dict(d=96), pa.PATH_EUNSUPPORTED),
    (dict(L=0), pa.PATH_EINVAL),
    (dict(dtype=7), pa.PATH_EINVAL),
    (dict(wsb=1024), pa.PATH_EINVAL),                          # below one head's share
    (dict(dq=ctypes.c_void_p(A * 9 + 8)), pa.PATH_EINVAL),     # misaligned
    (dict(dk=P(8)), pa.PATH_EINVAL),                           # two outputs alias
    (dict(dq=P(0)), pa.PATH_EINVAL),                           # output over an input
    (dict(dbeta=P(4)), pa.PATH_EINVAL),                        # dbeta over beta
    (dict(dv=ctypes.c_void_p(A * 64)), pa.PATH_EINVAL),        # output inside the workspace
    (dict(ws=P(1)), pa.PATH_EINVAL),                           # workspace over an input
    (dict(scale=float("inf")), pa.PATH_EINVAL),
])
def test_bwd_rejects_bad_arguments(over, status):
    assert bwd_call(**over) == status
