"""fp64 CPU oracle for PaTH attention (forward, PaTH-FoX bias, decode step, backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library never loads it, and it shares no code with the HIP path.

The arithmetic lives in ``path_oracle.c`` (plain C, fp64, pthreads over
rows); this module only marshals numpy arrays into it.  The definition it
follows is the attention logit of the Japanese technical summary
"技術要約: PaTH Attention" (gist.science), section 2: s_ij = k_j^T (H_{j+1} ...
H_i) q_i with H_s = I - beta_s w_s w_s^T, followed by the causal softmax and
the weighted sum of values described in section 3-4 of the iplexlaw blog
"거리에서 경로로, PaTH Attention".  Decode follows section 3 of the same
summary: the newest H_t is applied in place to every cached key; the decode
cache after a prefix is what those in-place updates would have produced.
The backward is the chain rule applied to the same definition (the pages
give the blockwise algorithm as what makes training possible but print no
gradient formulas).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "path_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs = {}


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library (gcc -O2, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
         "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile path_oracle.c into liboracle.so next to it (when stale or forced)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _load(path=None):
    path = path or build()
    if path not in _libs:
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, i64p, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int64, dp, dp, dp, dp, dp, dp,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, ctypes.c_int]
        lib.oracle_scores_head.restype = None
        lib.oracle_scores_head.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, dp]
        lib.oracle_decode_cache.restype = ctypes.c_int
        lib.oracle_decode_cache.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp]
        lib.oracle_produce.restype = ctypes.c_int
        lib.oracle_produce.argtypes = [dp, dp, dp, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, dp, dp]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_transport.restype = None
        lib.oracle_transport.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp]
        _libs[path] = lib
    return _libs[path]


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen exactly (bf16 -> fp32 -> fp64 is exact)
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def fwd(q, k, v, w, beta, logf=None, scale=None, rows=None, nthreads=None, lib=None):
    """PaTH forward in fp64.

    q, k, v, w: [..., L, d] (leading dims are flattened into G heads);
    beta, logf: [..., L].  scale defaults to 1/sqrt(d).
    rows: optional int array [R, 2] of (flat head g, row i); then the result is
    (out [R, d], lse [R]); otherwise (out [..., L, d], lse [..., L]).
    """
    q, k, v, w, beta, logf = (_f64(x) for x in (q, k, v, w, beta, logf))
    lead = q.shape[:-2]
    L, d = q.shape[-2], q.shape[-1]
    G = int(np.prod(lead)) if lead else 1
    for t in (k, v, w):
        assert t.shape == q.shape, (t.shape, q.shape)
    assert beta.shape == q.shape[:-1]
    if logf is not None:
        assert logf.shape == q.shape[:-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nthreads = nthreads or default_threads()
    lib = _load(lib)
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
        out = np.zeros((r.shape[0], d))
        lse = np.zeros((r.shape[0],))
        rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        nr = r.shape[0]
    else:
        out = np.zeros((G, L, d))
        lse = np.zeros((G, L))
        rp, nr = None, 0
    rc = lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), G, L, d, float(scale),
                        rp, nr, _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_fwd: bad arguments")
    if rows is None:
        out = out.reshape(lead + (L, d))
        lse = lse.reshape(lead + (L,))
    return out, lse


def scores(q, k, w, beta, logf=None, scale=None, lib=None):
    """All logits of one head: [L, L], -inf above the diagonal."""
    q, k, w, beta, logf = (_f64(x) for x in (q, k, w, beta, logf))
    L, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    S = np.zeros((L, L))
    _load(lib).oracle_scores_head(_ptr(q), _ptr(k), _ptr(w), _ptr(beta), _ptr(logf), L, d, float(scale), _ptr(S))
    return S


def transport(x, w, beta, lo, hi, lib=None):
    """H_lo H_{lo+1} ... H_hi x for one vector x [d] (w: [n, d], beta: [n])."""
    x, w, beta = _f64(x), _f64(w), _f64(beta)
    out = np.zeros_like(x)
    _load(lib).oracle_transport(_ptr(x), _ptr(w), _ptr(beta), x.shape[0], int(lo), int(hi), _ptr(out))
    return out


def decode(kc, vc, n, q, w, beta, k_new=None, v_new=None, scale=None, nthreads=None, lib=None, logf=None,
           fcache=None):
    """One decode step in fp64.

    kc, vc: [..., rowcap, d] cache (copied; the updated copy is returned).
    q, w: [..., d]; beta: [...].  Rows [0, n) get k <- H_t k; with k_new/v_new
    ([..., d]) the pair is written at row n afterwards and n+1 rows attend.
    Forget gate: logf [...] = log f_t and fcache [..., rowcap] = c_j (cumulative
    log f up to row j); row j's logit gets c_t - c_j with c_t = c_{n-1} + log f_t.
    Returns (kc_new, vc_new, out [..., d], lse [...]), plus the updated fcache
    when logf is given.
    """
    kc = _f64(kc).copy()
    vc = _f64(vc).copy()
    q, w, beta, k_new, v_new, logf = (_f64(x) for x in (q, w, beta, k_new, v_new, logf))
    fc = _f64(fcache).copy() if fcache is not None else None
    lead = q.shape[:-1]
    d = q.shape[-1]
    G = int(np.prod(lead)) if lead else 1
    rowcap = kc.shape[-2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((G, d))
    lse = np.zeros((G,))
    rc = _load(lib).oracle_decode(_ptr(kc), _ptr(vc), _ptr(fc), int(n), int(rowcap), _ptr(q), _ptr(w), _ptr(beta),
                               _ptr(logf), _ptr(k_new), _ptr(v_new), G, d, float(scale), _ptr(out), _ptr(lse),
                               int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_decode: bad arguments")
    res = (kc, vc, out.reshape(lead + (d,)), lse.reshape(lead))
    return res + (fc,) if logf is not None else res


def decode_cache(k, w, beta, lib=None, logf=None):
    """Decode cache after a prefix of L tokens, fp64: row j = H_{L-1} ... H_{j+1} k_j.

    k, w: [..., L, d]; beta: [..., L].  Returns [..., L, d]; with logf
    ([..., L]) also the gate cache [..., L] of inclusive prefix sums of log f.
    """
    k, w, beta, logf = _f64(k), _f64(w), _f64(beta), _f64(logf)
    lead = k.shape[:-2]
    L, d = k.shape[-2], k.shape[-1]
    G = int(np.prod(lead)) if lead else 1
    assert w.shape == k.shape and beta.shape == k.shape[:-1]
    out = np.zeros((G, L, d))
    fc = np.zeros((G, L)) if logf is not None else None
    rc = _load(lib).oracle_decode_cache(_ptr(k), _ptr(w), _ptr(beta), _ptr(logf), G, L, d, _ptr(out), _ptr(fc))
    if rc != 0:
        raise ValueError("oracle_decode_cache: bad arguments")
    out = out.reshape(lead + (L, d))
    return (out, fc.reshape(lead + (L,))) if logf is not None else out


def produce(wraw, conv_w, zbeta, beta_clip=0.0, lib=None):
    """Producer of w and beta in fp64 (short causal convolution of width 3,
    L2 normalisation, beta = 2 sigmoid(z), capped at beta_clip when > 0).

    wraw: [B, H, L, d]; conv_w: [H, d, 3]; zbeta: [B, H, L].
    Returns (w [B, H, L, d], beta [B, H, L]).
    """
    wraw, conv_w, zbeta = _f64(wraw), _f64(conv_w), _f64(zbeta)
    B, H, L, d = wraw.shape
    assert conv_w.shape == (H, d, 3) and zbeta.shape == (B, H, L)
    G = B * H
    w = np.zeros((G, L, d))
    beta = np.zeros((G, L))
    rc = _load(lib).oracle_produce(_ptr(wraw), _ptr(conv_w), _ptr(zbeta), float(beta_clip), G, H, L, d, _ptr(w),
                                   _ptr(beta))
    if rc != 0:
        raise ValueError("oracle_produce: bad arguments")
    return w.reshape(B, H, L, d), beta.reshape(B, H, L)


def fwd_fused(q, k, v, wraw, conv_w, zbeta, beta_clip=0.0, logf=None, scale=None, rows=None, nthreads=None,
              lib=None):
    """PaTH forward with w and beta made by the producer (see produce), fp64."""
    w, beta = produce(wraw, conv_w, zbeta, beta_clip, lib=lib)
    return fwd(q, k, v, w, beta, logf, scale=scale, rows=rows, nthreads=nthreads, lib=lib)


def bwd(q, k, v, w, beta, logf, dout, dlse=None, scale=None, nthreads=None, lib=None):
    """Gradient of sum(dout * o) + sum(dlse * lse) for the forward above, fp64.

    q, k, v, w, dout: [..., L, d]; beta, logf, dlse: [..., L] (logf, dlse may
    be None).  Returns a dict with dq, dk, dv, dw [..., L, d], dbeta [..., L],
    dlogf [..., L] (None without logf), and the forward's o and lse.
    """
    q, k, v, w, beta, logf, dout, dlse = (_f64(x) for x in (q, k, v, w, beta, logf, dout, dlse))
    lead = q.shape[:-2]
    L, d = q.shape[-2], q.shape[-1]
    G = int(np.prod(lead)) if lead else 1
    for t in (k, v, w, dout):
        assert t.shape == q.shape, (t.shape, q.shape)
    for t in (beta, logf, dlse):
        assert t is None or t.shape == q.shape[:-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    res = {n: np.zeros((G, L, d)) for n in ("dq", "dk", "dv", "dw", "o")}
    res["dbeta"] = np.zeros((G, L))
    res["lse"] = np.zeros((G, L))
    res["dlogf"] = np.zeros((G, L)) if logf is not None else None
    rc = _load(lib).oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(dout), _ptr(dlse),
                               G, L, d, float(scale), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]),
                               _ptr(res["dw"]), _ptr(res["dbeta"]), _ptr(res["dlogf"]), _ptr(res["o"]),
                               _ptr(res["lse"]), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_bwd: bad arguments")
    for n, a in list(res.items()):
        if a is not None:
            res[n] = a.reshape(lead + a.shape[1:])
    return res
