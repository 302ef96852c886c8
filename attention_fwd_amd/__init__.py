"""PaTH attention for AMD MI355X: a thin ctypes binding of libpath_attn.so.

Every step of the computation runs in the library's HIP kernels; this module
only marshals torch tensors (device memory) and the current HIP stream into
the C ABI declared in include/path_attn.h.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["fwd", "fwd_fused", "fwd_prep", "fwd_scan", "decode_step", "decode_cache_from_fwd", "fwd_workspace_size",
           "decode_workspace_size", "bwd", "bwd_workspace_size", "lib", "PathError", "PATH_OK", "PATH_EINVAL", "PATH_EUNSUPPORTED", "PATH_EHIP", "PATH_ESCRATCH", "decode_step_noalloc", "PATH_DTYPE_F32", "PATH_DTYPE_BF16",
           "PATH_FWD_SKIP_NEGLIGIBLE", "decode_step_fused", "decode_fused_workspace_size"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpath_attn.so")

PATH_OK, PATH_EINVAL, PATH_EUNSUPPORTED, PATH_EHIP, PATH_ESCRATCH = 0, 1, 2, 3, 4
PATH_DTYPE_F32, PATH_DTYPE_BF16 = 0, 1
_DTYPES = {torch.float32: PATH_DTYPE_F32, torch.bfloat16: PATH_DTYPE_BF16}

_lib = None


class PathError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = _lib.path_status_string(status).decode() if _lib is not None else str(status)
        super().__init__("%s: %s (status %d)" % (what, msg, status))


def lib():
    """The loaded C library (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpath_attn.so is not built (run __graft_entry__.build() or "
                               "python attention_fwd_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i, i64, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.path_abi_version.restype = ctypes.c_int
        L.path_abi_version.argtypes = []
        L.path_status_string.restype = ctypes.c_char_p
        L.path_status_string.argtypes = [ctypes.c_int]
        L.path_attn_fwd_workspace_size.restype = sz
        L.path_attn_fwd_workspace_size.argtypes = [i, i, i, i, ctypes.c_int]
        L.path_attn_fwd.restype = ctypes.c_int
        L.path_attn_fwd.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, ctypes.c_int, ctypes.c_float,
                                    vp, sz, vp]
        L.path_attn_fwd_ex.restype = ctypes.c_int
        L.path_attn_fwd_ex.argtypes = list(L.path_attn_fwd.argtypes[:-1]) + [ctypes.c_uint, vp]
        L.path_attn_fwd_fused.restype = ctypes.c_int
        L.path_attn_fwd_fused.argtypes = [vp, vp, vp, vp, fp, fp, ctypes.c_float, fp, vp, fp, i, i, i, i, ctypes.c_int,
                                          ctypes.c_float, vp, sz, vp]
        L.path_attn_fwd_prep.restype = ctypes.c_int
        L.path_attn_fwd_prep.argtypes = list(L.path_attn_fwd.argtypes)
        L.path_attn_fwd_scan.restype = ctypes.c_int
        L.path_attn_fwd_scan.argtypes = [vp, fp, i, i, i, i, i, ctypes.c_int, ctypes.c_float, vp, sz, vp]
        L.path_decode_workspace_size.restype = sz
        L.path_decode_workspace_size.argtypes = [i, i, i64, i, ctypes.c_int]
        L.path_decode_step.restype = ctypes.c_int
        L.path_decode_step.argtypes = [vp, vp, i64, i64, vp, vp, fp, vp, vp, vp, fp, i, i, i, ctypes.c_int,
                                       ctypes.c_float, vp, sz, vp]
        L.path_decode_step_ex.restype = ctypes.c_int
        L.path_decode_step_ex.argtypes = [vp, vp, i64, i64, vp, vp, fp, fp, fp, vp, vp, vp, fp, i, i, i,
                                          ctypes.c_int, ctypes.c_float, vp, sz, vp]
        L.path_decode_fused_workspace_size.restype = sz
        L.path_decode_fused_workspace_size.argtypes = [i, i, i64, i, ctypes.c_int]
        L.path_decode_step_fused.restype = ctypes.c_int
        L.path_decode_step_fused.argtypes = [vp, vp, i64, i64, vp, vp, fp, fp, ctypes.c_float, vp, fp, fp, vp, vp, vp,
                                             fp, i, i, i, ctypes.c_int, ctypes.c_float, vp, sz, vp]
        L.path_decode_noalloc_max_bytes.restype = sz
        L.path_decode_noalloc_max_bytes.argtypes = []
        L.path_decode_step_noalloc.restype = ctypes.c_int
        L.path_decode_step_noalloc.argtypes = [vp, vp, i64, i64, vp, vp, fp, fp, fp, vp, vp, vp, fp, i, i, i,
                                               ctypes.c_int, ctypes.c_float, vp]
        L.path_decode_cache_from_fwd.restype = ctypes.c_int
        L.path_decode_cache_from_fwd.argtypes = [vp, sz, vp, fp, vp, vp, fp, i64, i, i, i, i, ctypes.c_int, vp]
        L.path_attn_bwd_workspace_size.restype = sz
        L.path_attn_bwd_workspace_size.argtypes = [i, i, i, i, ctypes.c_int]
        L.path_attn_bwd.restype = ctypes.c_int
        L.path_attn_bwd.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, vp, vp, vp, fp, fp, i, i, i, i,
                                    ctypes.c_int, ctypes.c_float, vp, sz, vp]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda/hip) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _record(stream, *tensors):
    """Tensors this binding allocated (on the current stream) and a kernel on
    `stream` uses: tell the caching allocator, so their memory is not handed
    out again before that stream's work is done."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def fwd_workspace_size(B, H, L, d, dtype=torch.bfloat16):
    return int(lib().path_attn_fwd_workspace_size(B, H, L, d, _DTYPES[dtype]))


def decode_workspace_size(B, H, rows, d, dtype=torch.bfloat16):
    return int(lib().path_decode_workspace_size(B, H, rows, d, _DTYPES[dtype]))


def decode_fused_workspace_size(B, H, rows, d, dtype=torch.bfloat16):
    return int(lib().path_decode_fused_workspace_size(B, H, rows, d, _DTYPES[dtype]))


PATH_FWD_SKIP_NEGLIGIBLE = 1


def fwd(q, k, v, w, beta, logf=None, scale=None, out=None, lse=None, return_lse=False, workspace=None,
        stream=None, skip_negligible=False):
    """Causal PaTH attention forward (path_attn_fwd / path_attn_fwd_ex).

    q, k, v, w: [B, H, L, d] bf16 or fp32 device tensors; beta, logf: [B, H, L]
    fp32 (logf optional, enables the PaTH-FoX bias).  skip_negligible (with
    logf) stops the walk over key blocks once the rest provably contributes
    below 2^-64 of the running maximum per key.  Returns out (and lse when
    return_lse or an lse tensor is given).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (w, "w")):
        _check(t, n, dt, (B, H, L, d), dev)
    _check(beta, "beta", torch.float32, (B, H, L), dev)
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H, L), dev)
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    _check(out, "out", dt, (B, H, L, d), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, L), device=dev, dtype=torch.float32)
        mine.append(lse)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, L), dev)
    need = fwd_workspace_size(B, H, L, d, dt)
    if need == 0:
        raise PathError(PATH_EUNSUPPORTED if d not in (64, 128) else PATH_EINVAL, "path_attn_fwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
        mine.append(workspace)
    _check(workspace, "workspace", None, None, dev)
    with torch.cuda.device(dev):
        _record(stream, *mine)
        st = lib().path_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(out),
                                    _ptr(lse), B, H, L, d, _DTYPES[dt], float(scale or 0.0), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    PATH_FWD_SKIP_NEGLIGIBLE if skip_negligible else 0, _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_attn_fwd_ex")
    return (out, lse) if (return_lse or lse is not None) else out


def fwd_fused(q, k, v, wraw, conv_w, zbeta, beta_clip=0.0, logf=None, scale=None, out=None, lse=None,
              return_lse=False, workspace=None, stream=None):
    """PaTH forward with the producer of w and beta fused in (path_attn_fwd_fused).

    wraw: [B, H, L, d] (dtype of q) pre-convolution rows; conv_w: [H, d, 3] fp32
    causal width-3 depthwise weights; zbeta: [B, H, L] fp32 pre-sigmoid values;
    beta_clip: cap on beta = 2 sigmoid(z) (0: none).  Otherwise as fwd.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (wraw, "wraw")):
        _check(t, n, dt, (B, H, L, d), dev)
    _check(conv_w, "conv_w", torch.float32, (H, d, 3), dev)
    _check(zbeta, "zbeta", torch.float32, (B, H, L), dev)
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H, L), dev)
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    _check(out, "out", dt, (B, H, L, d), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, L), device=dev, dtype=torch.float32)
        mine.append(lse)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, L), dev)
    need = fwd_workspace_size(B, H, L, d, dt)
    if need == 0:
        raise PathError(PATH_EUNSUPPORTED if d not in (64, 128) else PATH_EINVAL, "path_attn_fwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
        mine.append(workspace)
    _check(workspace, "workspace", None, None, dev)
    with torch.cuda.device(dev):
        _record(stream, *mine)
        st = lib().path_attn_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(wraw), _ptr(conv_w), _ptr(zbeta),
                                       float(beta_clip), _ptr(logf), _ptr(out), _ptr(lse), B, H, L, d, _DTYPES[dt],
                                       float(scale or 0.0), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_attn_fwd_fused")
    return (out, lse) if (return_lse or lse is not None) else out


def fwd_prep(q, k, v, w, beta, logf, out, lse, workspace, scale=None, stream=None):
    """First stage of the forward (path_attn_fwd_prep); tensors preallocated by the caller."""
    B, H, L, d = q.shape
    dev, dt = q.device, q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (w, "w"), (out, "out")):
        _check(t, n, dt, (B, H, L, d), dev)
    _check(beta, "beta", torch.float32, (B, H, L), dev)
    for t, n in ((logf, "logf"), (lse, "lse")):
        if t is not None:
            _check(t, n, torch.float32, (B, H, L), dev)
    _check(workspace, "workspace", None, None, dev)
    st = lib().path_attn_fwd_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(out), _ptr(lse),
                                  B, H, L, d, _DTYPES[q.dtype], float(scale or 0.0), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_attn_fwd_prep")


def fwd_scan(out, lse, has_logf, workspace, scale=None, stream=None):
    """Second stage of the forward (path_attn_fwd_scan) on a workspace filled by fwd_prep."""
    B, H, L, d = out.shape
    _check(out, "out", None, None, None)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, L), out.device)
    _check(workspace, "workspace", None, None, out.device)
    st = lib().path_attn_fwd_scan(_ptr(out), _ptr(lse), int(bool(has_logf)), B, H, L, d, _DTYPES[out.dtype],
                                  float(scale or 0.0), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_attn_fwd_scan")


def decode_step(kcache, vcache, n, q, w, beta, k_new=None, v_new=None, scale=None, out=None, lse=None,
                return_lse=False, workspace=None, stream=None, logf=None, fcache=None):
    """One PaTH decode step (path_decode_step, or path_decode_step_ex with the
    forget gate): updates kcache rows [0, n) in place.

    kcache, vcache: [B, H, ncap, d]; q, w, k_new, v_new: [B, H, d]; beta: [B, H] fp32.
    PaTH-FoX: logf [B, H] fp32 (log f of the current token) with fcache
    [B, H, ncap] fp32 (cumulative log f per cached row; row n is written when
    k_new is given).  Returns out [B, H, d] (and lse [B, H] when requested).
    """
    if kcache.dim() != 4:
        raise ValueError("kcache must be [B, H, ncap, d]")
    B, H, ncap, d = kcache.shape
    dt = kcache.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = kcache.device
    _check(kcache, "kcache", dt, (B, H, ncap, d), dev)
    _check(vcache, "vcache", dt, (B, H, ncap, d), dev)
    for t, nm in ((q, "q"), (w, "w")):
        _check(t, nm, dt, (B, H, d), dev)
    _check(beta, "beta", torch.float32, (B, H), dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if (logf is None) != (fcache is None):
        raise ValueError("logf and fcache go together")
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H), dev)
        _check(fcache, "fcache", torch.float32, (B, H, ncap), dev)
    if k_new is not None:
        _check(k_new, "k_new", dt, (B, H, d), dev)
        _check(v_new, "v_new", dt, (B, H, d), dev)
    mine = []
    if out is None:
        out = torch.empty((B, H, d), device=dev, dtype=dt)
        mine.append(out)
    _check(out, "out", dt, (B, H, d), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H), device=dev, dtype=torch.float32)
        mine.append(lse)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    rows = int(n) + (1 if k_new is not None else 0)
    need = decode_workspace_size(B, H, max(rows, 1), d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
        mine.append(workspace)
    _check(workspace, "workspace", None, None, dev)
    common = (_ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse), B, H, d, _DTYPES[dt], float(scale or 0.0),
              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    with torch.cuda.device(dev):
        _record(stream, *mine)
        if logf is None:
            name = "path_decode_step"
            st = lib().path_decode_step(_ptr(kcache), _ptr(vcache), int(n), ncap, _ptr(q), _ptr(w), _ptr(beta),
                                        *common)
        else:
            name = "path_decode_step_ex"
            st = lib().path_decode_step_ex(_ptr(kcache), _ptr(vcache), int(n), ncap, _ptr(q), _ptr(w), _ptr(beta),
                                           _ptr(logf), _ptr(fcache), *common)
    if st != PATH_OK:
        raise PathError(st, name)
    return (out, lse) if (return_lse or lse is not None) else out


def decode_step_fused(kcache, vcache, n, q, wraw, conv_w, zbeta, conv_state, beta_clip=0.0, k_new=None,
                      v_new=None, scale=None, out=None, lse=None, return_lse=False, workspace=None, stream=None,
                      logf=None, fcache=None):
    """One decode step with the producer of w and beta fused in (path_decode_step_fused):
    y_t = the width-3 causal convolution of (conv_state rows x_{t-2}, x_{t-1}, wraw = x_t)
    with conv_w, w_t = y_t / ||y_t||, beta_t = 2 sigmoid(zbeta) (capped at beta_clip > 0),
    then decode_step with (w_t, beta_t).  conv_state moves on to (x_{t-1}, x_t) in place.

    wraw: [B, H, d] and conv_state: [B, H, 2, d] in the cache's dtype; conv_w: [H, d, 3] fp32;
    zbeta: [B, H] fp32.  Every other argument as in decode_step.
    """
    if kcache.dim() != 4:
        raise ValueError("kcache must be [B, H, ncap, d]")
    B, H, ncap, d = kcache.shape
    dt = kcache.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = kcache.device
    _check(kcache, "kcache", dt, (B, H, ncap, d), dev)
    _check(vcache, "vcache", dt, (B, H, ncap, d), dev)
    for t, nm in ((q, "q"), (wraw, "wraw")):
        _check(t, nm, dt, (B, H, d), dev)
    _check(conv_state, "conv_state", dt, (B, H, 2, d), dev)
    _check(conv_w, "conv_w", torch.float32, (H, d, 3), dev)
    _check(zbeta, "zbeta", torch.float32, (B, H), dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if (logf is None) != (fcache is None):
        raise ValueError("logf and fcache go together")
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H), dev)
        _check(fcache, "fcache", torch.float32, (B, H, ncap), dev)
    if k_new is not None:
        _check(k_new, "k_new", dt, (B, H, d), dev)
        _check(v_new, "v_new", dt, (B, H, d), dev)
    mine = []
    if out is None:
        out = torch.empty((B, H, d), device=dev, dtype=dt)
        mine.append(out)
    _check(out, "out", dt, (B, H, d), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H), device=dev, dtype=torch.float32)
        mine.append(lse)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    rows = int(n) + (1 if k_new is not None else 0)
    need = decode_fused_workspace_size(B, H, max(rows, 1), d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
        mine.append(workspace)
    _check(workspace, "workspace", None, None, dev)
    with torch.cuda.device(dev):
        _record(stream, *mine)
        st = lib().path_decode_step_fused(_ptr(kcache), _ptr(vcache), int(n), ncap, _ptr(q), _ptr(wraw), _ptr(conv_w),
                                          _ptr(zbeta), float(beta_clip), _ptr(conv_state), _ptr(logf), _ptr(fcache),
                                          _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse), B, H, d, _DTYPES[dt],
                                          float(scale or 0.0), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_decode_step_fused")
    return (out, lse) if (return_lse or lse is not None) else out


def decode_step_noalloc(kcache, vcache, n, q, w, beta, out, k_new=None, v_new=None, scale=None, lse=None,
                        stream=None, logf=None, fcache=None):
    """decode_step through path_decode_step_noalloc: no workspace, the library's fixed
    scratch instead (calls overlapping on one device race).  The caller passes out
    (and lse, if wanted); nothing is allocated.  Returns out (and lse when given)."""
    if kcache.dim() != 4:
        raise ValueError("kcache must be [B, H, ncap, d]")
    B, H, ncap, d = kcache.shape
    dt = kcache.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = kcache.device
    _check(kcache, "kcache", dt, (B, H, ncap, d), dev)
    _check(vcache, "vcache", dt, (B, H, ncap, d), dev)
    for t, nm in ((q, "q"), (w, "w"), (out, "out")):
        _check(t, nm, dt, (B, H, d), dev)
    _check(beta, "beta", torch.float32, (B, H), dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if (logf is None) != (fcache is None):
        raise ValueError("logf and fcache go together")
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H), dev)
        _check(fcache, "fcache", torch.float32, (B, H, ncap), dev)
    if k_new is not None:
        _check(k_new, "k_new", dt, (B, H, d), dev)
        _check(v_new, "v_new", dt, (B, H, d), dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    with torch.cuda.device(dev):
        st = lib().path_decode_step_noalloc(_ptr(kcache), _ptr(vcache), int(n), ncap, _ptr(q), _ptr(w), _ptr(beta),
                                            _ptr(logf), _ptr(fcache), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse),
                                            B, H, d, _DTYPES[dt], float(scale or 0.0), _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_decode_step_noalloc")
    return (out, lse) if lse is not None else out


def decode_cache_from_fwd(workspace, v, kcache, vcache, stream=None, logf=None, fcache=None):
    """Fill decode caches from a forward pass's workspace (path_decode_cache_from_fwd).

    workspace: the workspace a fwd / fwd_prep call over this prefix used (same
    B, H, L, d, dtype); v: [B, H, L, d] prefix values; kcache, vcache:
    [B, H, ncap, d] with ncap >= L, rows [0, L) written: kcache row j =
    H_{L-1} ... H_{j+1} k_j, vcache row j = v_j.  With logf [B, H, L] and
    fcache [B, H, ncap] (fp32) the gate cache gets the prefix sums of log f.
    """
    if v.dim() != 4 or kcache.dim() != 4:
        raise ValueError("v must be [B, H, L, d] and kcache [B, H, ncap, d]")
    B, H, L, d = v.shape
    ncap = kcache.shape[2]
    dt, dev = v.dtype, v.device
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    _check(v, "v", dt, (B, H, L, d), dev)
    _check(kcache, "kcache", dt, (B, H, ncap, d), dev)
    _check(vcache, "vcache", dt, (B, H, ncap, d), dev)
    _check(workspace, "workspace", None, None, dev)
    if (logf is None) != (fcache is None):
        raise ValueError("logf and fcache go together")
    if logf is not None:
        _check(logf, "logf", torch.float32, (B, H, L), dev)
        _check(fcache, "fcache", torch.float32, (B, H, ncap), dev)
    with torch.cuda.device(dev):
        st = lib().path_decode_cache_from_fwd(_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(v),
                                              _ptr(logf), _ptr(kcache), _ptr(vcache), _ptr(fcache), int(ncap), B, H,
                                              L, d, _DTYPES[dt], _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_decode_cache_from_fwd")
    return kcache, vcache


def bwd_workspace_size(B, H, L, d, dtype=torch.bfloat16):
    return int(lib().path_attn_bwd_workspace_size(B, H, L, d, _DTYPES[dtype]))


def bwd(q, k, v, w, beta, logf, out, lse, dout, dlse=None, scale=None, workspace=None, stream=None, grads=None):
    """Backward of fwd (path_attn_bwd): gradients of sum(dout * out) + sum(dlse * lse).

    q, k, v, w, out, dout: [B, H, L, d] (bf16 or fp32, one dtype); beta, lse, logf,
    dlse: [B, H, L] fp32 (logf, dlse optional); out and lse are fwd's outputs.
    Returns (dq, dk, dv, dw, dbeta, dlogf) with dlogf None without logf; grads
    may supply those output tensors.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (w, "w"), (out, "out"), (dout, "dout")):
        _check(t, n, dt, (B, H, L, d), dev)
    for t, n in ((beta, "beta"), (lse, "lse"), (logf, "logf"), (dlse, "dlse")):
        if t is not None:
            _check(t, n, torch.float32, (B, H, L), dev)
    mine = []
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                 torch.empty((B, H, L), device=dev, dtype=torch.float32),
                 torch.empty((B, H, L), device=dev, dtype=torch.float32) if logf is not None else None)
        mine.extend(grads)
    dq, dk, dv, dw, dbeta, dlogf = grads
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dw, "dw")):
        _check(t, n, dt, (B, H, L, d), dev)
    _check(dbeta, "dbeta", torch.float32, (B, H, L), dev)
    if dlogf is not None:
        _check(dlogf, "dlogf", torch.float32, (B, H, L), dev)
    if workspace is None:
        need = bwd_workspace_size(B, H, L, d, dt)
        if need == 0:
            raise PathError(PATH_EUNSUPPORTED if d not in (64, 128) else PATH_EINVAL, "path_attn_bwd_workspace_size")
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
        mine.append(workspace)
    _check(workspace, "workspace", None, None, dev)
    with torch.cuda.device(dev):
        _record(stream, *mine)
        st = lib().path_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(out), _ptr(lse),
                                 _ptr(dout), _ptr(dlse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(dbeta),
                                 _ptr(dlogf), B, H, L, d, _DTYPES[dt], float(scale or 0.0), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PATH_OK:
        raise PathError(st, "path_attn_bwd")
    return dq, dk, dv, dw, dbeta, dlogf
