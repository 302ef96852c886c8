"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` function takes the path of an oracle build and raises
AssertionError when that build disagrees with an independent fact:
  * a hand-derived example (tests/golden/hand_L3_d2.txt),
  * explicit dense d x d products of the transition matrices (brute force),
  * the UT-transform closed form of a product of transitions, P = I - W^T T^-1 W
    with T = diag(1/beta) + strictly-upper(W W^T) (Japanese technical summary
    "技術要約: PaTH Attention", section 3, UT-transform representation; the
    pages only say T is triangular and derived from beta, the explicit T is
    the classical compact representation of accumulated Householder-like
    transforms),
  * beta = 0 reducing to plain causal softmax attention (torch SDPA, fp64),
  * beta = 2 making every H an orthogonal reflection (norms, det = (-1)^n),
  * beta = 1 making every H a projector,
  * all w equal with beta = 2 (H^2 = I: closed form by parity),
  * decode reproducing forward rows (the in-place key update of section 3),
  * the decode cache after a prefix equal to explicit products and to feeding
    the prefix through decode steps one token at a time,
  * the backward: finite differences of a dense forward, autograd of a dense
    torch fp64 forward, the softmax-attention gradient at beta = 0, and exact
    invariances of the loss.
They are used by test_oracle_pins.py on the real oracle and by
test_oracle_mutants.py on deliberately broken copies of it.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_L3_d2.txt")


def _rand_inputs(L, d, seed, beta=None, fox=False):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    w = rng.standard_normal((L, d))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    b = 2.0 / (1.0 + np.exp(-rng.standard_normal(L))) if beta is None else np.full(L, float(beta))
    lf = np.log(1.0 / (1.0 + np.exp(-(3.0 + rng.standard_normal(L))))) if fox else None
    return q, k, v, w, b, lf


def _H(w, b):
    return np.eye(w.shape[0]) - b * np.outer(w, w)


def _brute_scores(q, k, w, b, lf, scale):
    L, d = q.shape
    S = np.full((L, L), -np.inf)
    for i in range(L):
        for j in range(i + 1):
            M = np.eye(d)
            for s in range(j + 1, i + 1):
                M = M @ _H(w[s], b[s])
            S[i, j] = scale * k[j] @ M @ q[i]
            if lf is not None:
                S[i, j] += sum(lf[s] for s in range(j + 1, i + 1))
    return S


def _softmax_out(S, v):
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    z = P.sum(axis=1, keepdims=True)
    return (P / z) @ v, (m + np.log(z))[:, 0]


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, "%s: max-abs %.3e > %.1e" % (what, err, tol)


def load_golden():
    g = {"s": {}, "bias": {}}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, *vals = line.split()
            vals = [float(x) for x in vals]
            if name in ("s", "bias"):
                g[name][(int(vals[0]), int(vals[1]))] = vals[2]
            else:
                g[name] = np.array(vals)
    for n in ("w", "q", "k", "v"):
        g[n] = g[n].reshape(-1, 2)
    return g


def pin_golden(lib):
    g = load_golden()
    S = oracle.scores(g["q"], g["k"], g["w"], g["beta"], scale=1.0, lib=lib)
    SF = oracle.scores(g["q"], g["k"], g["w"], g["beta"], logf=g["logf"], scale=1.0, lib=lib)
    for (i, j), s in g["s"].items():
        _close(S[i, j], s, 1e-13, "golden s_%d%d" % (i, j))
        _close(SF[i, j], s + g["bias"].get((i, j), 0.0), 1e-13, "golden FoX s_%d%d" % (i, j))
    for fox in (False, True):
        out, lse = oracle.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"] if fox else None,
                              scale=1.0, lib=lib)
        for i in range(3):
            logits = [g["s"][(i, j)] + (g["bias"].get((i, j), 0.0) if fox else 0.0) for j in range(i + 1)]
            e = [math.exp(x) for x in logits]
            z = sum(e)
            o = sum(e[j] * g["v"][j] for j in range(i + 1)) / z
            _close(out[i], o, 1e-13, "golden o_%d fox=%s" % (i, fox))
            _close(lse[i], math.log(z), 1e-13, "golden lse_%d" % i)


def pin_bruteforce(lib):
    for (L, d, seed, fox) in ((9, 5, 1, False), (12, 8, 2, True), (7, 3, 3, False)):
        q, k, v, w, b, lf = _rand_inputs(L, d, seed, fox=fox)
        scale = 1.0 / math.sqrt(d)
        Sb = _brute_scores(q, k, w, b, lf, scale)
        S = oracle.scores(q, k, w, b, logf=lf, scale=scale, lib=lib)
        _close(S[np.tril_indices(L)], Sb[np.tril_indices(L)], 1e-12, "brute scores L%d d%d" % (L, d))
        assert np.all(np.isneginf(S[np.triu_indices(L, 1)])), "non-causal scores present"
        ob, lb = _softmax_out(Sb, v)
        out, lse = oracle.fwd(q, k, v, w, b, logf=lf, scale=scale, lib=lib)
        _close(out, ob, 1e-12, "brute out L%d d%d" % (L, d))
        _close(lse, lb, 1e-12, "brute lse L%d d%d" % (L, d))


def _ut_product(W, beta, upper=True):
    """I - W^T T^-1 W with T = diag(1/beta) + strictly-upper (or -lower) part of W W^T."""
    G = W @ W.T
    T = np.diag(1.0 / beta) + (np.triu(G, 1) if upper else np.tril(G, -1))
    return np.eye(W.shape[1]) - W.T @ np.linalg.solve(T, W)


def pin_ut_closed_form(lib):
    for (n, d, seed) in ((7, 6, 4), (5, 9, 5), (12, 4, 6)):
        _, _, _, w, b, _ = _rand_inputs(n, d, seed)
        # columns of H_0 H_1 ... H_{n-1} from the oracle's transport of basis vectors
        P = np.stack([oracle.transport(np.eye(d)[c], w, b, 0, n - 1, lib=lib) for c in range(d)], axis=1)
        _close(P, _ut_product(w, b, upper=True), 1e-12, "UT form, increasing order")
        # reverse order H_{n-1} ... H_0 is the transpose (every H is symmetric), whose
        # UT form takes the strictly-lower part
        _close(P.T, _ut_product(w, b, upper=False), 1e-12, "UT form, decreasing order")
        # logits through the UT form of each path product
        q, k, _, _, _, _ = _rand_inputs(n, d, seed + 100)
        S = oracle.scores(q, k, w, b, scale=0.5, lib=lib)
        for i in range(n):
            for j in range(i):
                Pij = _ut_product(w[j + 1:i + 1], b[j + 1:i + 1])
                _close(S[i, j], 0.5 * k[j] @ Pij @ q[i], 1e-12, "UT logit (%d,%d)" % (i, j))


def pin_beta_zero(lib):
    L, d = 33, 16
    for fox in (False, True):
        q, k, v, w, b, lf = _rand_inputs(L, d, 7, beta=0.0, fox=fox)
        out, lse = oracle.fwd(q, k, v, w, b, logf=lf, lib=lib)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        if fox:
            c = np.cumsum(lf)
            mask = c[:, None] - c[None, :]
            mask[np.triu_indices(L, 1)] = -np.inf
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=torch.from_numpy(mask)[None, None])
        else:
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
        _close(out, ref[0, 0].numpy(), 1e-12, "beta=0 vs causal SDPA fox=%s" % fox)
        S = (q @ k.T) / math.sqrt(d)
        if fox:
            S = S + mask
        S[np.triu_indices(L, 1)] = -np.inf
        m = S.max(axis=1)
        _close(lse, m + np.log(np.exp(S - m[:, None]).sum(axis=1)), 1e-12, "beta=0 lse")


def pin_beta_two(lib):
    n, d = 10, 6
    q, _, _, w, b, _ = _rand_inputs(n, d, 8, beta=2.0)
    for lo, hi in ((0, n - 1), (3, 8), (5, 5)):
        P = np.stack([oracle.transport(np.eye(d)[c], w, b, lo, hi, lib=lib) for c in range(d)], axis=1)
        _close(P.T @ P, np.eye(d), 1e-12, "beta=2 orthogonality")
        _close(np.linalg.det(P), (-1.0) ** (hi - lo + 1), 1e-10, "beta=2 det")
        for i in range(n):
            u = oracle.transport(q[i], w, b, lo, hi, lib=lib)
            _close(np.linalg.norm(u), np.linalg.norm(q[i]), 1e-12, "beta=2 norm")


def pin_beta_one(lib):
    n, d = 6, 5
    q, _, _, w, b, _ = _rand_inputs(n, d, 9, beta=1.0)
    for s in range(n):
        _close(oracle.transport(w[s], w, b, s, s, lib=lib), np.zeros(d), 1e-14, "beta=1: H w = 0")
        once = oracle.transport(q[s], w, b, s, s, lib=lib)
        twice = oracle.transport(once, w, b, s, s, lib=lib)
        _close(twice, once, 1e-14, "beta=1: H^2 = H")
        _close(once @ w[s], 0.0, 1e-14, "beta=1: H q orthogonal to w")


def pin_equal_w(lib):
    L, d = 11, 7
    q, k, v, w, _, _ = _rand_inputs(L, d, 10, beta=2.0)
    w[:] = w[0]
    b = np.full(L, 2.0)
    S = oracle.scores(q, k, w, b, scale=1.0, lib=lib)
    for i in range(L):
        refl = q[i] - 2.0 * (w[0] @ q[i]) * w[0]
        for j in range(i + 1):
            ref = k[j] @ (q[i] if (i - j) % 2 == 0 else refl)
            _close(S[i, j], ref, 1e-12, "equal w, beta=2 parity closed form (%d,%d)" % (i, j))


def pin_small_L(lib):
    rng = np.random.default_rng(11)
    d = 4
    q, k, v, w = (rng.standard_normal((2, d)) for _ in range(4))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    b = np.array([0.7, 1.3])
    out, lse = oracle.fwd(q[:1], k[:1], v[:1], w[:1], b[:1], scale=0.5, lib=lib)
    _close(out[0], v[0], 1e-15, "L=1: o_0 = v_0")
    _close(lse[0], 0.5 * k[0] @ q[0], 1e-15, "L=1: lse")
    out, lse = oracle.fwd(q, k, v, w, b, scale=0.5, lib=lib)
    s10 = 0.5 * k[0] @ (q[1] - b[1] * (w[1] @ q[1]) * w[1])
    s11 = 0.5 * k[1] @ q[1]
    e0, e1 = math.exp(s10), math.exp(s11)
    _close(out[1], (e0 * v[0] + e1 * v[1]) / (e0 + e1), 1e-14, "L=2 by hand")


def pin_fox_zero(lib):
    q, k, v, w, b, _ = _rand_inputs(20, 8, 12)
    o1, l1 = oracle.fwd(q, k, v, w, b, lib=lib)
    o2, l2 = oracle.fwd(q, k, v, w, b, logf=np.zeros(20), lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "log f = 0 must reduce to plain PaTH"


def pin_rows_subset(lib):
    q, k, v, w, b, lf = _rand_inputs(30, 8, 13, fox=True)
    qs, ks, vs, ws = (np.stack([x, x[::-1].copy()]) for x in (q, k, v, w))
    bs, lfs = np.stack([b, b[::-1].copy()]), np.stack([lf, lf[::-1].copy()])
    full_o, full_l = oracle.fwd(qs, ks, vs, ws, bs, logf=lfs, lib=lib)
    rows = np.array([[0, 0], [1, 29], [0, 17], [1, 3]])
    ro, rl = oracle.fwd(qs, ks, vs, ws, bs, logf=lfs, rows=rows, lib=lib)
    for t, (g, i) in enumerate(rows):
        assert np.array_equal(ro[t], full_o[g, i]) and rl[t] == full_l[g, i], "row sampling differs"


def pin_decode(lib):
    """Decode from an empty cache reproduces forward rows; cache rows equal explicit H_t k_j."""
    T, d = 14, 6
    q, k, v, w, b, _ = _rand_inputs(T, d, 14)
    ref_o, ref_l = oracle.fwd(q, k, v, w, b, lib=lib)
    kc = np.zeros((T, d))
    vc = np.zeros((T, d))
    for t in range(T):
        before = kc.copy()
        kc, vc, o, l = oracle.decode(kc, vc, t, q[t], w[t], b[t], k_new=k[t], v_new=v[t], lib=lib)
        _close(o, ref_o[t], 1e-12, "decode step %d vs forward row" % t)
        _close(l, ref_l[t], 1e-12, "decode lse %d" % t)
        Ht = _H(w[t], b[t])
        _close(kc[:t], before[:t] @ Ht.T, 1e-13, "in-place cache update at step %d" % t)
        _close(kc[t], k[t], 0.0, "new key enters untransformed")
    # no new token: attend to the n updated rows only
    kc2, _, o, l = oracle.decode(kc, vc, T, q[0], w[0], b[0], lib=lib)
    ku = kc @ _H(w[0], b[0]).T
    s = ku @ q[0] / math.sqrt(d)
    p = np.exp(s - s.max())
    _close(o, p @ vc / p.sum(), 1e-13, "decode without new token")
    _close(kc2, ku, 1e-13, "decode cache without new token")


def pin_decode_fox(lib):
    """Decode with the forget gate from an empty cache reproduces the PaTH-FoX forward row by row,
    and the gate cache holds the inclusive prefix sums of log f."""
    T, d = 13, 5
    q, k, v, w, b, lf = _rand_inputs(T, d, 31, fox=True)
    ref_o, ref_l = oracle.fwd(q, k, v, w, b, lf, lib=lib)
    kc, vc, fc = np.zeros((T, d)), np.zeros((T, d)), np.zeros(T)
    for t in range(T):
        kc, vc, o, l, fc = oracle.decode(kc, vc, t, q[t], w[t], b[t], k_new=k[t], v_new=v[t], lib=lib,
                                         logf=np.array(lf[t]), fcache=fc)
        _close(o, ref_o[t], 1e-12, "gated decode step %d vs forward row" % t)
        _close(l, ref_l[t], 1e-12, "gated decode lse %d" % t)
    _close(fc, np.cumsum(lf), 1e-13, "gate cache = prefix sums of log f")
    _, fc2 = oracle.decode_cache(k, w, b, lib=lib, logf=lf)
    _close(fc2, fc, 1e-13, "decode-cache gate column = the gated decode's")
    # without a new token the query at position n attends to the n updated rows with bias c_n - c_j
    n = T
    kc2, _, o, _, _ = oracle.decode(kc, vc, n, q[0], w[0], b[0], lib=lib, logf=np.array(-0.7), fcache=fc)
    ct = fc[n - 1] - 0.7
    s_ = kc2 @ q[0] / math.sqrt(d) + (ct - fc)
    p = np.exp(s_ - s_.max())
    _close(o, p @ vc / p.sum(), 1e-13, "gated decode without new token")


def pin_decode_cache(lib):
    """Decode cache after a prefix: explicit products H_{L-1} ... H_{j+1} k_j (brute force),
    equality with feeding the prefix through decode steps one token at a time, and the
    special cases beta = 0 (cache = keys) and beta = 1 (every older row orthogonal to
    the last w, since H = I - w w^T annihilates w)."""
    L, d = 11, 5
    q, k, v, w, b, _ = _rand_inputs(L, d, 21)
    got = oracle.decode_cache(k, w, b, lib=lib)
    for j in range(L):
        M = np.eye(d)
        for s in range(j + 1, L):
            M = _H(w[s], b[s]) @ M  # H_{j+1} acts first
        _close(got[j], M @ k[j], 1e-13, "decode cache row %d vs explicit product" % j)
    kc = np.zeros((L, d))
    vc = np.zeros((L, d))
    for t in range(L):
        kc, vc, _, _ = oracle.decode(kc, vc, t, q[t], w[t], b[t], k_new=k[t], v_new=v[t], lib=lib)
    _close(got, kc, 1e-13, "decode cache vs token-by-token decode")
    _, _, _, w0, _, _ = _rand_inputs(L, d, 22)
    _close(oracle.decode_cache(k, w0, np.zeros(L), lib=lib), k, 0.0, "beta = 0 leaves the keys")
    c1 = oracle.decode_cache(k, w0, np.ones(L), lib=lib)
    _close(c1[:-1] @ w0[-1], np.zeros(L - 1), 1e-13, "beta = 1: older rows orthogonal to the last w")
    _close(c1[-1], k[-1], 0.0, "last row untransformed")


def pin_produce(lib):
    """Producer of w and beta: the causal width-3 depthwise convolution and the L2
    normalisation against torch's conv1d (fp64, padding 2, first L outputs: output t
    is sum_tau cw[tau] x_{t-2+tau}) and F.normalize (eps 1e-12), per head with the
    head's own weights; beta against 2 sigmoid(z) capped by torch.clamp; a token
    whose window is all zero gives w = 0; the fused forward ignores the scale of
    wraw and equals the forward on the produced (w, beta)."""
    B, H, L, d = 2, 3, 9, 5
    rng = np.random.default_rng(31)
    x = rng.standard_normal((B, H, L, d))
    x[1, 2, 3:6] = 0.0  # token 5 of that head sees only zeros
    cw = rng.standard_normal((H, d, 3))
    z = 2.0 * rng.standard_normal((B, H, L))
    z[0, 0, :3] = 8.0  # 2 sigmoid(8) > 1.98: the cap applies
    clip = 1.98
    w, b = oracle.produce(x, cw, z, clip, lib=lib)
    xt = torch.from_numpy(x)
    for h in range(H):
        inp = xt[:, h].transpose(1, 2)  # [B, d, L]
        y = torch.nn.functional.conv1d(inp, torch.from_numpy(cw[h]).unsqueeze(1), padding=2, groups=d)[..., :L]
        ref = torch.nn.functional.normalize(y.transpose(1, 2), dim=-1, eps=1e-12).numpy()
        _close(w[:, h], ref, 1e-14, "w of head %d vs conv1d + normalize" % h)
    _close(w[1, 2, 5], np.zeros(d), 0.0, "all-zero window gives w = 0")
    bref = torch.clamp(2.0 * torch.sigmoid(torch.from_numpy(z)), max=clip).numpy()
    _close(b, bref, 1e-15, "beta vs 2 sigmoid(z) capped")
    assert float(b.max()) == clip, "cap reached"
    _, b_free = oracle.produce(x, cw, z, 0.0, lib=lib)
    assert float(b_free.max()) > clip, "no cap without beta_clip"
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    o1, l1 = oracle.fwd_fused(q, k, v, x, cw, z, clip, lib=lib)
    o2, l2 = oracle.fwd_fused(q, k, v, 3.5 * x, cw, z, clip, lib=lib)
    _close(o1, o2, 1e-12, "fused forward independent of the scale of wraw")
    o3, l3 = oracle.fwd(q, k, v, w, b, lib=lib)
    _close(o1, o3, 0.0, "fused forward = forward on the produced (w, beta)")


# ---------------------------------------------------------------------------
# Backward pass.  The pages print no gradient formulas; what pins the oracle's
# gradient is the calculus itself: central finite differences of a forward
# written with explicit dense transition products (no shared code with the
# oracle), autograd of a dense torch fp64 implementation, the textbook
# softmax-attention gradient at beta = 0, and exact invariances of the loss.
# ---------------------------------------------------------------------------

def _bwd_case(L, d, seed, beta=None, fox=False):
    q, k, v, w, b, lf = _rand_inputs(L, d, seed, beta=beta, fox=fox)
    rng = np.random.default_rng(seed + 1000)
    return dict(q=q, k=k, v=v, w=w, beta=b, logf=lf), rng.standard_normal((L, d)), rng.standard_normal(L)


def _dense_loss(x, dout, dlse, scale):
    S = _brute_scores(x["q"], x["k"], x["w"], x["beta"], x["logf"], scale)
    o, lse = _softmax_out(S, x["v"])
    return float((o * dout).sum() + (lse * dlse).sum())


def pin_bwd_finite_diff(lib):
    """Directional derivatives of the loss against central differences of a dense numpy forward."""
    for (L, d, beta, fox, seed) in [(1, 3, None, False, 1), (2, 2, None, True, 2), (5, 3, None, True, 3),
                                    (9, 4, None, True, 4), (7, 3, 2.0, False, 5), (6, 3, 1.0, True, 6)]:
        x, dout, dlse = _bwd_case(L, d, seed, beta=beta, fox=fox)
        scale = 0.7
        g = oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], dout, dlse, scale=scale, lib=lib)
        S = _brute_scores(x["q"], x["k"], x["w"], x["beta"], x["logf"], scale)
        o, lse = _softmax_out(S, x["v"])
        _close(g["o"], o, 1e-12, "backward's forward output")
        _close(g["lse"], lse, 1e-12, "backward's lse")
        rng = np.random.default_rng(seed + 77)
        for name in ("q", "k", "v", "w", "beta", "logf"):
            if x[name] is None:
                continue
            for _ in range(3):
                dirn = rng.standard_normal(x[name].shape)
                eps = 1e-5
                xp, xm = dict(x), dict(x)
                xp[name] = x[name] + eps * dirn
                xm[name] = x[name] - eps * dirn
                fd = (_dense_loss(xp, dout, dlse, scale) - _dense_loss(xm, dout, dlse, scale)) / (2 * eps)
                an = float((g["d" + name] * dirn).sum())
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                    "d%s L%d: finite difference %.9g vs gradient %.9g" % (name, L, fd, an)


def _torch_dense_forward(t, scale):
    """Dense fp64 torch forward with explicit d x d products (for autograd)."""
    L, d = t["q"].shape
    I = torch.eye(d, dtype=torch.float64)
    Hs = [I - t["beta"][s] * torch.outer(t["w"][s], t["w"][s]) for s in range(L)]
    c = torch.cumsum(t["logf"], 0) if "logf" in t else None
    rows_o, rows_l = [], []
    for i in range(L):
        logits = []
        for j in range(i + 1):
            M = I
            for s in range(j + 1, i + 1):
                M = M @ Hs[s]
            sij = scale * (t["k"][j] @ (M @ t["q"][i]))
            if c is not None:
                sij = sij + (c[i] - c[j])
            logits.append(sij)
        sv = torch.stack(logits)
        p = torch.softmax(sv, 0)
        rows_o.append(p @ t["v"][: i + 1])
        rows_l.append(torch.logsumexp(sv, 0))
    return torch.stack(rows_o), torch.stack(rows_l)


def pin_bwd_autograd(lib):
    """Every gradient element against torch autograd of the dense fp64 forward."""
    for (L, d, beta, fox, seed) in [(4, 3, None, True, 11), (8, 5, None, True, 12), (6, 4, None, False, 13)]:
        x, dout, dlse = _bwd_case(L, d, seed, beta=beta, fox=fox)
        scale = 0.45
        t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items() if a is not None}
        o, lse = _torch_dense_forward(t, scale)
        ((o * torch.from_numpy(dout)).sum() + (lse * torch.from_numpy(dlse)).sum()).backward()
        g = oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], dout, dlse, scale=scale, lib=lib)
        for n in t:
            ref = t[n].grad.numpy()
            _close(g["d" + n], ref, 1e-11 * max(1.0, float(np.abs(ref).max())), "autograd d%s L%d" % (n, L))


def pin_bwd_beta_zero(lib):
    """beta = 0: the textbook gradient of causal softmax attention (torch SDPA, fp64), and dw = 0."""
    L, d = 24, 8
    for fox in (False, True):
        x, dout, dlse = _bwd_case(L, d, 21, beta=0.0, fox=fox)
        tq, tk, tv = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
        if fox:
            tl = torch.tensor(x["logf"], requires_grad=True)
            c = torch.cumsum(tl, 0)
            mask = (c[:, None] - c[None, :]).masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
            o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                                 attn_mask=mask[None, None])[0, 0]
        else:
            o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                                 is_causal=True)[0, 0]
        (o * torch.from_numpy(dout)).sum().backward()
        g = oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], dout, None, lib=lib)
        for n, tt in (("q", tq), ("k", tk), ("v", tv)):
            _close(g["d" + n], tt.grad.numpy(), 1e-11, "beta=0 d%s fox=%s" % (n, fox))
        if fox:
            _close(g["dlogf"], tl.grad.numpy(), 1e-11, "beta=0 dlogf")
        _close(g["dw"], np.zeros_like(x["w"]), 0.0, "beta=0 dw")


def pin_bwd_invariants(lib):
    """Exact identities of the loss: each H_t is unchanged by (w_t, beta_t) -> (a w_t, beta_t / a^2), so
    w_t . dw_t = 2 beta_t dbeta_t; the logits are unchanged by (q, k) -> (a q, k / a), so
    sum q . dq = sum k . dk; the weights of a row sum to 1, so sum_j dv_j = sum_i do_i; no bias path
    crosses token 0, so dlogf_0 = 0; and a zero upstream gradient gives zero gradients."""
    L, d = 40, 6
    x, dout, dlse = _bwd_case(L, d, 31, fox=True)
    g = oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], dout, dlse, lib=lib)
    gs = max(1.0, float(np.abs(g["dw"]).max()), float(np.abs(g["dbeta"]).max()))
    _close((g["dw"] * x["w"]).sum(-1), 2 * x["beta"] * g["dbeta"], 1e-10 * gs, "w.dw = 2 beta dbeta")
    _close((g["dq"] * x["q"]).sum(), (g["dk"] * x["k"]).sum(), 1e-10 * max(1.0, float(np.abs(g["dq"]).max())),
           "sum q.dq = sum k.dk")
    _close(g["dv"].sum(0), dout.sum(0), 1e-10, "sum_j dv_j = sum_i do_i")
    assert g["dlogf"][0] == 0.0, "dlogf_0 = %r" % g["dlogf"][0]
    z = oracle.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], np.zeros_like(dout), None, lib=lib)
    for n in ("dq", "dk", "dv", "dw", "dbeta", "dlogf"):
        _close(z[n], np.zeros_like(z[n]), 0.0, "zero upstream gradient " + n)


ALL_PINS = [pin_golden, pin_bruteforce, pin_ut_closed_form, pin_beta_zero, pin_beta_two, pin_beta_one,
            pin_equal_w, pin_small_L, pin_fox_zero, pin_rows_subset, pin_decode, pin_decode_fox, pin_decode_cache,
            pin_produce, pin_bwd_finite_diff, pin_bwd_autograd, pin_bwd_beta_zero, pin_bwd_invariants]
