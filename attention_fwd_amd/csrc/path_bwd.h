// path_bwd.h -- launch interface of the backward kernels (path_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace path {

// Byte offsets inside one head's share of the backward workspace (fp32 arrays;
// Lp = 64 * ceil(L / 64) padded rows, nb blocks, np = nb (nb - 1) / 2 pairs of
// a query block I and an earlier key block J, pair index I (I - 1) / 2 + J).
struct BwdLayout {
    int64_t qh, kh, vf, dof;  // [Lp, 64]: block-adjusted q and k (fp32), copies of v and do (input type)
    int64_t tt, ttt, ee;      // [nb, 64, 64]: block transitions and their transposes, scale * dS of the diagonal blocks
    int64_t dvd, dqo, dko, dvo;  // [Lp, 64]: diagonal value gradient; walk outputs dq^, dk^, dv
    int64_t dt;               // [nb, 64, 64]: gradient of each block transition
    int64_t xx, aa, qwm, nn, zz;  // [nb, 64, 64]: X, A, Q W^T o [r <= i], N, Z of each block (prep -> block backward)
    int64_t l2, dd, clq, ckk;  // [Lp]: lse in log2 units, do.o - dlse, gate prefix terms of rows / keys
    int64_t rsd, csd, rso, cso, dc;  // [Lp]: row / column sums of dS (diagonal, off-diagonal), gate adjoint
    int64_t tot;              // [nb]: gate total of each block
    int64_t mid;              // [np]: gate sum over the blocks strictly between I and J
    int64_t qs, gs;           // [np, 64, 64]: carried queries q~_I^(J) and adjoints G_I^(J-1)
    int64_t ps, ds;           // [np, 64, 64]: softmax weights P and dS of every pair
    int64_t csp;              // [np, 64]: column sums of each pair's dS (fp32)
    // qs, gs, ps, ds hold the input element type (bf16 for bf16 inputs, else fp32)
    int64_t head;             // bytes per head
};

BwdLayout bwd_layout(int L, int elem_bytes);

struct BwdArgs {
    const void *q, *k, *v, *w;
    const float *beta, *logf;
    const void *out;
    const float *lse;
    const void *dout;
    const float *dlse;
    void *dq, *dk, *dv, *dw;
    float *dbeta, *dlogf;
    void *ws;
    int B, H, L, d;
    float scale;
    int nb;
    int g0, hc, hc_max;  // heads [g0, g0 + hc) in flight; at most hc_max per pass over the workspace
    BwdLayout ly;
};

hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t st);

}  // namespace path
