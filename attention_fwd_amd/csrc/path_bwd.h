// path_bwd.h -- launch interface of the backward kernels (path_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace path {

// Byte offsets inside one head's share of the backward workspace.  Lp = 64 nb
// padded rows, nb blocks, np = nb (nb - 1) / 2 pairs of a query block I and an
// earlier key block J (pair index I (I - 1) / 2 + J).  "Fragments" are stored
// in matrix-core fragment order in the element type S of the inputs (bf16 or
// fp32): a matrix X of R rows and K contraction columns is kept as (R / 32) x
// (K / 16) fragments of 64 lanes x 8 elements (see path_common.h), so a walk
// reads each operand with one 16- or 32-byte load per lane.
struct BwdLayout {
    int D, es;
    // per block, fp32 64 x 64: X, A, Q W^T o [r <= i], N = K W^T o [r > j], Z, and scale * dS of the diagonal block
    int64_t xx, aa, qwm, nn, zz, ee;
    // per block, fragments (S): the up walk's record -- k^ (rows keys, k over d), V (rows keys), k^^T
    // (rows d, k over keys) and (T - I)^T of the block transition T (rows d, k over d), contiguous, of
    // rec_elems elements (parts at 0, 64 D, 128 D, 192 D) -- and dO (rows queries), dO^T (rows d; none
    // for bf16 inputs), T - I (rows d, k over d)
    int64_t urec, rec_elems, do1, do2, nt;
    // fp32 [Lp, D]: q^; the diagonal value gradient; walk outputs dq^, dk^, dv; W dT and W dT^T of the
    // block backward
    int64_t qh, dvd, dqo, dko, dvo, uu, vv;
    int64_t dtt;  // per block, fp32 [D, D]: dT^T (the transpose of the transition gradient)
    // fp32 [Lp]: do.o - dlse; the query and key terms of the exponent of P in log2 units (a query's
    // block-local gate prefix less its lse, a key's gate sum to the end of its block); row / column
    // sums of dS (diagonal, off-diagonal); gate adjoint
    int64_t dd, cql, ckl, rsd, csd, rso, cso, dc;
    int64_t tot;  // [nb]: gate total of each block (log2 units)
    int64_t mid;  // [np]: gate sum over the blocks strictly between I and J (log2 units)
    // per pair, fragments (S): q~ (rows queries, k over d), q~^T (rows d, k over queries; none for bf16
    // inputs), G^(J-1)^T (rows d; for bf16 inputs G^(J-1) with rows queries, k over d; plus one
    // spare set at the end)
    int64_t qs1, qs2, gs2;
    int64_t head;  // bytes per head
};

BwdLayout bwd_layout(int L, int D, int elem_bytes);

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
