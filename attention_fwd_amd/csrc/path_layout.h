// path_layout.h -- sizes and offsets of the forward workspace (host and device).
//
// The sequence of every (batch, head) is cut into blocks of kBlk = 64 tokens
// (nb = ceil(L / 64) blocks, Lp = 64 * nb padded rows).  The prep kernel
// writes, per block J:
//   record J   : K-hat (64 x d), V^T (d x 64) and -M_J (d x d), each stored as
//                matrix-core fragments (see path_common.h), contiguous, so the
//                forward kernel streams one record per key block;
//   qhat       : boundary-adjusted queries times scale * log2(e) (logits in
//                log2 units), [Lp, d] natural row order;
//   mdiag/ldiag: running max (log2 units) and sum of the diagonal block;
//   fq/fk/fb   : forget-gate prefix terms (log2 units), used with logf only;
//   kn         : per block, max_j ||k_j|| if every transition of the block is a
//                contraction (0 <= beta ||w||^2 <= 2), else +inf (with logf);
//   redo       : per wave of the forward kernel (at most bh * (2 nb + 8) of
//                them), 1 when the bounded walk of its queries must be
//                repeated with the running max (written by the forward
//                kernel's bounded walk).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace path {

constexpr int kBlk = 64;

struct FwdLayout {
    int64_t bh, nb, lp, d, es;
    int64_t rec_elems;  // elements per key-block record
    size_t off_rec, off_qhat, off_mdiag, off_ldiag, off_fq, off_fk, off_fb, off_kn, off_redo, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline FwdLayout fwd_layout(int64_t B, int64_t H, int64_t L, int64_t d, int64_t es) {
    FwdLayout f;
    f.bh = B * H;
    f.nb = (L + kBlk - 1) / kBlk;
    f.lp = f.nb * kBlk;
    f.d = d;
    f.es = es;
    f.rec_elems = 2 * kBlk * d + d * d;
    size_t o = 0;
    f.off_rec = o;
    o = align256(o + (size_t)(f.bh * f.nb * f.rec_elems * es));
    f.off_qhat = o;
    o = align256(o + (size_t)(f.bh * f.lp * d * es));
    f.off_mdiag = o;
    o = align256(o + (size_t)(f.bh * f.lp * 4));
    f.off_ldiag = o;
    o = align256(o + (size_t)(f.bh * f.lp * 4));
    f.off_fq = o;
    o = align256(o + (size_t)(f.bh * f.lp * 4));
    f.off_fk = o;
    o = align256(o + (size_t)(f.bh * f.lp * 4));
    f.off_fb = o;
    o = align256(o + (size_t)(f.bh * f.nb * 4));
    f.off_kn = o;
    o = align256(o + (size_t)(f.bh * f.nb * 4));
    f.off_redo = o;
    o = align256(o + (size_t)(f.bh * (2 * f.nb + 8) * 4));
    f.total = o;
    return f;
}

}  // namespace path
