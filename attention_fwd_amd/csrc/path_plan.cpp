// path_plan.cpp -- host-side planning shared by the C ABI and the launchers:
// the decode split plan and the backward workspace layout (plain C++, no
// device code).
#include <stdint.h>

#include "path_bwd.h"
#include "path_kernels.h"

namespace path {

void decode_plan(int64_t BH, int64_t rows, int *nsplit, int64_t *chunk) {
    // about 16384 workgroups in all (on B16 H32 with 32768 rows: 4 iterations of
    // 256 rows each; 8192 and 32768 workgroups were 3-4% and 10% slower there);
    // splits are whole multiples of the rows a workgroup covers per iteration
    const int64_t target_wg = 16384;
    const int64_t step = kDecodeRowStep;
    int64_t per_head = (target_wg + BH - 1) / BH;
    const int64_t max_split = (rows + step - 1) / step;
    if (per_head > max_split) per_head = max_split;
    if (per_head < 1) per_head = 1;
    int64_t c = (rows + per_head - 1) / per_head;
    c = (c + step - 1) / step * step;
    if (c < step) c = step;
    *chunk = c;
    *nsplit = (int)((rows + c - 1) / c);
    if (*nsplit < 1) *nsplit = 1;
}

BwdLayout bwd_layout(int L, int D, int es) {
    BwdLayout ly{};
    ly.D = D;
    ly.es = es;
    const int64_t nb = (L + 63) / 64, Lp = nb * 64, np = nb * (nb - 1) / 2;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    const int64_t tok = nb * 64 * 64 * 4;          // a 64 x 64 fp32 matrix per block
    const int64_t fr = nb * 64 * D * es;           // a 64 x D fragment set per block
    const int64_t frd = nb * (int64_t)D * D * es;  // a D x D fragment set per block
    const int64_t nat = Lp * D * 4, rows = Lp * 4;
    ly.xx = take(tok); ly.aa = take(tok); ly.qwm = take(tok); ly.nn = take(tok); ly.zz = take(tok); ly.ee = take(tok);
    ly.rec_elems = 3 * 64 * (int64_t)D + (int64_t)D * D;
    ly.urec = take(nb * ly.rec_elems * es);
    // dO^T: not stored for bf16, whose key walk gathers it from dO
    ly.do1 = take(fr); ly.do2 = take(es == 2 ? 0 : fr);
    ly.nt = take(frd);
    ly.qh = take(nat); ly.dvd = take(nat); ly.dqo = take(nat); ly.dko = take(nat); ly.dvo = take(nat);
    ly.uu = take(nat); ly.vv = take(nat);
    ly.dtt = take(nb * (int64_t)D * D * 4);
    ly.dd = take(rows); ly.cql = take(rows); ly.ckl = take(rows); ly.rsd = take(rows);
    ly.csd = take(rows); ly.rso = take(rows); ly.cso = take(rows); ly.dc = take(rows);
    ly.tot = take(nb * 4); ly.mid = take(np * 4);
    const int64_t pr = np * 64 * D * es;  // a 64 x D fragment set per pair
    ly.qs1 = take(pr);
    // q~ with rows d: not stored for bf16, whose key walk gathers it from the other orientation
    ly.qs2 = take(es == 2 ? 0 : pr);
    ly.gs2 = take(pr + 64 * D * es);  // one spare set after the last pair's: target of discarded stores
    ly.head = off;
    return ly;
}

}  // namespace path
