// path_plan.cpp -- host-side planning shared by the C ABI and the launchers:
// the decode split plan and the backward workspace layout (plain C++, no
// device code).
#include <stdint.h>

#include "path_bwd.h"
#include "path_kernels.h"

namespace path {

void decode_plan(int64_t BH, int64_t rows, int *nsplit, int64_t *chunk) {
    // about 8192 workgroups in all; splits are whole multiples of the rows a
    // workgroup covers per iteration
    const int64_t target_wg = 8192;
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

BwdLayout bwd_layout(int L, int es) {
    BwdLayout ly{};
    const int64_t nb = (L + 64 - 1) / 64, Lp = nb * 64, np = nb * (nb - 1) / 2;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    const int64_t tile = Lp * 64 * 4, rows = Lp * 4;
    ly.qh = take(tile); ly.kh = take(tile); ly.vf = take(Lp * 64 * es); ly.dof = take(Lp * 64 * es);
    ly.tt = take(nb * 64 * 64 * 4);
    ly.ttt = take(nb * 64 * 64 * 4);
    ly.xx = take(nb * 64 * 64 * 4); ly.aa = take(nb * 64 * 64 * 4); ly.qwm = take(nb * 64 * 64 * 4);
    ly.nn = take(nb * 64 * 64 * 4); ly.zz = take(nb * 64 * 64 * 4);
    ly.ee = take(nb * 64 * 64 * 4); ly.dvd = take(tile); ly.dqo = take(tile); ly.dko = take(tile); ly.dvo = take(tile);
    ly.dt = take(nb * 64 * 64 * 4);
    ly.l2 = take(rows); ly.dd = take(rows); ly.clq = take(rows); ly.ckk = take(rows); ly.rsd = take(rows);
    ly.csd = take(rows); ly.rso = take(rows); ly.cso = take(rows); ly.dc = take(rows);
    ly.tot = take(nb * 4); ly.mid = take(np * 4);
    ly.qs = take(np * 64 * 64 * es); ly.gs = take(np * 64 * 64 * es);
    ly.ps = take(np * 64 * 64 * es); ly.ds = take(np * 64 * 64 * es); ly.csp = take(np * 64 * 4);
    ly.head = off;
    return ly;
}

}  // namespace path
