// path_abi.cpp -- the C ABI declared in include/path_attn.h: argument
// validation (before anything is enqueued), workspace sizing and launches.
#include "path_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "path_bwd.h"
#include "path_kernels.h"
#include "path_layout.h"

namespace {

constexpr int64_t kMaxGrid = 2147483647;  // blockIdx.x range

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t elem_size(path_dtype_t t) { return t == PATH_DTYPE_BF16 ? 2 : (t == PATH_DTYPE_F32 ? 4 : 0); }

// [p, p+n) and [q, q+m) overlap?
bool overlap(const void *p, int64_t n, const void *q, int64_t m) {
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// Checked product of positive sizes; -1 on overflow past 2^62.
int64_t mul_chk(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x < 0) return -1;
        if (x != 0 && r > (int64_t(1) << 62) / x) return -1;
        r *= x;
    }
    return r;
}

path_status_t fwd_sizes_ok(int B, int H, int L, int d, path_dtype_t dtype) {
    if (B < 1 || H < 1 || L < 1 || d < 1 || elem_size(dtype) == 0) return PATH_EINVAL;
    if (d != 64 && d != 128) return PATH_EUNSUPPORTED;
    const int64_t nb = ((int64_t)L + path::kBlk - 1) / path::kBlk;
    if (mul_chk({B, H, nb * path::kBlk, d, 8}) < 0) return PATH_EINVAL;
    if (mul_chk({B, H, nb}) > kMaxGrid) return PATH_EINVAL;
    return PATH_OK;
}

path_status_t dec_sizes_ok(int B, int H, int64_t rows, int d, path_dtype_t dtype) {
    if (B < 1 || H < 1 || rows < 1 || d < 1 || elem_size(dtype) == 0) return PATH_EINVAL;
    if (d != 64 && d != 128) return PATH_EUNSUPPORTED;
    if (mul_chk({B, H, rows, d, 8}) < 0) return PATH_EINVAL;
    return PATH_OK;
}

size_t dec_ws_bytes(int B, int H, int64_t rows, int d) {
    int nsplit;
    int64_t chunk;
    path::decode_plan((int64_t)B * H, rows, &nsplit, &chunk);
    return (size_t)B * H * nsplit * (d + 2) * sizeof(float);
}

}  // namespace

extern "C" {

int path_abi_version(void) { return PATH_ABI_VERSION; }

const char *path_status_string(path_status_t s) {
    switch (s) {
        case PATH_OK: return "ok";
        case PATH_EINVAL: return "invalid argument";
        case PATH_EUNSUPPORTED: return "unsupported configuration";
        case PATH_EHIP: return "HIP launch error";
        case PATH_ESCRATCH: return "problem larger than the fixed scratch of the no-allocation entry point";
    }
    return "unknown status";
}

size_t path_attn_fwd_workspace_size(int B, int H, int L, int d, path_dtype_t dtype) {
    if (fwd_sizes_ok(B, H, L, d, dtype) != PATH_OK) return 0;
    return path::fwd_layout(B, H, L, d, elem_size(dtype)).total;
}

namespace {

path_status_t fwd_check(const void *q, const void *k, const void *v, const void *w, const float *beta,
                        const float *logf, void *out, float *lse, int B, int H, int L, int d, path_dtype_t dtype,
                        float scale, void *workspace, size_t workspace_bytes) {
    path_status_t st = fwd_sizes_ok(B, H, L, d, dtype);
    if (st != PATH_OK) return st;
    if (!q || !k || !v || !w || !beta || !out || !workspace) return PATH_EINVAL;
    for (const void *p : {q, k, v, w, (const void *)out, (const void *)workspace})
        if (!aligned(p, 16)) return PATH_EINVAL;
    for (const void *p : {(const void *)beta, (const void *)logf, (const void *)lse})
        if (p && !aligned(p, 4)) return PATH_EINVAL;
    const size_t need = path::fwd_layout(B, H, L, d, elem_size(dtype)).total;
    if (workspace_bytes < need) return PATH_EINVAL;
    if (!(std::isfinite(scale))) return PATH_EINVAL;
    const int64_t tens = (int64_t)B * H * L * d * elem_size(dtype), tok = (int64_t)B * H * L * 4;
    for (const void *p : {q, k, v, w})
        if (overlap(out, tens, p, tens) || overlap(workspace, (int64_t)need, p, tens)) return PATH_EINVAL;
    for (const void *p : {(const void *)beta, (const void *)logf})
        if (overlap(out, tens, p, tok) || overlap(workspace, (int64_t)need, p, tok) || overlap(lse, tok, p, tok))
            return PATH_EINVAL;
    if (overlap(out, tens, workspace, (int64_t)need) || overlap(lse, tok, workspace, (int64_t)need) ||
        overlap(lse, tok, out, tens))
        return PATH_EINVAL;
    for (const void *p : {q, k, v, w})
        if (overlap(lse, tok, p, tens)) return PATH_EINVAL;
    return PATH_OK;
}

path_status_t scan_check(void *out, float *lse, int B, int H, int L, int d, path_dtype_t dtype, float scale,
                         void *workspace, size_t workspace_bytes) {
    path_status_t st = fwd_sizes_ok(B, H, L, d, dtype);
    if (st != PATH_OK) return st;
    if (!out || !workspace || !aligned(out, 16) || !aligned(workspace, 16)) return PATH_EINVAL;
    if (lse && !aligned(lse, 4)) return PATH_EINVAL;
    const size_t need = path::fwd_layout(B, H, L, d, elem_size(dtype)).total;
    if (workspace_bytes < need || !std::isfinite(scale)) return PATH_EINVAL;
    const int64_t tens = (int64_t)B * H * L * d * elem_size(dtype), tok = (int64_t)B * H * L * 4;
    if (overlap(out, tens, workspace, (int64_t)need) || overlap(lse, tok, workspace, (int64_t)need) ||
        overlap(lse, tok, out, tens))
        return PATH_EINVAL;
    return PATH_OK;
}

path_status_t launch_prep_stage(const void *q, const void *k, const void *v, const void *w, const float *beta,
                                const float *logf, void *out, float *lse, int B, int H, int L, int d,
                                path_dtype_t dtype, float scale, void *workspace, hipStream_t s,
                                const float *conv_w = nullptr, const float *zbeta = nullptr,
                                float beta_clip = 0.f) {
    path::PrepArgs pa{q, k, v, w, beta, logf, out, lse, workspace, B, H, L, d, scale, conv_w, zbeta, beta_clip};
    return path::launch_prep(pa, dtype == PATH_DTYPE_BF16, s) == hipSuccess ? PATH_OK : PATH_EHIP;
}

path_status_t launch_scan_stage(void *out, float *lse, bool fox, int B, int H, int L, int d, path_dtype_t dtype,
                                float scale, void *workspace, hipStream_t s, bool skip = false) {
    path::FwdArgs fa{out, lse, workspace, B, H, L, d, scale, fox ? 1 : 0, (fox && skip) ? 1 : 0};
    return path::launch_fwd(fa, dtype == PATH_DTYPE_BF16, s) == hipSuccess ? PATH_OK : PATH_EHIP;
}

float eff_scale(float scale, int d) { return scale <= 0.f ? 1.0f / std::sqrt((float)d) : scale; }

}  // namespace

path_status_t path_attn_fwd_ex(const void *q, const void *k, const void *v, const void *w, const float *beta,
                               const float *logf, void *out, float *lse, int B, int H, int L, int d,
                               path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                               unsigned flags, path_stream_t stream) {
    if (flags & ~PATH_FWD_SKIP_NEGLIGIBLE) return PATH_EINVAL;
    path_status_t st = fwd_check(q, k, v, w, beta, logf, out, lse, B, H, L, d, dtype, scale, workspace,
                                 workspace_bytes);
    if (st != PATH_OK) return st;
    scale = eff_scale(scale, d);
    hipStream_t s = (hipStream_t)stream;
    st = launch_prep_stage(q, k, v, w, beta, logf, out, lse, B, H, L, d, dtype, scale, workspace, s);
    if (st != PATH_OK) return st;
    return launch_scan_stage(out, lse, logf != nullptr, B, H, L, d, dtype, scale, workspace, s,
                             (flags & PATH_FWD_SKIP_NEGLIGIBLE) != 0);
}

path_status_t path_attn_fwd_fused(const void *q, const void *k, const void *v, const void *wraw,
                                  const float *conv_w, const float *zbeta, float beta_clip, const float *logf,
                                  void *out, float *lse, int B, int H, int L, int d, path_dtype_t dtype, float scale,
                                  void *workspace, size_t workspace_bytes, path_stream_t stream) {
    path_status_t st = fwd_check(q, k, v, wraw, zbeta, logf, out, lse, B, H, L, d, dtype, scale, workspace,
                                 workspace_bytes);
    if (st != PATH_OK) return st;
    if (!conv_w || !aligned(conv_w, 16) || !std::isfinite(beta_clip) || beta_clip < 0.f) return PATH_EINVAL;
    const int64_t cwb = (int64_t)H * d * 3 * 4, tens = (int64_t)B * H * L * d * elem_size(dtype);
    const int64_t tok = (int64_t)B * H * L * 4;
    const size_t need = path::fwd_layout(B, H, L, d, elem_size(dtype)).total;
    if (overlap(out, tens, conv_w, cwb) || overlap(workspace, (int64_t)need, conv_w, cwb) ||
        overlap(lse, tok, conv_w, cwb))
        return PATH_EINVAL;
    scale = eff_scale(scale, d);
    hipStream_t s = (hipStream_t)stream;
    st = launch_prep_stage(q, k, v, wraw, nullptr, logf, out, lse, B, H, L, d, dtype, scale, workspace, s, conv_w,
                           zbeta, beta_clip);
    if (st != PATH_OK) return st;
    return launch_scan_stage(out, lse, logf != nullptr, B, H, L, d, dtype, scale, workspace, s);
}

path_status_t path_attn_fwd(const void *q, const void *k, const void *v, const void *w, const float *beta,
                            const float *logf, void *out, float *lse, int B, int H, int L, int d,
                            path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                            path_stream_t stream) {
    return path_attn_fwd_ex(q, k, v, w, beta, logf, out, lse, B, H, L, d, dtype, scale, workspace, workspace_bytes,
                            0u, stream);
}

path_status_t path_attn_fwd_prep(const void *q, const void *k, const void *v, const void *w, const float *beta,
                                 const float *logf, void *out, float *lse, int B, int H, int L, int d,
                                 path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                 path_stream_t stream) {
    path_status_t st = fwd_check(q, k, v, w, beta, logf, out, lse, B, H, L, d, dtype, scale, workspace,
                                 workspace_bytes);
    if (st != PATH_OK) return st;
    return launch_prep_stage(q, k, v, w, beta, logf, out, lse, B, H, L, d, dtype, eff_scale(scale, d), workspace,
                             (hipStream_t)stream);
}

path_status_t path_attn_fwd_scan(void *out, float *lse, int has_logf, int B, int H, int L, int d,
                                 path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                 path_stream_t stream) {
    path_status_t st = scan_check(out, lse, B, H, L, d, dtype, scale, workspace, workspace_bytes);
    if (st != PATH_OK) return st;
    return launch_scan_stage(out, lse, has_logf != 0, B, H, L, d, dtype, eff_scale(scale, d), workspace,
                             (hipStream_t)stream);
}

size_t path_decode_workspace_size(int B, int H, int64_t n, int d, path_dtype_t dtype) {
    if (dec_sizes_ok(B, H, n, d, dtype) != PATH_OK) return 0;
    return dec_ws_bytes(B, H, n, d);
}

}  // extern "C"

namespace {

// Workspace of the fused decode step: the decode partials, then the step's w (element
// type, [B, H, d]) and beta (fp32, [B, H]) made by the producer.
struct FusedDecWs {
    int64_t w_off, b_off, total;
};
FusedDecWs fused_dec_ws(int B, int H, int64_t rows, int d, int64_t es) {
    const int64_t a = ((int64_t)dec_ws_bytes(B, H, rows, d) + 255) / 256 * 256;
    const int64_t b = (a + (int64_t)B * H * d * es + 255) / 256 * 256;
    return {a, b, b + (int64_t)B * H * 4};
}

}  // namespace

extern "C" {

size_t path_decode_fused_workspace_size(int B, int H, int64_t n, int d, path_dtype_t dtype) {
    if (dec_sizes_ok(B, H, n, d, dtype) != PATH_OK) return 0;
    return (size_t)fused_dec_ws(B, H, n, d, elem_size(dtype)).total;
}

}  // extern "C"

namespace {

// Argument checks shared by the decode entry points (nothing is enqueued).  With
// own_scratch the kernels use the library's fixed scratch array instead of a
// caller workspace: `workspace` is then NULL and the scratch must hold `need`.
path_status_t dec_check(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q, const void *w,
                        const float *beta, const float *logf, float *fcache, const void *k_new, const void *v_new,
                        void *out, float *lse, int B, int H, int d, path_dtype_t dtype, float scale,
                        const void *workspace, size_t workspace_bytes, bool own_scratch, int64_t *natt_out) {
    if (n < 0 || ncap < 1 || n > ncap) return PATH_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr)) return PATH_EINVAL;
    if ((logf == nullptr) != (fcache == nullptr)) return PATH_EINVAL;
    const int64_t natt = n + (k_new ? 1 : 0);
    if (natt > ncap) return PATH_EINVAL;
    path_status_t st = dec_sizes_ok(B, H, natt, d, dtype);
    if (st != PATH_OK) return st;
    if (mul_chk({B, H, ncap, d, 8}) < 0) return PATH_EINVAL;
    if (!kcache || !vcache || !q || !w || !beta || !out) return PATH_EINVAL;
    if (!own_scratch && !workspace) return PATH_EINVAL;
    for (const void *p : {(const void *)kcache, (const void *)vcache, q, w, k_new, v_new, (const void *)out,
                          workspace})
        if (p && !aligned(p, 16)) return PATH_EINVAL;
    if (!aligned(beta, 4) || (lse && !aligned(lse, 4))) return PATH_EINVAL;
    if (logf && (!aligned(logf, 4) || !aligned(fcache, 4))) return PATH_EINVAL;
    const size_t need = dec_ws_bytes(B, H, natt, d);
    if (!own_scratch && workspace_bytes < need) return PATH_EINVAL;
    if (!(std::isfinite(scale))) return PATH_EINVAL;
    {
        int nsplit;
        int64_t chunk;
        path::decode_plan((int64_t)B * H, natt, &nsplit, &chunk);
        if ((int64_t)nsplit * B * H > kMaxGrid) return PATH_EINVAL;
    }
    const int64_t es = elem_size(dtype);
    const int64_t cache = (int64_t)B * H * ncap * d * es, vec = (int64_t)B * H * d * es, sc = (int64_t)B * H * 4;
    if (overlap(kcache, cache, vcache, cache)) return PATH_EINVAL;
    for (const void *p : {q, w, k_new, v_new, (const void *)out, workspace}) {
        const int64_t sz = p == workspace ? (int64_t)need : vec;
        if (overlap(kcache, cache, p, sz) || overlap(vcache, cache, p, sz)) return PATH_EINVAL;
    }
    for (const void *p : {q, w, k_new, v_new, workspace})
        if (overlap(out, vec, p, p == workspace ? (int64_t)need : vec)) return PATH_EINVAL;
    if (lse && (overlap(lse, sc, beta, sc) || overlap(lse, sc, out, vec) || overlap(lse, sc, workspace, (int64_t)need) ||
                overlap(lse, sc, kcache, cache) || overlap(lse, sc, vcache, cache)))
        return PATH_EINVAL;
    if (fcache) {
        const int64_t fcs = (int64_t)B * H * ncap * 4;
        for (const void *p : {(const void *)kcache, (const void *)vcache})
            if (overlap(fcache, fcs, p, cache)) return PATH_EINVAL;
        for (const void *p : {q, w, k_new, v_new, (const void *)out, workspace})
            if (overlap(fcache, fcs, p, p == workspace ? (int64_t)need : vec)) return PATH_EINVAL;
        for (const void *p : {(const void *)beta, (const void *)logf, (const void *)lse})
            if (overlap(fcache, fcs, p, sc)) return PATH_EINVAL;
    }
    if (own_scratch && need > path::decode_scratch_bytes()) return PATH_ESCRATCH;
    *natt_out = natt;
    return PATH_OK;
}

path_status_t dec_launch(void *kcache, void *vcache, int64_t n, int64_t ncap, int64_t natt, const void *q,
                         const void *w, const float *beta, const float *logf, float *fcache, const void *k_new,
                         const void *v_new, void *out, float *lse, int B, int H, int d, path_dtype_t dtype, float scale,
                         void *workspace, path_stream_t stream) {
    path::DecodeArgs da{};
    da.kc = kcache; da.vc = vcache; da.n = n; da.ncap = ncap;
    da.q = q; da.w = w; da.beta = beta; da.logf = logf; da.fcache = fcache; da.knew = k_new; da.vnew = v_new;
    da.out = out; da.lse = lse; da.ws = workspace;
    da.B = B; da.H = H; da.d = d; da.scale = eff_scale(scale, d);
    path::decode_plan((int64_t)B * H, natt, &da.nsplit, &da.chunk);
    if (path::launch_decode(da, dtype == PATH_DTYPE_BF16, (hipStream_t)stream) != hipSuccess) return PATH_EHIP;
    return PATH_OK;
}

}  // namespace

extern "C" {

path_status_t path_decode_step_ex(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q, const void *w,
                                  const float *beta, const float *logf, float *fcache, const void *k_new,
                                  const void *v_new, void *out, float *lse, int B, int H, int d, path_dtype_t dtype,
                                  float scale, void *workspace, size_t workspace_bytes, path_stream_t stream) {
    int64_t natt = 0;
    path_status_t st = dec_check(kcache, vcache, n, ncap, q, w, beta, logf, fcache, k_new, v_new, out, lse, B, H, d,
                                 dtype, scale, workspace, workspace_bytes, false, &natt);
    if (st != PATH_OK) return st;
    return dec_launch(kcache, vcache, n, ncap, natt, q, w, beta, logf, fcache, k_new, v_new, out, lse, B, H, d, dtype,
                      scale, workspace, stream);
}

size_t path_decode_noalloc_max_bytes(void) { return path::decode_scratch_bytes(); }

path_status_t path_decode_step_noalloc(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q,
                                       const void *w, const float *beta, const float *logf, float *fcache,
                                       const void *k_new, const void *v_new, void *out, float *lse, int B, int H,
                                       int d, path_dtype_t dtype, float scale, path_stream_t stream) {
    int64_t natt = 0;
    path_status_t st = dec_check(kcache, vcache, n, ncap, q, w, beta, logf, fcache, k_new, v_new, out, lse, B, H, d,
                                 dtype, scale, nullptr, 0, true, &natt);
    if (st != PATH_OK) return st;
    void *scratch = nullptr;  // this device's copy of the library's scratch array
    if (path::decode_scratch(&scratch) != hipSuccess) return PATH_EHIP;
    return dec_launch(kcache, vcache, n, ncap, natt, q, w, beta, logf, fcache, k_new, v_new, out, lse, B, H, d, dtype,
                      scale, scratch, stream);
}

path_status_t path_decode_step(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q, const void *w,
                               const float *beta, const void *k_new, const void *v_new, void *out, float *lse, int B,
                               int H, int d, path_dtype_t dtype, float scale, void *workspace,
                               size_t workspace_bytes, path_stream_t stream) {
    return path_decode_step_ex(kcache, vcache, n, ncap, q, w, beta, nullptr, nullptr, k_new, v_new, out, lse, B, H, d,
                               dtype, scale, workspace, workspace_bytes, stream);
}

path_status_t path_decode_step_fused(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q,
                                     const void *wraw, const float *conv_w, const float *zbeta, float beta_clip,
                                     void *conv_state, const float *logf, float *fcache, const void *k_new,
                                     const void *v_new, void *out, float *lse, int B, int H, int d,
                                     path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                     path_stream_t stream) {
    if (!workspace || !wraw || !conv_w || !zbeta || !conv_state) return PATH_EINVAL;
    if (!std::isfinite(beta_clip) || beta_clip < 0.f) return PATH_EINVAL;
    if (n < 0 || n > ncap) return PATH_EINVAL;
    const int64_t rows = n + (k_new ? 1 : 0);
    path_status_t st = dec_sizes_ok(B, H, rows, d, dtype);
    if (st != PATH_OK) return st;
    const int64_t es = elem_size(dtype);
    const FusedDecWs fw = fused_dec_ws(B, H, rows, d, es);
    if ((int64_t)workspace_bytes < fw.total || !aligned(workspace, 16)) return PATH_EINVAL;
    void *wp = (char *)workspace + fw.w_off;
    float *bp = (float *)((char *)workspace + fw.b_off);
    // the decode step's own checks, with the produced w and beta in the workspace after its partials
    int64_t natt = 0;
    st = dec_check(kcache, vcache, n, ncap, q, wp, bp, logf, fcache, k_new, v_new, out, lse, B, H, d, dtype, scale,
                   workspace, (size_t)fw.w_off, false, &natt);
    if (st != PATH_OK) return st;
    // the producer's inputs and its state
    if (!aligned(wraw, 16) || !aligned(conv_state, 16) || !aligned(conv_w, 16) || !aligned(zbeta, 4))
        return PATH_EINVAL;
    const int64_t vec = (int64_t)B * H * d * es, sc = (int64_t)B * H * 4, stb = 2 * vec, cwb = (int64_t)H * d * 3 * 4;
    const int64_t cache = (int64_t)B * H * ncap * d * es, fcs = (int64_t)B * H * ncap * 4;
    const struct {
        const void *p;
        int64_t n;
    } others[] = {{kcache, cache}, {vcache, cache}, {q, vec},      {wraw, vec},    {conv_w, cwb},
                  {zbeta, sc},     {logf, sc},      {fcache, fcs}, {k_new, vec},   {v_new, vec},
                  {out, vec},      {lse, sc},       {workspace, fw.total}};
    for (const auto &o : others)  // the state is read and written: it shares memory with nothing
        if (overlap(conv_state, stb, o.p, o.n)) return PATH_EINVAL;
    const struct {
        const void *p;
        int64_t n;
    } written[] = {{kcache, cache}, {vcache, cache}, {out, vec}, {lse, sc}, {fcache, fcs}, {workspace, fw.total}};
    for (const auto &o : written)
        if (overlap(o.p, o.n, wraw, vec) || overlap(o.p, o.n, conv_w, cwb) || overlap(o.p, o.n, zbeta, sc))
            return PATH_EINVAL;
    path::ProduceArgs pa{};
    pa.wraw = wraw; pa.conv_w = conv_w; pa.zbeta = zbeta; pa.beta_clip = beta_clip; pa.state = conv_state;
    pa.w_out = wp; pa.beta_out = bp; pa.B = B; pa.H = H; pa.d = d;
    if (path::launch_decode_produce(pa, dtype == PATH_DTYPE_BF16, (hipStream_t)stream) != hipSuccess)
        return PATH_EHIP;
    return dec_launch(kcache, vcache, n, ncap, natt, q, wp, bp, logf, fcache, k_new, v_new, out, lse, B, H, d, dtype,
                      scale, workspace, stream);
}

path_status_t path_decode_cache_from_fwd(const void *workspace, size_t workspace_bytes, const void *v,
                                         const float *logf, void *kcache, void *vcache, float *fcache,
                                         int64_t ncap, int B, int H, int L, int d, path_dtype_t dtype,
                                         path_stream_t stream) {
    path_status_t st = fwd_sizes_ok(B, H, L, d, dtype);
    if (st != PATH_OK) return st;
    if (ncap < L || mul_chk({B, H, ncap, d, 8}) < 0) return PATH_EINVAL;
    if (!workspace || !v || !kcache || !vcache) return PATH_EINVAL;
    if ((logf == nullptr) != (fcache == nullptr)) return PATH_EINVAL;
    if (logf && (!aligned(logf, 4) || !aligned(fcache, 4))) return PATH_EINVAL;
    for (const void *p : {workspace, v, (const void *)kcache, (const void *)vcache})
        if (!aligned(p, 16)) return PATH_EINVAL;
    const size_t need = path::fwd_layout(B, H, L, d, elem_size(dtype)).total;
    if (workspace_bytes < need) return PATH_EINVAL;
    const int64_t es = elem_size(dtype);
    const int64_t cache = (int64_t)B * H * ncap * d * es, tens = (int64_t)B * H * L * d * es;
    if (overlap(kcache, cache, vcache, cache)) return PATH_EINVAL;
    for (const void *p : {(const void *)kcache, (const void *)vcache})
        if (overlap(p, cache, workspace, (int64_t)need) || overlap(p, cache, v, tens)) return PATH_EINVAL;
    if (fcache) {
        const int64_t fcs = (int64_t)B * H * ncap * 4, lfs = (int64_t)B * H * L * 4;
        for (const void *p : {(const void *)kcache, (const void *)vcache})
            if (overlap(fcache, fcs, p, cache)) return PATH_EINVAL;
        if (overlap(fcache, fcs, workspace, (int64_t)need) || overlap(fcache, fcs, v, tens) ||
            overlap(fcache, fcs, logf, lfs))
            return PATH_EINVAL;
    }
    path::CacheArgs ca{workspace, v, logf, fcache, kcache, vcache, ncap, B, H, L, d};
    if ((int64_t)B * H > kMaxGrid) return PATH_EINVAL;
    return path::launch_cache(ca, dtype == PATH_DTYPE_BF16, (hipStream_t)stream) == hipSuccess ? PATH_OK : PATH_EHIP;
}

namespace {

// default workspace: all heads, or what fits in 32 GiB (an eighth of the device's 288 GB; fewer,
// larger passes over the heads leave fewer kernel tails)
constexpr int64_t kBwdCap = int64_t(32) << 30;

path_status_t bwd_sizes_ok(int B, int H, int L, int d, path_dtype_t dtype) {
    if (B < 1 || H < 1 || L < 1 || d < 1 || elem_size(dtype) == 0) return PATH_EINVAL;
    if (d != 64 && d != 128) return PATH_EUNSUPPORTED;
    const int64_t nb = ((int64_t)L + 63) / 64;
    if (mul_chk({B, H, nb * 64, d, 8}) < 0 || mul_chk({nb, nb, 64, d, 8}) < 0) return PATH_EINVAL;
    if (nb > 65535 || mul_chk({B, H, nb}) > kMaxGrid) return PATH_EINVAL;
    return PATH_OK;
}

}  // namespace

size_t path_attn_bwd_workspace_size(int B, int H, int L, int d, path_dtype_t dtype) {
    if (bwd_sizes_ok(B, H, L, d, dtype) != PATH_OK) return 0;
    const int64_t share = path::bwd_layout(L, d, (int)elem_size(dtype)).head, G = (int64_t)B * H;
    int64_t hc = kBwdCap / share;
    if (hc < 1) hc = 1;
    if (hc > G) hc = G;
    return (size_t)(hc * share);
}

path_status_t path_attn_bwd(const void *q, const void *k, const void *v, const void *w, const float *beta,
                            const float *logf, const void *out, const float *lse, const void *dout,
                            const float *dlse, void *dq, void *dk, void *dv, void *dw, float *dbeta, float *dlogf,
                            int B, int H, int L, int d, path_dtype_t dtype, float scale, void *workspace,
                            size_t workspace_bytes, path_stream_t stream) {
    path_status_t st = bwd_sizes_ok(B, H, L, d, dtype);
    if (st != PATH_OK) return st;
    if (!q || !k || !v || !w || !beta || !out || !lse || !dout || !dq || !dk || !dv || !dw || !dbeta || !workspace)
        return PATH_EINVAL;
    if ((logf == nullptr) != (dlogf == nullptr)) return PATH_EINVAL;
    const void *tens_in[] = {q, k, v, w, out, dout};
    void *tens_out[] = {dq, dk, dv, dw};
    const void *tok_in[] = {beta, logf, lse, dlse};
    void *tok_out[] = {dbeta, dlogf};
    for (const void *p : tens_in)
        if (!aligned(p, 16)) return PATH_EINVAL;
    for (const void *p : tens_out)
        if (!aligned(p, 16)) return PATH_EINVAL;
    if (!aligned(workspace, 16)) return PATH_EINVAL;
    for (const void *p : tok_in)
        if (p && !aligned(p, 4)) return PATH_EINVAL;
    for (const void *p : tok_out)
        if (p && !aligned(p, 4)) return PATH_EINVAL;
    if (!std::isfinite(scale)) return PATH_EINVAL;
    const int64_t share = path::bwd_layout(L, d, (int)elem_size(dtype)).head, G = (int64_t)B * H;
    if ((int64_t)workspace_bytes < share) return PATH_EINVAL;
    int64_t hc = (int64_t)workspace_bytes / share;
    if (hc > G) hc = G;
    if (hc > 65535) hc = 65535;
    const int64_t wsb = hc * share;
    const int64_t tens = (int64_t)B * H * L * d * elem_size(dtype), tok = (int64_t)B * H * L * 4;
    // every output against every other buffer
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(tens_out[i], tens, tens_out[j], tens)) return PATH_EINVAL;
        for (const void *p : tens_in)
            if (overlap(tens_out[i], tens, p, tens)) return PATH_EINVAL;
        for (const void *p : tok_in)
            if (overlap(tens_out[i], tens, p, tok)) return PATH_EINVAL;
        for (void *p : tok_out)
            if (overlap(tens_out[i], tens, p, tok)) return PATH_EINVAL;
        if (overlap(tens_out[i], tens, workspace, wsb)) return PATH_EINVAL;
    }
    for (int i = 0; i < 2; ++i) {
        if (!tok_out[i]) continue;
        if (i == 0 && overlap(dbeta, tok, dlogf, tok)) return PATH_EINVAL;
        for (const void *p : tens_in)
            if (overlap(tok_out[i], tok, p, tens)) return PATH_EINVAL;
        for (const void *p : tok_in)
            if (overlap(tok_out[i], tok, p, tok)) return PATH_EINVAL;
        if (overlap(tok_out[i], tok, workspace, wsb)) return PATH_EINVAL;
    }
    for (const void *p : tens_in)
        if (overlap(workspace, wsb, p, tens)) return PATH_EINVAL;
    for (const void *p : tok_in)
        if (overlap(workspace, wsb, p, tok)) return PATH_EINVAL;

    path::BwdArgs ba{};
    ba.q = q; ba.k = k; ba.v = v; ba.w = w; ba.beta = beta; ba.logf = logf; ba.out = out; ba.lse = lse;
    ba.dout = dout; ba.dlse = dlse; ba.dq = dq; ba.dk = dk; ba.dv = dv; ba.dw = dw; ba.dbeta = dbeta;
    ba.dlogf = dlogf; ba.ws = workspace;
    ba.B = B; ba.H = H; ba.L = L; ba.d = d; ba.scale = eff_scale(scale, d);
    ba.nb = (L + 63) / 64;
    ba.hc_max = (int)hc;
    ba.ly = path::bwd_layout(L, d, (int)elem_size(dtype));
    return path::launch_bwd(ba, dtype == PATH_DTYPE_BF16, (hipStream_t)stream) == hipSuccess ? PATH_OK : PATH_EHIP;
}

}  // extern "C"
