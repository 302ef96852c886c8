// path_decode.hip -- PaTH decode step: in-place rank-1 key-cache update fused
// with single-query attention.
//
// Source: "技術要約: PaTH Attention" (gist.science), section 3 (inference):
// the historical keys are updated in place with the newest transition matrix
// H_t = I - beta_t w_t w_t^T, so no cache of w / beta is kept, and decoding
// then proceeds like ordinary softmax decoding over the (updated) cache.
//
// Per cached row j (one pass over HBM: read k_j, write k_j', read v_j):
//   a_j   = w . k_j,  b_j = q . k_j            (one 8-lane reduction for both)
//   k_j'  = k_j - beta a_j w                   (stored back, rounded to the cache type)
//   s_j   = scale * q . k_j' = scale * (b_j - beta a_j (q . w))
//           (+ c_t - c_j with the forget gate: c_j = sum_{s<=j} log f_s is kept
//            per cached row, c_t = c_{n-1} + log f_t; "거리에서 경로로, PaTH
//            Attention", section 4, PaTH-FoX)
// followed by an online softmax over the rows of a split.  Eight lanes share
// a row (8 elements = 16 bytes of bf16 each), a wave covers 8 rows per load,
// and every lane keeps the rows of two iterations in flight (the next rows are
// loaded before the current ones are processed).  The cache is streamed once,
// so its loads and stores carry the non-temporal hint (5% faster here).  Splits of the cache write partial
// (max, sum, accumulator) records that a second small kernel merges in a fixed
// order, so results are bitwise reproducible.
#include <mutex>

#include "path_common.h"
#include "path_kernels.h"

namespace path {

// Scratch of the no-allocation decode entry point: the split partials (max, sum,
// d accumulators per head and split) live in this fixed array instead of a
// caller workspace.  Each device holds its own copy from module load to the end
// of the process.  Host code must not use the name itself (on the host it is
// only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device in decode_scratch().
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current: its copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

constexpr int kDecThreads = 256;
constexpr int kCombThreads = 256;  // threads of the merge kernel (a multiple of D)
// rows each lane group keeps in flight per iteration (fewer for the wider head
// and for fp32 rows, so that the raw rows of two iterations, 128 VGPRs, fit):
// for bf16, half as many rows were 5% (d = 64) and 12% (d = 128) slower on
// B16 H32 n32768, twice as many no faster
template <typename S, int D>
constexpr int rows_per_iter() { return (D == 64 ? 8 : 4) / (int)(sizeof(S) / 2); }

template <typename S>
__device__ __forceinline__ void load8(const S *p, float *x) {  // 8 consecutive elements as fp32
    if constexpr (sizeof(S) == 2) {
        u32x4 u = *(const u32x4 *)p;
        x[0] = bf16_to_f32(u.x & 0xffff); x[1] = bf16_to_f32(u.x >> 16);
        x[2] = bf16_to_f32(u.y & 0xffff); x[3] = bf16_to_f32(u.y >> 16);
        x[4] = bf16_to_f32(u.z & 0xffff); x[5] = bf16_to_f32(u.z >> 16);
        x[6] = bf16_to_f32(u.w & 0xffff); x[7] = bf16_to_f32(u.w >> 16);
    } else {
        f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <typename S>
__device__ __forceinline__ void store8(S *p, const float *x) {
    if constexpr (sizeof(S) == 2) {
        u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
        __builtin_nontemporal_store(u, (u32x4 *)p);
    } else {
        f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
        __builtin_nontemporal_store(a, (f32x4 *)p);
        __builtin_nontemporal_store(b, (f32x4 *)(p + 4));
    }
}

template <typename S, int N>
__device__ __forceinline__ void loadn(const S *p, float *x) {  // N (multiple of 8) consecutive elements
#pragma unroll
    for (int c = 0; c < N; c += 8) load8<S>(p + c, x + c);
}
template <typename S, int N>
__device__ __forceinline__ void storen(S *p, const float *x) {
#pragma unroll
    for (int c = 0; c < N; c += 8) store8<S>(p + c, x + c);
}

template <typename S, int D>
__global__ __launch_bounds__(kDecThreads) void path_decode_kernel(DecodeArgs a) {
    static_assert(D == 64 || D == 128, "decode kernel: head dimension 64 or 128");
    constexpr int EPL = D / 8;           // elements per lane: 8 lanes share a row
    constexpr int kRowsPerIter = rows_per_iter<S, D>();
    constexpr int NG = kDecThreads / 8;  // lane groups (rows in flight per load) per workgroup
    __shared__ float sred[NG][D + 2];

    const int split = (int)(blockIdx.x % a.nsplit);
    const int64_t bh = blockIdx.x / a.nsplit;
    const int tid = threadIdx.x, grp = tid >> 3, sub = tid & 7;
    const int64_t natt = a.n + (a.knew ? 1 : 0);
    const int64_t r0 = (int64_t)split * a.chunk;
    const int64_t r1 = min(natt, r0 + a.chunk);

    S *kc = (S *)a.kc + bh * a.ncap * D;
    S *vc = (S *)a.vc + bh * a.ncap * D;
    float q[EPL], w[EPL];
    loadn<S, EPL>((const S *)a.q + bh * D + EPL * sub, q);
    loadn<S, EPL>((const S *)a.w + bh * D + EPL * sub, w);
    const float beta = a.beta[bh];
    float qw = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qw += q[e] * w[e];
    qw = sum8(qw);
    const float c2 = a.scale * kLog2e;
    const bool gate = a.logf != nullptr;
    float *fcr = gate ? a.fcache + bh * a.ncap : nullptr;
    const float ct = gate ? (a.n > 0 ? fcr[a.n - 1] : 0.f) + a.logf[bh] : 0.f;

    float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    // Rows are kept in the cache type (raw 16-byte words) until used, and the rows of the
    // next iteration are loaded before the current ones are processed, so every lane keeps
    // 2 kRowsPerIter rows of K and V in flight.
    constexpr int RW = EPL * (int)sizeof(S) / 16;  // 16-byte words per lane per row
    typedef u32x4 Raw[RW];
    const int64_t stride = (int64_t)NG * kRowsPerIter;
    auto fetch = [&](int64_t base, Raw *kr, Raw *vr, float *fr) {
#pragma unroll
        for (int u = 0; u < kRowsPerIter; ++u) {
            const int64_t j = base + (int64_t)u * NG;
            const bool ok = j < r1, fresh = ok && j == a.n;
            // rows past the split read row r0 (in bounds), the appended token reads k_new / v_new
            const S *ks = fresh ? (const S *)a.knew + bh * D : kc + (ok ? j : r0 < a.n ? r0 : 0) * D;
            const S *vs = fresh ? (const S *)a.vnew + bh * D : vc + (ok ? j : r0 < a.n ? r0 : 0) * D;
#pragma unroll
            for (int c = 0; c < RW; ++c) {
                kr[u][c] = __builtin_nontemporal_load((const u32x4 *)(ks + EPL * sub + c * (16 / (int)sizeof(S))));
                vr[u][c] = __builtin_nontemporal_load((const u32x4 *)(vs + EPL * sub + c * (16 / (int)sizeof(S))));
            }
            if (gate) fr[u] = fcr[ok && !fresh ? j : 0];  // the row's gate prefix sum c_j
        }
    };
    auto widen = [&](const Raw &r, float *x) {
#pragma unroll
        for (int c = 0; c < RW; ++c) {
            if constexpr (sizeof(S) == 2) {
                const u32x4 u = r[c];
                x[8 * c + 0] = bf16_to_f32(u.x & 0xffff); x[8 * c + 1] = bf16_to_f32(u.x >> 16);
                x[8 * c + 2] = bf16_to_f32(u.y & 0xffff); x[8 * c + 3] = bf16_to_f32(u.y >> 16);
                x[8 * c + 4] = bf16_to_f32(u.z & 0xffff); x[8 * c + 5] = bf16_to_f32(u.z >> 16);
                x[8 * c + 6] = bf16_to_f32(u.w & 0xffff); x[8 * c + 7] = bf16_to_f32(u.w >> 16);
            } else {
                const f32x4 f = __builtin_bit_cast(f32x4, r[c]);
                x[4 * c + 0] = f.x; x[4 * c + 1] = f.y; x[4 * c + 2] = f.z; x[4 * c + 3] = f.w;
            }
        }
    };
    // one iteration: prefetch the rows at base + stride into (kn, vn), process (kc_, vc_)
    auto step = [&](int64_t base, Raw *kcur, Raw *vcur, float *fcur, Raw *knext, Raw *vnext, float *fnext) {
        if (base + stride < r1) fetch(base + stride, knext, vnext, fnext);
        float x[kRowsPerIter];
#pragma unroll
        for (int u = 0; u < kRowsPerIter; ++u) {
            const int64_t j = base + (int64_t)u * NG;
            const bool ok = j < r1, fresh = ok && j == a.n;  // fresh: the appended token
            float kx[EPL];
            widen(kcur[u], kx);
            float pa = 0.f, pb = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                pa += w[e] * kx[e];
                pb += q[e] * kx[e];
            }
            const float ta = sum8(pa), tb = sum8(pb);
            if (fresh) {
                // new key enters untransformed; store k_new, v_new at row n
                float vx[EPL];
                widen(vcur[u], vx);
                storen<S, EPL>(kc + j * D + EPL * sub, kx);
                storen<S, EPL>(vc + j * D + EPL * sub, vx);
                if (gate && sub == 0) fcr[j] = ct;
                x[u] = tb * c2;
            } else if (ok) {
                const float cb = beta * ta;
                float kn[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) kn[e] = kx[e] - cb * w[e];
                storen<S, EPL>(kc + j * D + EPL * sub, kn);
                x[u] = (tb - cb * qw) * c2 + (gate ? (ct - fcur[u]) * kLog2e : 0.f);
            } else {
                x[u] = -INFINITY;
            }
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < kRowsPerIter; ++u) mx = fmaxf(mx, x[u]);
        if (mx != -INFINITY) {
            const float alpha = fast_exp2(m - mx);
            l *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
            for (int u = 0; u < kRowsPerIter; ++u) {
                const float p = fast_exp2(x[u] - mx);
                l += p;
                float vx[EPL];
                widen(vcur[u], vx);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] += p * vx[e];
            }
            m = mx;
        }
    };
    Raw ka[kRowsPerIter], va[kRowsPerIter], kb[kRowsPerIter], vb[kRowsPerIter];
    float fa[kRowsPerIter], fb[kRowsPerIter];
    if (r0 + grp < r1) fetch(r0 + grp, ka, va, fa);
    for (int64_t base = r0 + grp; base < r1; base += 2 * stride) {
        step(base, ka, va, fa, kb, vb, fb);
        if (base + stride >= r1) break;
        step(base + stride, kb, vb, fb, ka, va, fa);
    }

    // merge the lane groups of the workgroup in a fixed order
#pragma unroll
    for (int e = 0; e < EPL; ++e) sred[grp][EPL * sub + e] = acc[e];
    if (sub == 0) {
        sred[grp][D] = m;
        sred[grp][D + 1] = l;
    }
    __syncthreads();
    if (tid < D) {
        float mm = -INFINITY;
        for (int g = 0; g < NG; ++g) mm = fmaxf(mm, sred[g][D]);
        float ls = 0.f, as = 0.f;
        for (int g = 0; g < NG; ++g) {
            const float mg = sred[g][D];
            const float wgt = mg == -INFINITY ? 0.f : fast_exp2(mg - mm);
            ls += wgt * sred[g][D + 1];
            as += wgt * sred[g][tid];
        }
        float *part = (float *)a.ws + ((int64_t)bh * a.nsplit + split) * (D + 2);
        part[tid] = as;
        if (tid == 0) {
            part[D] = mm;
            part[D + 1] = ls;
        }
    }
}

// Merge of the split partials of one (batch, head): the maximum over the
// splits, then the weighted sums, both spread over the workgroup (thread group
// g of D threads sums splits g, g + NG, ...; the NG group sums are then added
// in order), so the merge stays short when a head has many splits and its
// result does not depend on timing.
template <typename S, int D>
__global__ __launch_bounds__(kCombThreads) void path_decode_combine_kernel(DecodeArgs a) {
    constexpr int NG = kCombThreads / D;
    __shared__ float smax[kCombThreads];
    __shared__ float ssum[NG][D + 1];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x, g = tid / D, c = tid % D;
    const float *part = (const float *)a.ws + (int64_t)bh * a.nsplit * (D + 2);
    float mm = -INFINITY;
    for (int s = tid; s < a.nsplit; s += kCombThreads) mm = fmaxf(mm, part[(int64_t)s * (D + 2) + D]);
    smax[tid] = mm;
    __syncthreads();
#pragma unroll
    for (int o = kCombThreads / 2; o > 0; o >>= 1) {
        if (tid < o) smax[tid] = fmaxf(smax[tid], smax[tid + o]);
        __syncthreads();
    }
    mm = smax[0];
    float ls = 0.f, as = 0.f;
#pragma unroll 4
    for (int s = g; s < a.nsplit; s += NG) {
        const float *p = part + (int64_t)s * (D + 2);
        const float pm = p[D];
        const float wgt = pm == -INFINITY ? 0.f : fast_exp2(pm - mm);
        ls += wgt * p[D + 1];
        as += wgt * p[c];
    }
    ssum[g][c] = as;
    if (c == 0) ssum[g][D] = ls;
    __syncthreads();
    if (tid < D) {
        float at = 0.f, lt = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) {
            at += ssum[g2][tid];
            lt += ssum[g2][D];
        }
        ((S *)a.out)[bh * D + tid] = Elem<S>::from_float(at / lt);
        if (tid == 0 && a.lse) a.lse[bh] = (mm + __log2f(lt)) * kLn2;
    }
}

}  // namespace

// the split plan (decode_plan, host code) sizes splits in multiples of the rows one
// workgroup iteration covers; it assumes this value
static_assert(kDecodeRowStep == (kDecThreads / 8) * rows_per_iter<uint16_t, 64>(), "decode row step");
static_assert(kDecodeRowStep % ((kDecThreads / 8) * rows_per_iter<uint16_t, 128>()) == 0, "decode row step");
static_assert(kDecodeRowStep % ((kDecThreads / 8) * rows_per_iter<float, 64>()) == 0, "decode row step");
static_assert(kDecodeRowStep % ((kDecThreads / 8) * rows_per_iter<float, 128>()) == 0, "decode row step");

template <typename S, int D>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st) {
    dim3 grid((unsigned)(a.nsplit * a.B * a.H));
    hipLaunchKernelGGL((path_decode_kernel<S, D>), grid, dim3(kDecThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((path_decode_combine_kernel<S, D>), dim3((unsigned)(a.B * a.H)), dim3(kCombThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t st) {
    if (a.d == 64) return bf16 ? launch_decode_t<uint16_t, 64>(a, st) : launch_decode_t<float, 64>(a, st);
    if (a.d == 128) return bf16 ? launch_decode_t<uint16_t, 128>(a, st) : launch_decode_t<float, 128>(a, st);
    return hipErrorInvalidValue;
}

// The producer of w and beta for one decode step ("거리에서 경로로, PaTH Attention",
// section 3: a short convolution of width 3 and an L2 normalisation; "技術要約: PaTH
// Attention", section 2: beta = 2 sigmoid(.)), computed as the fused forward's prep does
// for a whole sequence: y_t[c] = sum_tau conv_w[h][c][tau] x_{t-2+tau}[c] over the raw
// rows (x_{t-2}, x_{t-1} from the convolution state), rounded to the element type, and
// beta_t = 2 sigmoid(z_t) (capped) divided by max(||y_t||^2, 1e-24), the squared norm of
// the rounded row: I - beta' y y^T is then H_t with w_t = y_t / max(||y_t||, 1e-12).  One
// wave per (batch, head), lane c holding channels c, c + 64, ...; the state moves on to
// (x_{t-1}, x_t), each lane rewriting only the channels it has read.
template <typename S, int D>
__global__ __launch_bounds__(64) void path_decode_produce_kernel(ProduceArgs a) {
    typedef Elem<S> E;
    constexpr int CPL = D / 64;  // channels per lane
    const int64_t g = blockIdx.x;
    const int hd = (int)(g % a.H), lane = threadIdx.x;
    const S *xr = (const S *)a.wraw + g * D;
    S *st = (S *)a.state + g * 2 * D;
    const float *cw = a.conv_w + (int64_t)hd * D * 3;
    S *wo = (S *)a.w_out + g * D;
    float yy = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        const S s0 = st[c], s1 = st[D + c], s2 = xr[c];
        const float y = cw[3 * c] * E::to_f32(s0) + cw[3 * c + 1] * E::to_f32(s1) + cw[3 * c + 2] * E::to_f32(s2);
        const S yr = E::from_float(y);
        wo[c] = yr;
        const float yf = E::to_f32(yr);
        yy += yf * yf;
        st[c] = s1;
        st[D + c] = s2;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) yy += __shfl_xor(yy, o);
    if (lane == 0) {
        float bt = 2.f / (1.f + expf(-a.zbeta[g]));
        if (a.beta_clip > 0.f) bt = fminf(bt, a.beta_clip);
        a.beta_out[g] = bt / fmaxf(yy, 1e-24f);
    }
}

hipError_t launch_decode_produce(const ProduceArgs &a, bool bf16, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H));
    if (a.d == 64) {
        if (bf16) hipLaunchKernelGGL((path_decode_produce_kernel<uint16_t, 64>), grid, dim3(64), 0, st, a);
        else hipLaunchKernelGGL((path_decode_produce_kernel<float, 64>), grid, dim3(64), 0, st, a);
    } else if (a.d == 128) {
        if (bf16) hipLaunchKernelGGL((path_decode_produce_kernel<uint16_t, 128>), grid, dim3(64), 0, st, a);
        else hipLaunchKernelGGL((path_decode_produce_kernel<float, 128>), grid, dim3(64), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
