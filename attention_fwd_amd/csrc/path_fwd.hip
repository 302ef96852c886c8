// path_fwd.hip -- blockwise PaTH forward kernel: right-to-left scan over key
// blocks with online softmax.
//
// Source: "技術要約: PaTH Attention" (gist.science), section 3: per-block
// boundary-adjusted queries/keys, a right-to-left scan over key/value blocks
// that accumulates the block Householder products, and FlashAttention-style
// online softmax so the L x L matrix is never formed.
//
// For a query i in block I and a key j in block J < I the logit factors as
//   s_ij = khat_j^T  P_{J+1} ... P_{I-1}  qhat_i,   P_B = H_first(B) ... H_last(B)
// so walking J = I-1, I-2, ..., 0 the query side only needs
//   qt <- P_J qt = qt - M_J qt            after block J has been scored.
// Each wave owns 64 queries of one block (two 32-column accumulator tiles) and
// keeps qt^T (d x 64), the output O^T (d x 64) and the logits S^T (64 keys x
// 64 queries) in matrix-core accumulators.  Working transposed makes every
// accumulator directly reusable as the B operand of the next product:
//   S^T  = khat_J  qt^T        (A: khat fragments, B: qt^T accumulators)
//   qt^T = qt^T + (-M_J) qt^T  (A: -M fragments,   B: qt^T accumulators)
//   O^T += V_J^T  P^T          (A: V^T fragments,  B: softmax of S^T)
// Softmax runs down accumulator columns: 32 values in-lane plus one swap
// between lane halves.  The diagonal block was already folded into `out` and
// the (max, sum) workspace by the prep kernel, so every block here is a full,
// unmasked 64 x 64 tile.  A workgroup is 4 waves = 4 consecutive query blocks
// sharing each key-block record (khat, V^T, -M: 24 KiB bf16 at d = 64),
// double-buffered in LDS.
#include "path_common.h"
#include "path_kernels.h"
#include "path_layout.h"

namespace path {
namespace {

template <typename S, int D, bool FOX>
__global__ __launch_bounds__(256, 1) void path_fwd_kernel(FwdArgs a) {
    static_assert(D == 64, "forward kernel is laid out for head dimension 64");
    typedef Elem<S> E;
    typedef typename E::Frag Frag;
    constexpr int REC = 2 * kBlk * D + D * D;  // elements per key-block record
    constexpr int KCH = D / 16, DT = D / 32;
    constexpr int VEC = 16 / (int)sizeof(S);   // elements per 16-byte load
    constexpr int NLD = REC / VEC / 256;       // 16-byte loads per thread per record
    static_assert(REC % (VEC * 256) == 0, "record must split evenly over the workgroup");
    __shared__ __attribute__((aligned(32))) S srec[2][REC];
    __shared__ float stail[2][kBlk];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    const int nb = (int)lay.nb;
    const int ntile = (nb + 3) / 4;

    // Work item: heads are kept together on one XCD (workgroups are dealt
    // round-robin over the 8 XCDs, each with its own L2), longest tiles first.
    const int64_t total = (int64_t)ntile * lay.bh;
    int64_t g = blockIdx.x;
    int64_t item = (total % 8 == 0) ? (g % 8) * (total / 8) + g / 8 : g;
    const int64_t bh = item / ntile;
    const int tile = ntile - 1 - (int)(item % ntile);

    const int I = 4 * tile + wv;                 // this wave's query block
    const bool active = I >= 1 && I < nb;        // block 0 is complete after prep
    const int Jtop = min(4 * tile + 3, nb - 1) - 1;
    if (Jtop < 0) return;

    const S *recs = (const S *)((const char *)a.ws + lay.off_rec) + bh * lay.nb * REC;
    const float *fk = (const float *)((const char *)a.ws + lay.off_fk) + bh * lay.lp;
    const float *fb = (const float *)((const char *)a.ws + lay.off_fb) + bh * lay.nb;

    // ---- per-wave state
    f32x16 qt[DT][2], o[DT][2];
    Frag qb[2][KCH];
    float m[2], lp[2], off[2];
    if (active) {
        const S *qh = (const S *)((const char *)a.ws + lay.off_qhat) + (bh * lay.lp + (int64_t)I * kBlk) * D;
        const S *od = (const S *)a.out + (bh * a.L + (int64_t)I * kBlk) * D;
        const float *md = (const float *)((const char *)a.ws + lay.off_mdiag) + bh * lay.lp + (int64_t)I * kBlk;
        const float *ld = (const float *)((const char *)a.ws + lay.off_ldiag) + bh * lay.lp + (int64_t)I * kBlk;
        const float *fq = (const float *)((const char *)a.ws + lay.off_fq) + bh * lay.lp + (int64_t)I * kBlk;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int i = 32 * ct + l32;
            const bool valid = (int64_t)I * kBlk + i < a.L;
            m[ct] = md[i];
            const float ls = ld[i];
            lp[ct] = h == 0 ? ls : 0.f;
            off[ct] = FOX ? fq[i] : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = 32 * dt + acc_row(r, h);
                    qt[dt][ct][r] = E::to_f32(qh[(int64_t)i * D + d]);
                    o[dt][ct][r] = valid ? E::to_f32(od[(int64_t)i * D + d]) * ls : 0.f;
                }
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int kc = 0; kc < KCH; ++kc) qb[ct][kc] = acc_frag<S>(qt[kc >> 1][ct], kc & 1);
    }

    // ---- stage the first record
    u32x4 pre[NLD];
    float pre_tail = 0.f;
    {
        const u32x4 *src = (const u32x4 *)(recs + (int64_t)Jtop * REC);
#pragma unroll
        for (int t = 0; t < NLD; ++t) pre[t] = src[tid + 256 * t];
        if (FOX && tid < kBlk) pre_tail = fk[(int64_t)Jtop * kBlk + tid];
        u32x4 *dst = (u32x4 *)srec[0];
#pragma unroll
        for (int t = 0; t < NLD; ++t) dst[tid + 256 * t] = pre[t];
        if (FOX && tid < kBlk) stail[0][tid] = pre_tail;
    }

    const float c2 = a.scale * kLog2e;
    for (int J = Jtop; J >= 0; --J) {
        const int buf = (Jtop - J) & 1;
        __syncthreads();
        if (J > 0) {  // prefetch the next record into registers
            const u32x4 *src = (const u32x4 *)(recs + (int64_t)(J - 1) * REC);
#pragma unroll
            for (int t = 0; t < NLD; ++t) pre[t] = src[tid + 256 * t];
            if (FOX && tid < kBlk) pre_tail = fk[(int64_t)(J - 1) * kBlk + tid];
        }
        if (active && J < I) {
            const S *sk = srec[buf];
            const S *sv = srec[buf] + kBlk * D;
            const S *sm = srec[buf] + 2 * kBlk * D;
            // S^T = khat_J qt^T
            f32x16 s[2][2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) s[rt][ct] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KCH; ++kc)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const Frag af = *(const Frag *)(sk + ((rt * KCH + kc) * 64 + lane) * 8);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) E::mma(s[rt][ct], af, qb[ct][kc]);
                }
            // qt <- P_J qt for the next (older) block
            if (J > 0) {
#pragma unroll
                for (int kc = 0; kc < KCH; ++kc)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const Frag af = *(const Frag *)(sm + ((dt * KCH + kc) * 64 + lane) * 8);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) E::mma(qt[dt][ct], af, qb[ct][kc]);
                    }
            }
            // online softmax down each column (log2 domain)
            float fbJ = 0.f;
            if (FOX) fbJ = fb[J];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                float mx = -INFINITY;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float x = s[rt][ct][r] * c2;
                        if (FOX) x += stail[buf][32 * rt + acc_row(r, h)] + off[ct];
                        s[rt][ct][r] = x;
                        mx = fmaxf(mx, x);
                    }
                mx = other_half_max(mx);
                const float mnew = fmaxf(m[ct], mx);
                const float alpha = fast_exp2(m[ct] - mnew);
                m[ct] = mnew;
                float sum = 0.f;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(s[rt][ct][r] - mnew);
                        s[rt][ct][r] = p;
                        sum += p;
                    }
                lp[ct] = lp[ct] * alpha + sum;
                if (__any(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[dt][ct][r] *= alpha;
                }
                if (FOX) off[ct] += fbJ;
            }
            // O^T += V_J^T P^T
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                Frag pf[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) pf[ct] = acc_frag<S>(s[kc >> 1][ct], kc & 1);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const Frag af = *(const Frag *)(sv + ((dt * 4 + kc) * 64 + lane) * 8);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) E::mma(o[dt][ct], af, pf[ct]);
                }
            }
            if (J > 0) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int kc = 0; kc < KCH; ++kc) qb[ct][kc] = acc_frag<S>(qt[kc >> 1][ct], kc & 1);
            }
        }
        if (J > 0) {
            u32x4 *dst = (u32x4 *)srec[buf ^ 1];
#pragma unroll
            for (int t = 0; t < NLD; ++t) dst[tid + 256 * t] = pre[t];
            if (FOX && tid < kBlk) stail[buf ^ 1][tid] = pre_tail;
        }
    }

    // ---- epilogue
    if (active) {
        S *go = (S *)a.out + (bh * a.L + (int64_t)I * kBlk) * D;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int i = 32 * ct + l32;
            const float lsum = other_half_sum(lp[ct]);
            if ((int64_t)I * kBlk + i >= a.L) continue;
            const float inv = 1.f / lsum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * dt + 8 * g4 + 4 * h;
                    S *p = go + (int64_t)i * D + d;
                    const f32x16 &c = o[dt][ct];
                    if constexpr (sizeof(S) == 2) {
                        u32x2 u = {pack_bf16(c[4 * g4] * inv, c[4 * g4 + 1] * inv),
                                   pack_bf16(c[4 * g4 + 2] * inv, c[4 * g4 + 3] * inv)};
                        *(u32x2 *)p = u;
                    } else {
                        f32x4 v = {c[4 * g4] * inv, c[4 * g4 + 1] * inv, c[4 * g4 + 2] * inv, c[4 * g4 + 3] * inv};
                        *(f32x4 *)p = v;
                    }
                }
            if (a.lse && h == 0) a.lse[bh * a.L + (int64_t)I * kBlk + i] = (m[ct] + __log2f(lsum)) * kLn2;
        }
    }
}

}  // namespace

template <typename S, int D, bool FOX>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    const int64_t ntile = (lay.nb + 3) / 4;
    dim3 grid((unsigned)(ntile * lay.bh));
    hipLaunchKernelGGL((path_fwd_kernel<S, D, FOX>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs &a, bool bf16, hipStream_t st) {
    if (a.d != 64) return hipErrorInvalidValue;
    if (bf16) return a.fox ? launch_fwd_t<uint16_t, 64, true>(a, st) : launch_fwd_t<uint16_t, 64, false>(a, st);
    return a.fox ? launch_fwd_t<float, 64, true>(a, st) : launch_fwd_t<float, 64, false>(a, st);
}

}  // namespace path
