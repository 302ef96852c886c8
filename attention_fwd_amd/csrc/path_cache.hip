// path_cache.hip -- decode cache from a forward pass (prefill -> decode).
//
// Source: "技術要約: PaTH Attention" (gist.science), section 3: at inference
// the newest transition matrix is applied in place to every cached key.  After
// a prefix of L tokens has gone through the forward pass, the cache a sequence
// of decode steps would have built holds, in row j,
//   ktilde_j = H_{L-1} ... H_{j+1} k_j
// (row L-1 is k_{L-1} itself), and the value rows unchanged.
//
// Built from the key-block records the forward pass left in its workspace:
// for a key j in block J, ktilde_j^T = khat_j^T P_{J+1} ... P_{nb-1}, where
// khat_j = H_last(J) ... H_{j+1} k_j and P_B = I - M_B are in record J.  So one
// right-to-left walk over the blocks of a head carries the suffix product
//   Sigma_J = P_{J+1} ... P_{nb-1}   (d x d, Sigma_{nb-1} = I, Sigma_{J-1} = P_J Sigma_J)
// and emits Ktilde_J = Khat_J Sigma_J.  Rows past L (zero padding in the last
// block) have w = 0, so their transitions are the identity.
//
// A workgroup owns one (batch, head); wave c keeps the 32 columns
// [32 c, 32 c + 32) of Sigma as d/32 fp32 accumulator tiles.  Per block it
// computes the transposed output tile Ktilde^T = Sigma^T Khat^T (so every
// lane holds one key row and stores 4 contiguous elements per register group)
// and the update Sigma <- Sigma + (-M_J) Sigma, both on matrix cores.  In bf16
// the accumulator Sigma is fed to the products as a pair of bf16 terms
// (hi + lo, about 16 significant bits), so the walk adds no rounding beyond
// that of the records and of the stored cache.
#include "path_common.h"
#include "path_kernels.h"
#include "path_layout.h"

namespace path {
namespace {

// hi and lo bf16 fragments of 8 fp32 values x (x ~= hi + lo to about 2^-17 relative).
__device__ __forceinline__ void split_frag(const f32x16 &acc, int c, i16x8 &hi, i16x8 &lo) {
    float xh[8], xl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = acc[8 * c + e];
        xh[e] = bf16_to_f32(to_bf16(x));
        xl[e] = x - xh[e];
    }
    hi = Elem<uint16_t>::from_f32(xh);
    lo = Elem<uint16_t>::from_f32(xl);
}

template <typename S, int D>
__global__ __launch_bounds__(64 * (D / 32)) void path_cache_kernel(CacheArgs a) {
    typedef Elem<S> E;
    typedef typename E::Frag Frag;
    constexpr int DT = D / 32, KCH = D / 16;
    constexpr int REC = 2 * kBlk * D + D * D;
    const int tid = threadIdx.x, ct = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    const int64_t bh = blockIdx.x;
    const int nb = (int)lay.nb;
    const S *recs = (const S *)((const char *)a.ws + lay.off_rec) + bh * lay.nb * REC;
    S *kc = (S *)a.kc + bh * a.ncap * D;

    // values: rows [0, L) copied as they are (16-byte chunks over the workgroup)
    {
        const S *vs = (const S *)a.v + bh * (int64_t)a.L * D;
        S *vd = (S *)a.vc + bh * a.ncap * D;
        constexpr int CH = 16 / (int)sizeof(S);
        const int64_t nch = (int64_t)a.L * D / CH;
        for (int64_t i = tid; i < nch; i += 64 * DT) *(u32x4 *)(vd + i * CH) = *(const u32x4 *)(vs + i * CH);
    }

    // forget gate: inclusive prefix sums of log f (wave 0, 64 tokens per pass)
    if (a.logf && ct == 0) {
        const float *lf = a.logf + bh * (int64_t)a.L;
        float *fc = a.fcache + bh * a.ncap;
        float carry = 0.f;
        for (int c0 = 0; c0 < a.L; c0 += 64) {
            float v = c0 + lane < a.L ? lf[c0 + lane] : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float u = __shfl_up(v, o);
                if (lane >= o) v += u;
            }
            v += carry;
            if (c0 + lane < a.L) fc[c0 + lane] = v;
            carry = __shfl(v, 63);
        }
    }

    // Sigma[:, 32 ct .. 32 ct + 31] = identity columns
    f32x16 sg[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sg[dt][r] = (32 * dt + acc_row(r, h) == 32 * ct + l32) ? 1.f : 0.f;

    for (int J = nb - 1; J >= 0; --J) {
        const S *rec = recs + (int64_t)J * REC;
        const S *rk = rec, *rm = rec + 2 * kBlk * D;
        Frag kf[2][KCH];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kc2 = 0; kc2 < KCH; ++kc2) kf[hf][kc2] = *(const Frag *)(rk + ((hf * KCH + kc2) * 64 + lane) * 8);
        // Sigma as operand fragments (k = input head dimension): A of Sigma^T and B of Sigma
        Frag sf[KCH], sl[KCH];
#pragma unroll
        for (int kc2 = 0; kc2 < KCH; ++kc2) {
            if constexpr (sizeof(S) == 2)
                split_frag(sg[kc2 >> 1], kc2 & 1, sf[kc2], sl[kc2]);
            else
                sf[kc2] = acc_frag<S>(sg[kc2 >> 1], kc2 & 1);
        }
        // Ktilde_J^T (columns 32 ct.., keys 32 hf..) = Sigma^T Khat_J^T -> cache rows 64 J + 32 hf + lane
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            f32x16 o = {};
#pragma unroll
            for (int kc2 = 0; kc2 < KCH; ++kc2) {
                E::mma(o, sf[kc2], kf[hf][kc2]);
                if constexpr (sizeof(S) == 2) E::mma(o, sl[kc2], kf[hf][kc2]);
            }
            const int64_t row = (int64_t)J * kBlk + 32 * hf + l32;
            if (row < a.L) {
                S *p = kc + row * D + 32 * ct;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int dd = 8 * g + 4 * h;
                    if constexpr (sizeof(S) == 2) {
                        *(u32x2 *)(p + dd) = u32x2{pack_bf16(o[4 * g], o[4 * g + 1]), pack_bf16(o[4 * g + 2], o[4 * g + 3])};
                    } else {
                        *(f32x4 *)(p + dd) = f32x4{o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]};
                    }
                }
            }
        }
        // Sigma <- Sigma + (-M_J) Sigma
        if (J > 0) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int kc2 = 0; kc2 < KCH; ++kc2) {
                    const Frag mf = *(const Frag *)(rm + ((dt * KCH + kc2) * 64 + lane) * 8);
                    E::mma(sg[dt], mf, sf[kc2]);
                    if constexpr (sizeof(S) == 2) E::mma(sg[dt], mf, sl[kc2]);
                }
        }
    }
}

}  // namespace

template <typename S, int D>
static hipError_t launch_cache_t(const CacheArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((path_cache_kernel<S, D>), dim3((unsigned)((int64_t)a.B * a.H)), dim3(64 * (D / 32)), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_cache(const CacheArgs &a, bool bf16, hipStream_t st) {
    if (a.d == 64) return bf16 ? launch_cache_t<uint16_t, 64>(a, st) : launch_cache_t<float, 64>(a, st);
    if (a.d == 128) return bf16 ? launch_cache_t<uint16_t, 128>(a, st) : launch_cache_t<float, 128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace path
