// path_prep.hip -- per-block UT-transform prep kernel of the PaTH forward pass.
//
// Sources: "技術要約: PaTH Attention" (gist.science), section 3: a product of
// Householder-like matrices H_s = I - beta_s w_s w_s^T has the compact form
// P = I - W^T T^-1 W with T triangular and built from beta (UT transform), and
// the blockwise algorithm precomputes boundary-adjusted queries and keys per
// block before a right-to-left scan over key blocks.
//
// One workgroup (4 waves) handles one block of 64 tokens of one (batch, head),
// rows s = 0..63 of the block (global token 64 J + s), D = head dimension.
// With G = W W^T (W: the block's w_s as rows) and D_b = diag(beta):
//   A   = (I + strictly_lower(D_b G))^-1 D_b   (lower triangular, fp32
//         forward substitution).  For any rows a <= b of the block,
//         H_a ... H_b = I - W_ab^T A_up[a..b] W_ab with A_up = A^T, and the
//         sub-block of A over a contiguous range is the same matrix for that
//         range, so every partial product of the block is a masked product.
//   U   = A W                          (64 x D)
//   M   = U^T W = W^T A^T W            (D x D): P_J = H_first ... H_last = I - M
//   qhat_i = H_first ... H_i q_i       = q_i - sum_{c<=i} (q_i.w_c) U_c
//   khat_j = H_last ... H_{j+1} k_j    = k_j - sum_{r>j} (k_j.w_r) (A^T W)_r
//   diagonal logits (j <= i in the block):
//     s_ij = k_j.q_i - sum_{r>j} (k_j.w_r) Z_ir,   Z = tril(Q W^T) A
// Outputs (see path_layout.h): the key-block record (khat, V^T, -M as matrix-
// core fragments), qhat, and the diagonal block's softmax state: its
// normalised output goes straight to `out`, its max/sum to the workspace.
// All matrices live in LDS; every product is a 32x32 MFMA tile.
#include "path_common.h"
#include "path_kernels.h"
#include "path_layout.h"

namespace path {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename S, int D>
struct PrepCfg {
    static constexpr bool kBf = sizeof(S) == 2;
    // Row padding.  fp32: 4 elements, rows stay 16-byte aligned.  bf16: 12 elements, a
    // row pitch of 38 (d = 64) or 70 (d = 128) dwords: the 8-byte fragment reads of 32
    // consecutive rows then cover all 64 banks once, and the 2-byte transposed reads,
    // whose lane halves sit 4 rows apart, fall on disjoint banks (a 16-byte pad, 36
    // dwords, paired the rows r and r + 16 on the same banks); rows are 8-byte aligned
    // only, so 16-byte accesses to them are split (lds_store16 / lds_load16).
    static constexpr int PAD = kBf ? 12 : 4;
    static constexpr int SP = 64 + PAD;    // padded row stride of [.][64] matrices (W^T)
    static constexpr int SPD = D + PAD;    // padded row stride of [64][D] matrices (W, Q, K)
    static constexpr int MAT = 64 * SP;    // one 64 x 64 matrix
    static constexpr int MATD = 64 * SPD;  // one 64 x D matrix, token rows
    static constexpr int MATT = D * SP;    // one D x 64 matrix, head-dimension rows
    // G and E of the triangular solve: fp32, only the ten 16 x 16 tiles on or
    // below the diagonal, tile (I, K) at TS * (I (I + 1) / 2 + K), row pitch TP
    // (unpadded: the solve runs while the other workgroups of the compute unit
    // keep it busy, and the LDS it saves keeps three workgroups per compute unit).
    static constexpr int TP = 16, TS = 16 * TP;
    // W, X, Y live for the whole kernel.  bf16 also keeps W^T (fp32 has no
    // room for transposed copies and reads them with a stride instead) in W's
    // slot once the products with W are done, written from registers.  A
    // second region is reused: Q, K while the products with them run, then G
    // and E for the triangular solve, then A, A^T and V^T.  X, Y, A, A^T and
    // V^T are kept in matrix-core fragment order (FRAG: 64 rows x 64 k, each
    // lane's 8 elements contiguous), so a wave reads each operand with
    // 16-byte accesses of consecutive lanes (conflict-free) and writes X and
    // Y straight from its accumulators.  At D = 64, bf16, this is 50 KiB, so
    // three workgroups share a CU.
    static constexpr int FRAG = 64 * 64;
    static constexpr bool kWtLate = kBf;
    static constexpr int WSLOT = kWtLate ? cmax(MATD, MATT) : MATD;
    static constexpr int FIX = WSLOT + 2 * FRAG;  // elements
    // (+ 1 KiB after Q, K in phases 1-2: per-thread partial norms of the fused producer)
    static constexpr int RB = cmax(cmax(2 * MATD * (int)sizeof(S) + 1024, 2 * 10 * TS * 4), (2 * FRAG + D * 64) * (int)sizeof(S));
    static constexpr int WG_PER_CU = kBf ? (D == 64 ? 3 : 2) : 1;  // = waves per SIMD (4-wave workgroups)
};

// Offset (floats) of tile (I, K), K <= I, in the packed lower-triangular tile store.
__device__ __forceinline__ int tri_tile(int I, int K) { return (I * (I + 1) / 2 + K) * (16 * 16); }

// Matrices of 64 k (tokens) in fragment order: fragment (row tile rt, k chunk kc) of
// lane l is 8 contiguous elements at ((4 rt + kc) 64 + l) 8; element e of lane l
// is (row 32 rt + l % 32, k 16 kc + frag_k(e, l / 32)).
template <typename S>
__device__ __forceinline__ typename Elem<S>::Frag frag_ld(const S *m, int rt, int kc, int lane) {
    return *(const typename Elem<S>::Frag *)(m + ((4 * rt + kc) * 64 + lane) * 8);
}
template <typename S>
__device__ __forceinline__ void frag_st(S *m, int rt, int kc, int lane, const typename Elem<S>::Frag &f) {
    *(typename Elem<S>::Frag *)(m + ((4 * rt + kc) * 64 + lane) * 8) = f;
}
// index of element (row, k)
__device__ __forceinline__ int frag_at(int row, int k) {
    return ((4 * (row >> 5) + (k >> 4)) * 64 + (row & 31) + 32 * ((k >> 2) & 1)) * 8 + 4 * ((k >> 3) & 1) + (k & 3);
}

// Fragment of the matrix view `m` (element (row, k) at row*SP + k when KC, at
// k*SP + row otherwise; SP = row stride in elements) for rows `row`, k in [k0, k0+16).
template <typename S, bool KC, int SP>
__device__ __forceinline__ typename Elem<S>::Frag lds_frag(const S *mat, int row, int k0, int h) {
    typedef typename Elem<S>::Frag Frag;
    if constexpr (KC) {
        const S *p = mat + row * SP + k0 + 4 * h;
        if constexpr (sizeof(S) == 2) {
            u32x2 a = *(const u32x2 *)p;
            u32x2 b = *(const u32x2 *)(p + 8);
            u32x4 u = {a.x, a.y, b.x, b.y};
            return __builtin_bit_cast(Frag, u);
        } else {
            f32x4 a = *(const f32x4 *)p;
            f32x4 b = *(const f32x4 *)(p + 8);
            Frag f;
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
            f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
            return f;
        }
    } else {
        S x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = mat[(k0 + frag_k(e, h)) * SP + row];
        if constexpr (sizeof(S) == 2) {
            u32x4 u;
            u.x = (uint32_t)x[0] | ((uint32_t)x[1] << 16);
            u.y = (uint32_t)x[2] | ((uint32_t)x[3] << 16);
            u.z = (uint32_t)x[4] | ((uint32_t)x[5] << 16);
            u.w = (uint32_t)x[6] | ((uint32_t)x[7] << 16);
            return __builtin_bit_cast(Frag, u);
        } else {
            Frag f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = x[e];
            return f;
        }
    }
}

// c += A(m0.., k) * B(n0.., k) over k in [0, K): one 32x32 tile (SA, SB: row strides).
template <typename S, bool AKC, bool BKC, int SA, int SB>
__device__ __forceinline__ void tile_mma(f32x16 &c, const S *A, const S *B, int m0, int n0, int K, int lane) {
    const int h = lane >> 5, l = lane & 31;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        auto a = lds_frag<S, AKC, SA>(A, m0 + l, k0, h);
        auto b = lds_frag<S, BKC, SB>(B, n0 + l, k0, h);
        Elem<S>::mma(c, a, b);
    }
}

// 16 bytes to / from a padded LDS row: one access for fp32 (rows 16-byte
// aligned), two 8-byte accesses for bf16 (rows 8-byte aligned).
template <typename S>
__device__ __forceinline__ void lds_store16(S *p, const u32x4 &v) {
    if constexpr (sizeof(S) == 2) {
        *(u32x2 *)p = u32x2{v.x, v.y};
        *(u32x2 *)(p + 4) = u32x2{v.z, v.w};
    } else {
        *(u32x4 *)p = v;
    }
}
template <typename S>
__device__ __forceinline__ u32x4 lds_load16(const S *p) {
    if constexpr (sizeof(S) == 2) {
        const u32x2 a = *(const u32x2 *)p, b = *(const u32x2 *)(p + 4);
        return u32x4{a.x, a.y, b.x, b.y};
    } else {
        return *(const u32x4 *)p;
    }
}

// Write the two fragments held in accumulator tile c (as the A operand whose
// rows are the tile's columns) to global memory: fragment f0 + c', lane-major.
template <typename S>
__device__ __forceinline__ void store_frags(S *dst, const f32x16 &c, int f0, int lane) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
        S *p = dst + ((int64_t)(f0 + cc) * 64 + lane) * 8;
        if constexpr (sizeof(S) == 2) {
            u32x4 u;
            u.x = pack_bf16(c[8 * cc + 0], c[8 * cc + 1]);
            u.y = pack_bf16(c[8 * cc + 2], c[8 * cc + 3]);
            u.z = pack_bf16(c[8 * cc + 4], c[8 * cc + 5]);
            u.w = pack_bf16(c[8 * cc + 6], c[8 * cc + 7]);
            *(u32x4 *)p = u;
        } else {
            f32x4 a = {c[8 * cc + 0], c[8 * cc + 1], c[8 * cc + 2], c[8 * cc + 3]};
            f32x4 b = {c[8 * cc + 4], c[8 * cc + 5], c[8 * cc + 6], c[8 * cc + 7]};
            *(f32x4 *)p = a;
            *(f32x4 *)(p + 4) = b;
        }
    }
}

// Store rows of a transposed accumulator tile (rows = d, cols = token) into a
// natural [token][D] global array: 4 contiguous d per register group.
template <typename S, int D>
__device__ __forceinline__ void store_rows_t(S *dst, const f32x16 &c, int d0, int tok, float mul, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int d = d0 + 8 * g + 4 * h;
        S *p = dst + (int64_t)tok * D + d;
        if constexpr (sizeof(S) == 2) {
            u32x2 u = {pack_bf16(c[4 * g] * mul, c[4 * g + 1] * mul), pack_bf16(c[4 * g + 2] * mul, c[4 * g + 3] * mul)};
            *(u32x2 *)p = u;
        } else {
            f32x4 v = {c[4 * g] * mul, c[4 * g + 1] * mul, c[4 * g + 2] * mul, c[4 * g + 3] * mul};
            *(f32x4 *)p = v;
        }
    }
}

// c += A(m0.., k) * B where B's fragments come from two accumulator tiles
// (rows = contraction index): k chunk kc is register half kc%2 of tile kc/2.
template <typename S, bool AKC, int SA>
__device__ __forceinline__ void tile_mma_breg(f32x16 &c, const S *A, int m0, const f32x16 *bt, int lane) {
    const int h = lane >> 5, l = lane & 31;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        auto a = lds_frag<S, AKC, SA>(A, m0 + l, 16 * kc, h);
        Elem<S>::mma(c, a, acc_frag<S>(bt[kc >> 1], kc & 1));
    }
}
// the same with A in fragment order (row tile rt)
template <typename S>
__device__ __forceinline__ void tile_mma_fbreg(f32x16 &c, const S *A, int rt, const f32x16 *bt, int lane) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(c, frag_ld<S>(A, rt, kc, lane), acc_frag<S>(bt[kc >> 1], kc & 1));
}

// c += A * B where A's fragments come from two accumulator tiles and B is in fragment
// order (row tile rt).
template <typename S>
__device__ __forceinline__ void tile_mma_areg_f(f32x16 &c, const f32x16 *at, const S *B, int rt, int lane) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(c, acc_frag<S>(at[kc >> 1], kc & 1), frag_ld<S>(B, rt, kc, lane));
}

template <typename S, int D, bool FOX>
__global__ __launch_bounds__(256, (PrepCfg<S, D>::WG_PER_CU)) void path_prep_kernel(PrepArgs a) {
    static_assert(D == 64 || D == 128, "prep kernel: head dimension 64 or 128");
    typedef PrepCfg<S, D> C;
    constexpr int SP = C::SP, SPD = C::SPD, MAT = C::MAT, TP = C::TP;
    static_assert(C::TS == 16 * 16, "tri_tile assumes 16 x 16 tiles");
    constexpr bool kBf = C::kBf, kWtLate = C::kWtLate;
    constexpr int CH = 16 / (int)sizeof(S);  // elements per 16-byte chunk
    constexpr int RCH = D / CH;              // chunks per row
    constexpr int VPT = 64 * RCH / 256;      // chunks per thread per matrix
    constexpr int DT = D / 32;               // 32-row head-dimension tiles
    __shared__ __attribute__((aligned(16))) S fixed[C::FIX];
    __shared__ __attribute__((aligned(16))) char region[C::RB];
    __shared__ float sBeta[64], sCl[64];

    // X = tril(Q W^T) (rows queries i, k over tokens c) and -Y, Y = strictly_upper(K W^T)
    // (rows keys j, k over tokens r), in fragment order
    S *sW = fixed, *sX = fixed + C::WSLOT, *sY = sX + C::FRAG;
    S *sWt = kBf ? fixed : nullptr;
    S *sQ = (S *)region, *sK = (S *)region + C::MATD;               // phases 1-2
    float *sPart = (float *)((char *)region + 2 * C::MATD * sizeof(S));  // phases 1-2, fused producer: [4][64]
    float *sG = (float *)region, *sE = (float *)region + 10 * C::TS;  // phase 3
    // phase 4, fragment order: A (rows t, k over c), A^T (rows r, k over c: A[c][r]), V^T (rows d, k over tokens)
    S *sA = (S *)region, *sAt = sA + C::FRAG, *sVt = sAt + C::FRAG;

    const int L = a.L;
    const FwdLayout lay = fwd_layout(a.B, a.H, L, D, sizeof(S));
    const int J = (int)(blockIdx.x % lay.nb);
    const int64_t bh = blockIdx.x / lay.nb;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int64_t row0 = (int64_t)J * kBlk;
    const int nvalid = min(kBlk, L - (int)row0);
    const int64_t tok0 = bh * L + row0;  // first token of the block in [B*H, L]

    // ---- 1. stage W, Q, K in LDS and V in registers (zero rows past L), beta, forget-gate prefix.
    // With the fused producer the staged W rows are the convolution outputs y_t (rounded to the
    // element type) and sBeta holds 2 sigmoid(z_t) (capped); it becomes beta_t / ||y_t||^2 below,
    // since I - beta w w^T with w = y / ||y|| equals I - (beta / ||y||^2) y y^T.
    const bool fused = a.conv_w != nullptr;
    u32x4 vreg[VPT];
    u32x4 wreg[VPT];
    float ynorm = 0.f;  // fused producer: this thread's part of ||y_row||^2 (row = lane)
    {
        const S *gq = (const S *)a.q + tok0 * D, *gk = (const S *)a.k + tok0 * D;
        const S *gw = (const S *)a.w + tok0 * D, *gv = (const S *)a.v + tok0 * D;
        // Every global load of this phase is issued first, without branches (rows past L
        // read row nvalid - 1 and are zeroed when consumed), so they are all in flight at once.
        // Q, K: consecutive lanes take consecutive chunks of a row (coalesced).  W, V:
        // consecutive lanes take consecutive rows (row = lane), so that the transposed LDS
        // copies (W^T, V^T) are written without bank conflicts.
        const u32x4 z4 = {0, 0, 0, 0};
        u32x4 lq[VPT], lk[VPT], lw[VPT], lv[VPT];
        u32x4 p1[VPT], p2[VPT];     // fused producer: rows t-1, t-2 from the previous block (lanes 0, 1)
        f32x4 cw4[VPT][3 * CH / 4];  // fused producer: this chunk's convolution weights
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            const int idx = tid + 256 * s;
            const int r = min(idx / RCH, nvalid - 1), cc = idx % RCH;
            lq[s] = *(const u32x4 *)(gq + r * D + cc * CH);
            lk[s] = *(const u32x4 *)(gk + r * D + cc * CH);
            const int rw = min(lane, nvalid - 1), cw = idx / 64;
            lw[s] = *(const u32x4 *)(gw + rw * D + cw * CH);
            lv[s] = *(const u32x4 *)(gv + rw * D + cw * CH);
            if (fused) {
                // previous-block rows exist for row0 >= 1 (t - 1) and row0 + lane >= 2 (t - 2)
                const int64_t o1 = (lane == 0 && row0 >= 1) ? -D : 0;
                const int64_t o2 = (lane < 2 && row0 + lane >= 2) ? (int64_t)(lane - 2) * D : 0;
                p1[s] = *(const u32x4 *)(gw + o1 + cw * CH);
                p2[s] = *(const u32x4 *)(gw + o2 + cw * CH);
                // the chunk (cw = wave + 4 s) is the same for the whole wave: one scalar read of its taps
                const int cwu = __builtin_amdgcn_readfirstlane(cw);
                const f32x4 *cwp = (const f32x4 *)(a.conv_w + ((int64_t)((int)bh % a.H) * D + cwu * CH) * 3);
#pragma unroll
                for (int u = 0; u < 3 * CH / 4; ++u) cw4[s][u] = cwp[u];
            }
        }
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            const int idx = tid + 256 * s;
            const int r = idx / RCH, cc = idx % RCH;
            const bool qok = r < nvalid, wok = lane < nvalid;
            lds_store16<S>(sQ + r * SPD + cc * CH, qok ? lq[s] : z4);
            lds_store16<S>(sK + r * SPD + cc * CH, qok ? lk[s] : z4);
            const int rw = lane, cw = idx / 64;
            u32x4 vw = wok ? lw[s] : z4;
            const u32x4 vv = wok ? lv[s] : z4;
            if (fused) {
                // y_t[c] = sum_tau cw[c][tau] x_{t-2+tau}[c] (causal, zero before token 0); rows
                // t-1 and t-2 of this block are the neighbouring lanes' x
                u32x4 x1, x2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x1[e] = (uint32_t)__shfl_up((int)vw[e], 1);
                    x2[e] = (uint32_t)__shfl_up((int)vw[e], 2);
                }
                if (rw == 0) x1 = row0 >= 1 ? p1[s] : z4;
                if (rw < 2) x2 = row0 + rw >= 2 ? p2[s] : z4;
                const float *tap = (const float *)cw4[s];
                const S *e0 = (const S *)&vw, *e1 = (const S *)&x1, *e2 = (const S *)&x2;
                float y[CH];
#pragma unroll
                for (int e = 0; e < CH; ++e)
                    y[e] = tap[3 * e] * Elem<S>::to_f32(e2[e]) + tap[3 * e + 1] * Elem<S>::to_f32(e1[e]) +
                           tap[3 * e + 2] * Elem<S>::to_f32(e0[e]);
                if constexpr (sizeof(S) == 2) {
                    vw = u32x4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                               pack_bf16(y[6], y[7])};
                } else {
                    vw = __builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]});
                }
                if (!wok) vw = z4;
                const S *ey = (const S *)&vw;  // the norm of the rounded row, as the products see it
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    const float t2 = Elem<S>::to_f32(ey[e]);
                    ynorm += t2 * t2;
                }
            }
            vreg[s] = vv;
            lds_store16<S>(sW + rw * SPD + cw * CH, vw);
            wreg[s] = vw;
        }
        if (tid < 64) {
            float bt = 0.f;
            if (tid < nvalid) {
                if (fused) {
                    bt = 2.f / (1.f + expf(-a.zbeta[tok0 + tid]));
                    if (a.beta_clip > 0.f) bt = fminf(bt, a.beta_clip);
                } else {
                    bt = a.beta[tok0 + tid];
                }
            }
            sBeta[tid] = bt;
        }
        if (FOX && wv == 0) {
            // inclusive prefix of log f inside the block (zero past L)
            float v = lane < nvalid ? a.logf[tok0 + lane] : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                float u = __shfl_up(v, o);
                if (lane >= o) v += u;
            }
            sCl[lane] = v;
            const float total = __shfl(v, 63);
            float *fq = (float *)((char *)a.ws + lay.off_fq), *fk = (float *)((char *)a.ws + lay.off_fk);
            float *fb = (float *)((char *)a.ws + lay.off_fb);
            fq[bh * lay.lp + row0 + lane] = v * kLog2e;
            fk[bh * lay.lp + row0 + lane] = (total - v) * kLog2e;
            if (lane == 0) fb[bh * lay.nb + J] = total * kLog2e;
        }
    }
    if (fused) sPart[wv * 64 + lane] = ynorm;
    __syncthreads();
    if ((FOX || fused) && wv == 3) {
        // row s = lane.  Fused producer: beta_s <- beta_s / max(||y_s||^2, 1e-24) (the
        // normalisation y / max(||y||, 1e-12)).  Forget gate: bound for skipping negligible
        // key blocks in the scan; the block's transitions are contractions when
        // 0 <= beta_s ||w_s||^2 <= 2.
        float kk = 0.f, ww = 0.f;
        if (fused) ww = (sPart[lane] + sPart[64 + lane]) + (sPart[128 + lane] + sPart[192 + lane]);
#pragma unroll
        for (int c0 = 0; c0 < D; c0 += CH) {
            if (!fused) {
                const u32x4 uw = lds_load16<S>(sW + lane * SPD + c0);
                const S *ew = (const S *)&uw;
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    const float xw = Elem<S>::to_f32(ew[e]);
                    ww += xw * xw;
                }
            }
            if (FOX) {
                const u32x4 uk = lds_load16<S>(sK + lane * SPD + c0);
                const S *ek = (const S *)&uk;
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    const float xk = Elem<S>::to_f32(ek[e]);
                    kk += xk * xk;
                }
            }
        }
        float bt = sBeta[lane];
        if (fused) {
            bt = bt / fmaxf(ww, 1e-24f);
            sBeta[lane] = bt;  // read again only after the next barrier
        }
        if (FOX) {
            const float bw = bt * ww;
            const bool contr = bw >= 0.f && bw <= 2.f;
            float kn = contr ? sqrtf(kk) * (1.f + 0x1p-10f) : INFINITY;  // rounded up
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) kn = fmaxf(kn, __shfl_xor(kn, o));
            if (lane == 0) ((float *)((char *)a.ws + lay.off_kn))[bh * lay.nb + J] = kn;
        }
    }

    const int mt = (wv >> 1) * 32, nt = (wv & 1) * 32;  // this wave's tile of a 64x64 product
    typedef typename Elem<S>::Frag Frag;

    // ---- 2. G = W W^T, X = tril(Q W^T), -Y = -strictly_upper(K W^T); products with Q and K
    f32x16 g = {};
    // Accumulators carried into phase 4: waves 0,1 the diagonal logits K Q^T (s), the waves of
    // phase 4b the Q^T and K^T tiles of their head-dimension tile (qi, ki).  At D = 64 no wave
    // has both, and s shares qi's registers.
    f32x16 carry[D == 64 ? 4 : 6];
    f32x16 *const s = carry, *const qi = D == 64 ? carry : carry + 2, *const ki = qi + 2;
    tile_mma<S, true, true, SPD, SPD>(g, sW, sW, mt, nt, D, lane);
    {
        // The accumulator tile W Q^T (rows c, columns i), read as fragments whose k is the
        // accumulator row, is X's fragments of row tile nt / 32, k chunks mt / 16 .. (likewise
        // W K^T and Y).  Tiles wholly outside a triangle are zero: for mt < nt every c <= i and
        // no r > j, for mt > nt the reverse.
        const Frag zf = {};
#pragma unroll
        for (int which = 0; which < 2; ++which) {  // 0: X, 1: -Y
            const bool full = which == 0 ? mt < nt : mt > nt, none = which == 0 ? mt > nt : mt < nt;
            S *dst = which == 0 ? sX : sY;
            if (none) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) frag_st<S>(dst, nt >> 5, (mt >> 4) + hf, lane, zf);
            } else {
                f32x16 cx = {};
                tile_mma<S, true, true, SPD, SPD>(cx, sW, which == 0 ? sQ : sK, mt, nt, D, lane);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = mt + 16 * hf + frag_k(e, h), col = nt + l32;
                        const bool keep = full || (which == 0 ? row <= col : row > col);
                        const float v = which == 0 ? cx[8 * hf + e] : -cx[8 * hf + e];
                        x[e] = keep ? v : 0.f;
                    }
                    frag_st<S>(dst, nt >> 5, (mt >> 4) + hf, lane, Elem<S>::from_f32(x));
                }
            }
        }
    }
    if (wv < 2) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            s[rt] = f32x16{};
            // key tiles after the query tile are wholly masked
            if (rt <= wv) tile_mma<S, true, true, SPD, SPD>(s[rt], sK, sQ, 32 * rt, 32 * wv, D, lane);
        }
    }
    if (wv >= 2 || D > 64) {
        // Q^T and K^T tiles (rows d, columns tokens) as products with identity fragments
        // (exact: one nonzero term per sum)
        Frag idp[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 16 * hf + frag_k(e, h) == l32 ? 1.f : 0.f;
            idp[hf] = Elem<S>::from_f32(x);
        }
        const int dt = D == 64 ? (wv & 1) : (wv ^ 2);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            qi[t] = f32x16{};
            ki[t] = f32x16{};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                Elem<S>::mma(qi[t], idp[hf], lds_frag<S, true, SPD>(sQ, 32 * t + l32, 32 * dt + 16 * hf, h));
                Elem<S>::mma(ki[t], idp[hf], lds_frag<S, true, SPD>(sK, 32 * t + l32, 32 * dt + 16 * hf, h));
            }
        }
    }
    __syncthreads();  // Q, K dead: their space becomes G and E (tiles on or below the diagonal)
    if (mt >= nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = mt + acc_row(r, h), col = nt + l32;
            if ((row >> 4) >= (col >> 4)) sG[tri_tile(row >> 4, col >> 4) + (row & 15) * TP + (col & 15)] = g[r];
        }
    }
    __syncthreads();
    // ---- 3. E = (I + strictly_lower(D_b G))^-1 in 16 x 16 tiles, A = E D_b.
    // (a) diagonal tiles, one per wave: column t, rows c = p (mod 4) per lane;
    //     x_r = [r == t] - beta_r sum_{c<r} G_rc x_c (entries not yet known are 0)
    {
        const int I16 = 16 * wv, t = lane >> 2, p = lane & 3;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
        const float *gt = sG + tri_tile(wv, wv);
        // the tile's entries this lane uses and the betas do not depend on the serial
        // loop: they are read PF steps ahead, so a step does not wait for its LDS reads
        constexpr int PF = 3;
        float gv[PF][4], bv[PF];
        auto fetch = [&](int r, int slot) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) gv[slot][q4] = gt[r * TP + p + 4 * q4];
            bv[slot] = sBeta[I16 + r];
        };
#pragma unroll
        for (int r = 0; r < PF; ++r) fetch(r, r);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int sl = r % PF;
            float part = (gv[sl][0] * xs[0] + gv[sl][1] * xs[1]) + (gv[sl][2] * xs[2] + gv[sl][3] * xs[3]);
            const float br = bv[sl];
            if (r + PF < 16) fetch(r + PF, sl);
            part = sum4(part);
            // branch-free (selects): lanes differ in t and p
            const float xv = -br * part;
            const float x = (r == t) ? 1.f : (r > t ? xv : 0.f);
            xs[r >> 2] = (p == (r & 3)) ? x : xs[r >> 2];
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) sE[tri_tile(wv, wv) + (4 * cc + p) * TP + t] = xs[cc];
    }
    __syncthreads();
    // (b) off-diagonal tiles by distance from the diagonal, one tile per wave:
    //     E_IJ = -E_II T_IJ,  T_IJ = D_I sum_{K=J}^{I-1} G_IK E_KJ,
    //     as 16x16x4 fp32 matrix-core products.  With the k order k(s, g) = 4g + s
    //     (lane group g = lane / 16 supplies k = 4g + s at step s), register s of
    //     a 16x16 accumulator (rows 4g .. 4g+3, column lane % 16) is exactly the B
    //     operand of step s, so T feeds the second product from registers.
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
        if (wv < 4 - lev) {
            const int Jt = wv, It = wv + lev, i16 = lane & 15, g4 = 4 * (lane >> 4);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int K = Jt; K < It; ++K) {
                const f32x4 ga = *(const f32x4 *)(sG + tri_tile(It, K) + i16 * TP + g4);
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[st], sE[tri_tile(K, Jt) + (g4 + st) * TP + i16], t,
                                                             0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] *= sBeta[16 * It + g4 + r];
            const f32x4 ea = *(const f32x4 *)(sE + tri_tile(It, It) + i16 * TP + g4);
            f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) e = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[st], t[st], e, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sE[tri_tile(It, Jt) + (g4 + r) * TP + i16] = -e[r];
        }
        __syncthreads();
    }
    {
        // A = E D_b (lower triangle only: tiles above the diagonal are zero).
        // Thread (column c, 16 rows of row tile wv).
        const int c = tid & 63, rg = 16 * wv;
        const float bc = sBeta[c];
        const bool tile_ok = (c >> 4) <= wv;
        const float *et = sE + tri_tile(wv, tile_ok ? (c >> 4) : 0) + (c & 15);
        float av[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float ev = et[e * TP];  // always in bounds; read unconditionally, then selected
            av[e] = (tile_ok && c <= rg + e) ? ev * bc : 0.f;
        }
        __syncthreads();  // E and G are dead: their space becomes A, A^T and V^T
        // -A: rows rg + e, k = c (one element each); A^T: row c, k = rg .. rg + 15 (k chunk wv),
        // the two lane halves of the row
#pragma unroll
        for (int e = 0; e < 16; ++e) sA[frag_at(rg + e, c)] = Elem<S>::from_float(-av[e]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = av[frag_k(e, h2)];
            frag_st<S>(sAt, c >> 5, wv, (c & 31) + 32 * h2, Elem<S>::from_f32(x));
        }
#pragma unroll
        for (int s2 = 0; s2 < VPT; ++s2) {
            const int idx = tid + 256 * s2, vr = idx % 64, cw = idx / 64;
            const S *ve = (const S *)&vreg[s2];
#pragma unroll
            for (int e = 0; e < CH; ++e) sVt[frag_at(cw * CH + e, vr)] = ve[e];
            if constexpr (kWtLate) {  // W is dead since phase 2: its slot becomes W^T
                const S *we = (const S *)&wreg[s2];
#pragma unroll
                for (int e = 0; e < CH; ++e) sWt[(cw * CH + e) * SP + vr] = we[e];
            }
        }
    }
    __syncthreads();

    S *rec = (S *)((char *)a.ws + lay.off_rec) + (bh * lay.nb + J) * lay.rec_elems;
    S *recK = rec, *recV = rec + 64 * D, *recM = rec + 128 * D;
    constexpr int KCH = D / 16;  // k chunks over the head dimension

    if (wv < 2) {
        // ---- 4a. diagonal block, query column tile ct: Z^T = A^T X^T (Z = tril(Q W^T) A),
        //      S^T = K Q^T - Y Z^T, causal softmax down columns, O^T = V^T P^T
        const int ct = wv;
        const int i = 32 * ct + l32;  // query row in the block
        f32x16 zt[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            zt[rt] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(zt[rt], frag_ld<S>(sAt, rt, kc, lane), frag_ld<S>(sX, ct, kc, lane));
        }
        // key tiles rt <= ct only: the later one is wholly masked (P = 0); the mask is needed in
        // the tile rt = ct alone
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            if (rt <= ct) tile_mma_fbreg<S>(s[rt], sY, rt, zt, lane);  // sY holds -Y
        const float c2 = a.scale * kLog2e;
        const float cli = FOX ? sCl[i] : 0.f;
        float mx = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (rt > ct) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = 32 * rt + acc_row(r, h);
                float x = s[rt][r] * c2;
                if (FOX) x += (cli - sCl[j]) * kLog2e;
                if (rt == ct) x = j <= i ? x : -INFINITY;
                s[rt][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = other_half_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (rt > ct) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(s[rt][r] - mx);
                s[rt][r] = p;
                sum += p;
            }
        }
        sum = other_half_sum(sum);
        f32x16 o[DT];
#pragma unroll
        for (int d2 = 0; d2 < DT; ++d2) o[d2] = f32x16{};
        // each of the two waves stores half of the V^T record: fragments d2 = wv, wv + 2, ...,
        // kept by selects during the products and stored after them (no branch among the products)
        Frag vkeep[DT / 2][4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const bool live = (kc >> 1) <= ct;
            auto pf = acc_frag<S>(s[kc >> 1], kc & 1);
#pragma unroll
            for (int d2 = 0; d2 < DT; ++d2) {
                const Frag vf = frag_ld<S>(sVt, d2, kc, lane);
                if (live) Elem<S>::mma(o[d2], vf, pf);
                if ((d2 & 1) == 0) vkeep[d2 >> 1][kc] = vf;
                else vkeep[d2 >> 1][kc] = wv == 1 ? vf : vkeep[d2 >> 1][kc];
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < DT / 2; ++k2)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                S *dst = recV + ((int64_t)((2 * k2 + wv) * 4 + kc) * 64 + lane) * 8;
                *(Frag *)dst = vkeep[k2][kc];
            }
        if (h == 0) {
            float *md = (float *)((char *)a.ws + lay.off_mdiag), *ld = (float *)((char *)a.ws + lay.off_ldiag);
            md[bh * lay.lp + row0 + i] = mx;
            ld[bh * lay.lp + row0 + i] = sum;
        }
        if (i < nvalid) {
            const float inv = 1.f / sum;
            S *go = (S *)a.out + tok0 * D;
#pragma unroll
            for (int d2 = 0; d2 < DT; ++d2) store_rows_t<S, D>(go, o[d2], 32 * d2, i, inv, lane);
            if (h == 0 && a.lse) a.lse[tok0 + i] = (mx + __log2f(sum)) * kLn2;
        }
    }
    if (wv >= 2 || D > 64) {
        // ---- 4b. head-dimension tile dt: -U = (-A) W and R = A^T W (rows = block token,
        //      cols = d), then qhat^T = Q^T - U^T X^T, khat^T = K^T + R^T (-Y)^T and
        //      (-M)^T = W^T (-U), each using those accumulators as operands (bf16 reads W^T,
        //      fp32 reads W with a stride).  D = 64: waves 2, 3 take one tile each; D = 128:
        //      every wave takes one (waves 0, 1 after the diagonal block).
        const int dt = D == 64 ? (wv & 1) : (wv ^ 2);
        f32x16 nu[2], nr[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            nu[rt] = f32x16{};
            nr[rt] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                Frag wb;
                if constexpr (kBf) wb = lds_frag<S, true, SP>(sWt, 32 * dt + l32, 16 * kc, h);
                else wb = lds_frag<S, false, SPD>(sW, 32 * dt + l32, 16 * kc, h);
                Elem<S>::mma(nu[rt], frag_ld<S>(sA, rt, kc, lane), wb);
                Elem<S>::mma(nr[rt], frag_ld<S>(sAt, rt, kc, lane), wb);
            }
        }
        S *gqh = (S *)((char *)a.ws + lay.off_qhat) + (bh * lay.lp + row0) * D;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            tile_mma_areg_f<S>(qi[t], nu, sX, t, lane);
            store_rows_t<S, D>(gqh, qi[t], 32 * dt, 32 * t + l32, a.scale * kLog2e, lane);  // log2 units
            tile_mma_areg_f<S>(ki[t], nr, sY, t, lane);  // sY holds -Y
            store_frags<S>(recK, ki[t], t * KCH + 2 * dt, lane);
        }
#pragma unroll
        for (int rt2 = 0; rt2 < DT; ++rt2) {
            f32x16 c = {};
            if constexpr (kBf) tile_mma_breg<S, true, SP>(c, sWt, 32 * rt2, nu, lane);
            else tile_mma_breg<S, false, SPD>(c, sW, 32 * rt2, nu, lane);
            store_frags<S>(recM, c, dt * KCH + 2 * rt2, lane);
        }
    }
}

}  // namespace

template <typename S, int D, bool FOX>
static hipError_t launch_prep_t(const PrepArgs &a, hipStream_t st) {
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    dim3 grid((unsigned)(lay.nb * lay.bh));
    hipLaunchKernelGGL((path_prep_kernel<S, D, FOX>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prep_d(const PrepArgs &a, bool bf16, hipStream_t st) {
    const bool fox = a.logf != nullptr;
    if (bf16) return fox ? launch_prep_t<uint16_t, D, true>(a, st) : launch_prep_t<uint16_t, D, false>(a, st);
    return fox ? launch_prep_t<float, D, true>(a, st) : launch_prep_t<float, D, false>(a, st);
}

hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st) {
    if (a.d == 64) return launch_prep_d<64>(a, bf16, st);
    if (a.d == 128) return launch_prep_d<128>(a, bf16, st);
    return hipErrorInvalidValue;
}

}  // namespace path
