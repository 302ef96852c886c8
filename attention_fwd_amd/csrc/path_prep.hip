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

template <typename S>
struct PrepCfg {
    static constexpr bool kBf = sizeof(S) == 2;
    static constexpr int SP = 64 + 16 / (int)sizeof(S);  // padded LDS row stride, elements
    static constexpr int MAT = 64 * SP;
    // matrix slots; bf16 keeps transposed copies of W and A (fp32 has no room
    // for them in 160 KiB of LDS and reads them with a stride instead).  During
    // the triangular solve G (fp32) lives in the UT/RT slots and the solver's
    // columns in the A/Z slots, which are only written after the solve.
    enum { W = 0, Q, K, X, Y, UT, RT, A, Z, AUP, WT };
    static constexpr int NMAT = kBf ? 11 : 9;
    static constexpr int GSTRIDE = 68;  // fp32 row stride of G in the solve layout
};

// Fragment of the matrix view `m` (element (row, k) at row*SP + k when KC, at
// k*SP + row otherwise) for rows `row`, k in [k0, k0+16).
template <typename S, bool KC>
__device__ __forceinline__ typename Elem<S>::Frag lds_frag(const S *mat, int row, int k0, int h) {
    constexpr int SP = PrepCfg<S>::SP;
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

// c += A(m0.., k) * B(n0.., k) over k in [0, K): one 32x32 tile.
template <typename S, bool AKC, bool BKC>
__device__ __forceinline__ void tile_mma(f32x16 &c, const S *A, const S *B, int m0, int n0, int K, int lane) {
    const int h = lane >> 5, l = lane & 31;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        auto a = lds_frag<S, AKC>(A, m0 + l, k0, h);
        auto b = lds_frag<S, BKC>(B, n0 + l, k0, h);
        Elem<S>::mma(c, a, b);
    }
}

// Store a 32x32 accumulator tile (rows m0.., cols n0..) into an LDS matrix,
// optionally transposed, after `f(row, col, value)`.
template <typename S, bool TRANS, typename F>
__device__ __forceinline__ void store_tile(S *mat, const f32x16 &c, int m0, int n0, int lane, F f) {
    constexpr int SP = PrepCfg<S>::SP;
    const int h = lane >> 5, col = n0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = m0 + acc_row(r, h);
        const float v = f(row, col, c[r]);
        if (TRANS)
            mat[col * SP + row] = Elem<S>::from_float(v);
        else
            mat[row * SP + col] = Elem<S>::from_float(v);
    }
}

// Accumulator tile initialised from the transpose of an LDS matrix:
// c(row, col) = mat[col][row] (rows = k index of mat, 4 contiguous per group).
template <typename S>
__device__ __forceinline__ void load_tile_t(f32x16 &c, const S *mat, int m0, int n0, int lane) {
    constexpr int SP = PrepCfg<S>::SP;
    const int h = lane >> 5, col = n0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = Elem<S>::to_f32(mat[col * SP + m0 + acc_row(r, h)]);
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

template <typename S, int D, bool FOX>
__global__ __launch_bounds__(256) void path_prep_kernel(PrepArgs a) {
    static_assert(D == 64, "prep kernel is laid out for head dimension 64");
    typedef PrepCfg<S> C;
    constexpr int SP = C::SP, MAT = C::MAT;
    constexpr int CH = 16 / (int)sizeof(S);  // elements per 16-byte chunk
    __shared__ __attribute__((aligned(16))) S lds[C::NMAT * MAT];
    __shared__ float sBeta[64], sCl[64];

    S *sW = lds + C::W * MAT, *sQ = lds + C::Q * MAT, *sK = lds + C::K * MAT, *sA = lds + C::A * MAT;
    S *sX = lds + C::X * MAT, *sY = lds + C::Y * MAT, *sUt = lds + C::UT * MAT, *sRt = lds + C::RT * MAT;
    S *sZ = lds + C::Z * MAT;
    S *sWt = C::kBf ? lds + C::WT * MAT : nullptr;
    S *sAup = C::kBf ? lds + C::AUP * MAT : nullptr;
    float *sG = (float *)sUt;  // alive only until the solve; UT/RT are written after it
    float *sE = (float *)sA;   // solver columns, alive only during the solve

    const int L = a.L;
    const FwdLayout lay = fwd_layout(a.B, a.H, L, D, sizeof(S));
    const int J = (int)(blockIdx.x % lay.nb);
    const int64_t bh = blockIdx.x / lay.nb;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int64_t row0 = (int64_t)J * kBlk;
    const int nvalid = min(kBlk, L - (int)row0);
    const int64_t tok0 = bh * L + row0;  // first token of the block in [B*H, L]

    // ---- 1. stage W, Q, K (zero rows past L), beta, and the forget-gate prefix
    {
        const S *gq = (const S *)a.q + tok0 * D, *gk = (const S *)a.k + tok0 * D, *gw = (const S *)a.w + tok0 * D;
        for (int idx = tid; idx < 64 * (D / CH); idx += 256) {
            const int r = idx / (D / CH), cc = idx % (D / CH);
            u32x4 vq = {0, 0, 0, 0}, vk = vq, vw = vq;
            if (r < nvalid) {
                vq = *(const u32x4 *)(gq + r * D + cc * CH);
                vk = *(const u32x4 *)(gk + r * D + cc * CH);
                vw = *(const u32x4 *)(gw + r * D + cc * CH);
            }
            *(u32x4 *)(sQ + r * SP + cc * CH) = vq;
            *(u32x4 *)(sK + r * SP + cc * CH) = vk;
            *(u32x4 *)(sW + r * SP + cc * CH) = vw;
            if constexpr (C::kBf) {
                const S *we = (const S *)&vw;
#pragma unroll
                for (int e = 0; e < CH; ++e) sWt[(cc * CH + e) * SP + r] = we[e];
            }
        }
        if (tid < 64) sBeta[tid] = tid < nvalid ? a.beta[tok0 + tid] : 0.f;
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
    __syncthreads();

    const int mt = (wv >> 1) * 32, nt = (wv & 1) * 32;  // this wave's tile of a 64x64 product

    // ---- 2. G = W W^T (fp32, solve layout), X = tril(Q W^T), Y = strictly-upper(K W^T)
    {
        f32x16 c = {};
        tile_mma<S, true, true>(c, sW, sW, mt, nt, D, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = mt + acc_row(r, h), col = nt + l32;
            sG[row * C::GSTRIDE + (col & 3) * 16 + (col >> 2)] = c[r];
        }
        c = f32x16{};
        tile_mma<S, true, true>(c, sQ, sW, mt, nt, D, lane);
        store_tile<S, false>(sX, c, mt, nt, lane, [](int i, int cc, float v) { return cc <= i ? v : 0.f; });
        c = f32x16{};
        tile_mma<S, true, true>(c, sK, sW, mt, nt, D, lane);
        store_tile<S, false>(sY, c, mt, nt, lane, [](int j, int r, float v) { return r > j ? v : 0.f; });
    }
    __syncthreads();

    // ---- 3. A = (I + strictly_lower(D_b G))^-1 D_b by forward substitution.
    // Column t of E = (I + strictly_lower(D_b G))^-1 solves
    //   x_r = [r == t] - beta_r sum_{c<r} G_rc x_c,
    // and A = E D_b.  Thread (t, p) owns column t and the rows c = p (mod 4) of
    // it (its private slice of sE); a row's sum is 16 products per thread plus
    // a 4-lane reduction.  Entries not yet computed are zero, so every row runs
    // the same fixed-length loop.
    {
        const int p = lane & 3, t = 4 * (lane >> 2) + wv;
        float *myE = sE + t * C::GSTRIDE + p * 16;
#pragma unroll
        for (int cc = 0; cc < 16; cc += 4) *(f32x4 *)(myE + cc) = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int r = 0; r < 64; ++r) {
            const float *g = sG + r * C::GSTRIDE + p * 16;
            float part = 0.f;
#pragma unroll
            for (int cc = 0; cc < 16; cc += 4) {
                const f32x4 gv = *(const f32x4 *)(g + cc), ev = *(const f32x4 *)(myE + cc);
                part += gv.x * ev.x + gv.y * ev.y + gv.z * ev.z + gv.w * ev.w;
            }
            part = sum4(part);
            const float x = (r == t) ? 1.f : (r > t ? -sBeta[r] * part : 0.f);
            if (p == (r & 3)) myE[r >> 2] = x;
        }
        float xs[16];
#pragma unroll
        for (int cc = 0; cc < 16; cc += 4) {
            const f32x4 ev = *(const f32x4 *)(myE + cc);
            xs[cc] = ev.x; xs[cc + 1] = ev.y; xs[cc + 2] = ev.z; xs[cc + 3] = ev.w;
        }
        const float bt = sBeta[t];
        __syncthreads();  // sE aliases sA
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            const int c = 4 * cc + p;
            const S v = Elem<S>::from_float(bt * xs[cc]);
            sA[c * SP + t] = v;
            if constexpr (C::kBf) sAup[t * SP + c] = v;
        }
    }
    __syncthreads();

    // ---- 4. UT = -(A W)^T, RT = -(A^T W)^T, Z = -tril(Q W^T) A
    {
        f32x16 c = {};
        if constexpr (C::kBf)
            tile_mma<S, true, true>(c, sA, sWt, mt, nt, 64, lane);
        else
            tile_mma<S, true, false>(c, sA, sW, mt, nt, 64, lane);
        store_tile<S, true>(sUt, c, mt, nt, lane, [](int, int, float v) { return -v; });
        c = f32x16{};
        if constexpr (C::kBf)
            tile_mma<S, true, true>(c, sAup, sWt, mt, nt, 64, lane);
        else
            tile_mma<S, false, false>(c, sA, sW, mt, nt, 64, lane);
        store_tile<S, true>(sRt, c, mt, nt, lane, [](int, int, float v) { return -v; });
        c = f32x16{};
        if constexpr (C::kBf)
            tile_mma<S, true, true>(c, sX, sAup, mt, nt, 64, lane);
        else
            tile_mma<S, true, false>(c, sX, sA, mt, nt, 64, lane);
        store_tile<S, false>(sZ, c, mt, nt, lane, [](int, int, float v) { return -v; });
    }
    __syncthreads();

    S *rec = (S *)((char *)a.ws + lay.off_rec) + (bh * lay.nb + J) * lay.rec_elems;
    S *recK = rec, *recV = rec + 64 * D, *recM = rec + 128 * D;
    constexpr int KCH = D / 16;  // k chunks over the head dimension

    if (wv < 2) {
        // ---- 5a. diagonal block: S^T = K Q^T + Y Z^T (Z already negated), causal softmax, O^T = V^T P^T
        const int ct = wv;                 // query column tile
        const int i = 32 * ct + l32;       // query row in the block
        f32x16 s[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            s[rt] = f32x16{};
            tile_mma<S, true, true>(s[rt], sK, sQ, 32 * rt, 32 * ct, D, lane);
            tile_mma<S, true, true>(s[rt], sY, sZ, 32 * rt, 32 * ct, 64, lane);
        }
        const float c2 = a.scale * kLog2e;
        const float cli = FOX ? sCl[i] : 0.f;
        float mx = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = 32 * rt + acc_row(r, h);
                float x = s[rt][r] * c2;
                if (FOX) x += (cli - sCl[j]) * kLog2e;
                x = j <= i ? x : -INFINITY;
                s[rt][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = other_half_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(s[rt][r] - mx);
                s[rt][r] = p;
                sum += p;
            }
        sum = other_half_sum(sum);
        // V^T fragments: row d = 32 dt + l32, k = key
        const S *gv = (const S *)a.v + tok0 * D;
        f32x16 o[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            auto pf = acc_frag<S>(s[kc >> 1], kc & 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = 16 * kc + frag_k(e, h);
                    x[e] = key < nvalid ? Elem<S>::to_f32(gv[(int64_t)key * D + 32 * dt + l32]) : 0.f;
                }
                auto vf = Elem<S>::from_f32(x);
                Elem<S>::mma(o[dt], vf, pf);
                if (dt == wv) {  // each of the two waves stores half of the V^T record
                    S *dst = recV + ((int64_t)(dt * 4 + kc) * 64 + lane) * 8;
                    *(typename Elem<S>::Frag *)dst = vf;
                }
            }
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
            for (int dt = 0; dt < D / 32; ++dt) store_rows_t<S, D>(go, o[dt], 32 * dt, i, inv, lane);
            if (h == 0 && a.lse) a.lse[tok0 + i] = (mx + __log2f(sum)) * kLn2;
        }
    } else {
        // ---- 5b. key-block record (khat, -M) and qhat
        const int half = wv - 2;
        // khat^T = K^T + RT Y^T  (RT holds -(A^T W)^T): tiles (dt, jt = half)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            f32x16 c;
            load_tile_t<S>(c, sK, 32 * dt, 32 * half, lane);
            tile_mma<S, true, true>(c, sRt, sY, 32 * dt, 32 * half, 64, lane);
            store_frags<S>(recK, c, half * KCH + 2 * dt, lane);
        }
        // (-M)^T = W^T UT^T: tiles (rt over d2, ct = half over d1); fragments of -M with row d1
#pragma unroll
        for (int rt = 0; rt < D / 32; ++rt) {
            f32x16 c = {};
            if constexpr (C::kBf)
                tile_mma<S, true, true>(c, sWt, sUt, 32 * rt, 32 * half, 64, lane);
            else
                tile_mma<S, false, true>(c, sW, sUt, 32 * rt, 32 * half, 64, lane);
            store_frags<S>(recM, c, half * KCH + 2 * rt, lane);
        }
        // qhat^T = Q^T + UT X^T: tiles (dt, it = half)
        S *gqh = (S *)((char *)a.ws + lay.off_qhat) + (bh * lay.lp + row0) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            f32x16 c;
            load_tile_t<S>(c, sQ, 32 * dt, 32 * half, lane);
            tile_mma<S, true, true>(c, sUt, sX, 32 * dt, 32 * half, 64, lane);
            store_rows_t<S, D>(gqh, c, 32 * dt, 32 * half + l32, 1.f, lane);
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

hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st) {
    if (a.d != 64) return hipErrorInvalidValue;
    const bool fox = a.logf != nullptr;
    if (bf16) return fox ? launch_prep_t<uint16_t, 64, true>(a, st) : launch_prep_t<uint16_t, 64, false>(a, st);
    return fox ? launch_prep_t<float, 64, true>(a, st) : launch_prep_t<float, 64, false>(a, st);
}

}  // namespace path
