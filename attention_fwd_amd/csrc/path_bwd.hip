// path_bwd.hip -- backward pass of PaTH attention (gradients of q, k, v, w,
// beta and the log forget gate), gfx950, head dimension 64 or 128.
//
// The pages present the blockwise algorithm (UT transform per block, scan over
// key blocks) as what makes PaTH trainable ("技術要約: PaTH Attention", section 3,
// and "거리에서 경로로, PaTH Attention", section 9) but print no gradient; what is
// computed here is the chain rule applied to the forward's definition
// (summary section 2: s_ij = scale k_j^T H_{j+1} ... H_i q_i, H = I - beta w w^T,
// plus the forget-gate path sum; blog sections 3-4: causal softmax, weighted
// sum of values), organised on the same 64-token blocks as the forward.
//
// Loss: sum do . o + sum dlse . lse, with o and lse the forward's outputs.
//
// Per block J (tokens s..e, local index 0..63), with W the block's w rows and
// B = diag(beta):
//   X = (I + B su(W W^T))^-1 (unit upper triangular), A = X B
//   q^_i = H_s ... H_i q_i      = q_i - (Z W)_i,  Z = (Q W^T o [r <= i]) A^T
//   k^_j = H_e ... H_{j+1} k_j  = k_j - (Y W)_j,  Y = N A,  N = K W^T o [r > j]
//   T_J  = H_s ... H_e          = I - W^T A W                (d x d)
//   diagonal logits  s_ij = scale (Q K^T - Z N^T)_ij + gate,  j <= i
// For query block I and key block J < I the logits are scale q~ . k^ with the
// query carried down q~^(J-1) = T_J q~^(J), q~^(I-1) = q^.  The adjoint of
// q~^(J) obeys G^(J) = G^(J-1) T_J + scale dS_IJ K^_J (rows), running upward
// while q~ runs downward, so the carried queries and adjoints of every pair
// go through the workspace:
//   prep (per block): the quantities above, kept as fp32 64 x 64 matrices for
//     the block backward and as matrix-core fragments for the walks; the
//     diagonal block's dS and value gradient;
//   down walk (per query block I): q~^(J) for J = I-1 .. 0, stored per pair
//     with rows queries and, for fp32 inputs, with rows d (the sums over
//     queries below need the query index inside a lane's fragment; the bf16
//     key walks gather that orientation from an LDS copy with transposing
//     reads);
//   up walk (per query block I): J = 0 .. I-1, the logits, P and dS from the
//     stored q~, the adjoint G, stored per pair (rows d for fp32 inputs, rows
//     queries for bf16, gathered like q~), and dq^_I = G^(I-1);
//   key walk (per key block J): over I > J the logits, P and dS again (from
//     q~, dO, k^, V: recomputing them costs less than moving them), and the
//     sums dV_J += P^T dO_I, dk^_J += scale dS^T q~, dT_J += G^(J-1)^T q~ --
//     owned by one workgroup, so no atomics (bitwise reproducible);
//   block backward (per block): the matrix-form chain rule through the
//     formulas above (including the triangular inverse: dT' = -X^T dX X^T)
//     gives dq, dk, dw, dbeta; dv adds the two value sums; the gate's
//     per-token adjoint dc_t = rowsum_t(dS) - colsum_t(dS);
//   gate: dlogf_t = sum_{t' >= t} dc_t' (one workgroup per head).
// The walks run on the matrix cores in the input's element type (bf16
// products with fp32 accumulation for bf16 inputs, fp32 products for fp32),
// with operands stored in fragment order and the carried q~ and G held as
// fp32 accumulators, rounded to the element type only as product operands,
// as in the forward scan.  The per-block kernels keep 64 x 64 tiles in LDS,
// looping over 64-wide chunks of the head dimension: fp32 tiles and products
// on v_mfma_f32_16x16x4f32 for fp32 inputs; for bf16 inputs tiles held as bf16
// hi + lo pairs (lo = 0 for tiles of input values) and products on
// v_mfma_f32_16x16x32_bf16 (hi*hi + hi*lo + lo*hi).
#include <hip/hip_runtime.h>

#include "path_bwd.h"
#include "path_common.h"

namespace path {
namespace {

constexpr int kC = 64;   // tokens per block
constexpr int kP = 68;   // LDS row stride of a 64x64 fp32 tile: rows 16-byte aligned, columns conflict-free
constexpr int kT = 512;  // threads per workgroup of the per-block kernels (8 waves, two per SIMD)
constexpr int kTile = kC * kP;

// ---------------------------------------------------------------------------
// 64x64 fp32 tiles in LDS (per-block kernels)
// ---------------------------------------------------------------------------

// A 64x64 fp32 matrix in LDS; element (r, c) at p[r * rs + c * cs].
struct LMat {
    const float *p;
    int rs, cs;
};
__device__ __forceinline__ LMat nat(const float *p) { return {p, kP, 1}; }
__device__ __forceinline__ LMat tr(const float *p) { return {p, 1, kP}; }

// acc += A * B for 64x64 operands on v_mfma_f32_16x16x4f32.  Wave w owns rows
// 16 (w >> 1) .. +16 and columns 32 (w & 1) .. +32 of the output as two 16x16
// tiles (accumulator elements 0-3 and 4-7), so all eight waves share every
// product.  The contraction runs in four blocks of sixteen k; in block g, MFMA
// t (0..3) takes k = 16g + 4q + t from lane group q = lane / 16, the same
// order for both operands.  An operand whose k index is contiguous in LDS is
// read with one 16-byte load per four MFMAs; otherwise with four single loads.
__device__ __forceinline__ void mm(f32x8 &acc, LMat A, LMat B, int lane, int wave) {
    const int r = 16 * (wave >> 1) + (lane & 15), c0 = 32 * (wave & 1) + (lane & 15), q = lane >> 4;
    f32x4 lo = acc.lo, hi = acc.hi;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int k0 = 16 * g + 4 * q;
        f32x4 x, y0, y1;
        if (A.cs == 1) {
            x = *reinterpret_cast<const f32x4 *>(A.p + r * A.rs + k0);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) x[t] = A.p[r * A.rs + (k0 + t) * A.cs];
        }
        if (B.rs == 1) {
            y0 = *reinterpret_cast<const f32x4 *>(B.p + c0 * B.cs + k0);
            y1 = *reinterpret_cast<const f32x4 *>(B.p + (c0 + 16) * B.cs + k0);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                y0[t] = B.p[(k0 + t) * B.rs + c0 * B.cs];
                y1[t] = B.p[(k0 + t) * B.rs + (c0 + 16) * B.cs];
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            lo = __builtin_amdgcn_mfma_f32_16x16x4f32(x[t], y0[t], lo, 0, 0, 0);
            hi = __builtin_amdgcn_mfma_f32_16x16x4f32(x[t], y1[t], hi, 0, 0, 0);
        }
    }
    acc.lo = lo;
    acc.hi = hi;
}

// The product of the generic per-block kernels, which serve fp32 inputs (bf16 inputs have the
// split-tile kernels below); EA, EB mark operands that are tiles of input values.
template <typename T, bool EA, bool EB>
__device__ __forceinline__ void mmx(f32x8 &acc, LMat A, LMat B, int lane, int wave) {
    static_assert(sizeof(T) == 4, "bf16 inputs use the split-tile kernels");
    mm(acc, A, B, lane, wave);
}

__device__ __forceinline__ f32x8 zero8() {
    f32x8 z;
#pragma unroll
    for (int v = 0; v < 8; ++v) z[v] = 0.f;
    return z;
}

// Row / column of accumulator element v (0..7) of this lane: a 16x16 MFMA
// tile holds (row, col) = (4 (lane / 16) + i, lane % 16) in register i.
__device__ __forceinline__ int arow(int v, int lane, int wave) { return 16 * (wave >> 1) + 4 * (lane >> 4) + (v & 3); }
__device__ __forceinline__ int acol(int v, int lane, int wave) { return 32 * (wave & 1) + 16 * (v >> 2) + (lane & 15); }

template <typename F>
__device__ __forceinline__ void store_lds(float *buf, const f32x8 &acc, int lane, int wave, F f) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        buf[r * kP + c] = f(r, c, acc[v]);
    }
}
struct Id {
    __device__ float operator()(int, int, float x) const { return x; }
};

// Global fp32 matrix [64 rows][row stride gs] <-> LDS tile.
__device__ __forceinline__ void g2l(float *buf, const float *g, int gs, int tid) {
#pragma unroll
    for (int e = tid; e < kC * kC / 4; e += kT) {
        const int r = e >> 4, c = (e & 15) * 4;
        *reinterpret_cast<f32x4 *>(buf + r * kP + c) = *reinterpret_cast<const f32x4 *>(g + (int64_t)r * gs + c);
    }
}
__device__ __forceinline__ void l2g(float *g, int gs, const float *buf, int tid) {
#pragma unroll
    for (int e = tid; e < kC * kC / 4; e += kT) {
        const int r = e >> 4, c = (e & 15) * 4;
        *reinterpret_cast<f32x4 *>(g + (int64_t)r * gs + c) = *reinterpret_cast<const f32x4 *>(buf + r * kP + c);
    }
}
__device__ __forceinline__ void zero_lds(float *buf, int tid) {
    for (int e = tid; e < kTile; e += kT) buf[e] = 0.f;
}
__device__ __forceinline__ void acc2g(float *g, int gs, const f32x8 &acc, int lane, int wave) {
#pragma unroll
    for (int v = 0; v < 8; ++v) g[(int64_t)arow(v, lane, wave) * gs + acol(v, lane, wave)] = acc[v];
}

// Eight consecutive elements of an input tensor as fp32 (one 16-byte load for
// bf16, two for fp32); the tensors are 16-byte aligned, rows are D elements.
__device__ __forceinline__ void load8(float *x, const uint16_t *g) {
    const u32x4 u = *reinterpret_cast<const u32x4 *>(g);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[2 * t] = __uint_as_float(u[t] << 16);
        x[2 * t + 1] = __uint_as_float(u[t] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(float *x, const float *g) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(g), b = *reinterpret_cast<const f32x4 *>(g + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[t] = a[t];
        x[4 + t] = b[t];
    }
}

// Columns c0 .. c0+63 of input rows [row0, row0 + 64) of one head (rows of D
// elements; rows >= L read as 0) -> LDS fp32; each thread converts eight
// consecutive elements of one row.
template <typename T>
__device__ __forceinline__ void in2l(float *buf, const T *g, int D, int c0, int row0, int L, int tid) {
    const int r = tid >> 3, c = (tid & 7) * 8;  // 512 threads = 64 rows x 8 groups
    float x[8];
    if (row0 + r < L) {
        load8(x, g + (int64_t)(row0 + r) * D + c0 + c);
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = 0.f;
    }
    f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
    *reinterpret_cast<f32x4 *>(buf + r * kP + c) = lo;
    *reinterpret_cast<f32x4 *>(buf + r * kP + c + 4) = hi;
}

__device__ __forceinline__ int64_t pair_index(int I, int J) { return (int64_t)I * (I - 1) / 2 + J; }

// Fragment (row tile rt, k chunk kc) of a fragment set with KC k chunks: 64
// lanes x 8 elements; lane l holds row 32 rt + l % 32, k = 16 kc + frag_k(e, l / 32).
template <typename S>
__device__ __forceinline__ typename Elem<S>::Frag ldfrag(const S *base, int rt, int kc, int KC, int lane) {
    return *reinterpret_cast<const typename Elem<S>::Frag *>(base + ((int64_t)(rt * KC + kc) * 64 + lane) * 8);
}
template <typename S>
__device__ __forceinline__ void stfrag(S *base, int rt, int kc, int KC, int lane, const typename Elem<S>::Frag &f) {
    *reinterpret_cast<typename Elem<S>::Frag *>(base + ((int64_t)(rt * KC + kc) * 64 + lane) * 8) = f;
}

// A 64x64 block of a matrix X (fp32 LDS tile) -> the 2 x 4 fragments of X it
// covers, one (fragment, lane) per thread.  TRANS false: X rows are the tile's
// rows and X's k the tile's columns; TRANS true: the transpose.  (rt0, kc0) is
// the block's first fragment in X's fragment set of KC k chunks.
template <typename S, bool TRANS>
__device__ __forceinline__ void tile2frag(S *dst, int KC, int rt0, int kc0, const float *buf, int tid) {
    const int f = tid >> 6, lane = tid & 63, rtl = f >> 2, kcl = f & 3, h = lane >> 5;
    const int row = 32 * rtl + (lane & 31);
    float x[8];
    if constexpr (!TRANS) {
        const float *p = buf + row * kP + 16 * kcl + 4 * h;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(p), hi = *reinterpret_cast<const f32x4 *>(p + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = lo[e];
            x[4 + e] = hi[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = buf[(16 * kcl + frag_k(e, h)) * kP + row];
    }
    stfrag<S>(dst, rt0 + rtl, kc0 + kcl, KC, lane, Elem<S>::from_f32(x));
}

// X = (I + diag(beta) su(G))^-1, unit upper triangular, in 16 x 16 blocks (512 threads).
// With N = diag(beta) su(G) and U = I + N: the diagonal blocks X_II = (I + N_II)^-1 by back
// substitution, one wave per block, then the blocks above the diagonal by distance from it,
// one block per wave and level: U X = I gives X_IJ = -X_II T, T = sum_{K=I+1}^{J} N_IK X_KJ,
// N_IK = diag(beta_I) G_IK (every entry of a block right of the diagonal is above it).
// Blocks below the diagonal are zero.  The caller synchronises before X is read.
__device__ __forceinline__ void unit_upper_inverse(float *X, const float *G, const float *beta, int tid) {
    const int wv = tid >> 6, lane = tid & 63;
    // zero the six blocks below the diagonal: 1536 entries, three per thread
#pragma unroll
    for (int e = tid; e < 6 * 256; e += kT) {
        const int blk = e >> 8, I = blk < 1 ? 1 : (blk < 3 ? 2 : 3), Jb = blk < 1 ? 0 : (blk < 3 ? blk - 1 : blk - 3);
        X[(16 * I + ((e >> 4) & 15)) * kP + 16 * Jb + (e & 15)] = 0.f;
    }
    // (a) diagonal blocks, one per wave: column t of the block, rows r = 4 q + p held by lane
    //     (t, p); x_r = [r == t] - beta_r sum_{t' > r} G_rt' x_t' (entries not yet known are 0)
    if (wv < 4) {
        const int I16 = 16 * wv, t = lane >> 2, p = lane & 3;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
        // the G entries and betas a step uses do not depend on the chain: read PF steps ahead
        constexpr int PF = 3;
        float gv[PF][4], bv[PF];
        auto fetch = [&](int r, int slot) {
#pragma unroll
            for (int q = 0; q < 4; ++q) gv[slot][q] = G[(I16 + r) * kP + I16 + 4 * q + p];
            bv[slot] = beta[I16 + r];
        };
#pragma unroll
        for (int k = 0; k < PF; ++k) fetch(15 - k, k);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int r = 15 - k, sl = k % PF;
            float part = (gv[sl][0] * xs[0] + gv[sl][1] * xs[1]) + (gv[sl][2] * xs[2] + gv[sl][3] * xs[3]);
            const float br = bv[sl];
            if (k + PF < 16) fetch(15 - k - PF, sl);
            part = sum4(part);
            const float x = (r == t) ? 1.f : (r < t ? -br * part : 0.f);
            xs[r >> 2] = (p == (r & 3)) ? x : xs[r >> 2];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) X[(I16 + 4 * q + p) * kP + I16 + t] = xs[q];
    }
    // (b) blocks above the diagonal as 16x16x4 fp32 matrix-core products.  With the k order
    //     k(s, g) = 4 g + s (lane group g = lane / 16 supplies k = 4 g + s at step s), register s
    //     of a 16 x 16 accumulator (rows 4 g .. 4 g + 3, column lane % 16) is the B operand of step
    //     s, so T feeds the second product from registers.
    const int i16 = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
        __syncthreads();
        if (wv < 4 - lev) {
            const int Ib = wv, Jb = wv + lev;
            f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
            for (int K = Ib + 1; K <= Jb; ++K) {
                const f32x4 ga = *reinterpret_cast<const f32x4 *>(G + (16 * Ib + i16) * kP + 16 * K + g4);
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    tacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[st], X[(16 * K + g4 + st) * kP + 16 * Jb + i16], tacc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) tacc[r] *= beta[16 * Ib + g4 + r];
            const f32x4 xa = *reinterpret_cast<const f32x4 *>(X + (16 * Ib + i16) * kP + 16 * Ib + g4);
            f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) e = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[st], tacc[st], e, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) X[(16 * Ib + g4 + r) * kP + 16 * Jb + i16] = -e[r];
        }
    }
}

// Block-local gate prefix sums (inclusive) of one block: cl[i] for its 64 rows.
__device__ __forceinline__ void gate_prefix(float *cl, const float *logf, int row0, int L, int tid) {
    if (tid == 0) {
        float c = 0.f;
        for (int i = 0; i < kC; ++i) {
            c += (logf && row0 + i < L) ? logf[row0 + i] : 0.f;
            cl[i] = c;
        }
    }
}

// ---------------------------------------------------------------------------
// Prep: one workgroup per (block J, head); fp32 inputs (bf16: bwd_prep_kernel_bf16).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kT) void bwd_prep_kernel(BwdArgs a) {
    constexpr int NCH = D / 64, KCD = D / 16;
    typedef T S;  // fragments are kept in the input's element type
    __shared__ __attribute__((aligned(16))) float sm[9 * kTile + 4 * kC];
    float *bW = sm, *bQ = bW + kTile, *bK = bQ + kTile, *bG = bK + kTile, *bA = bG + kTile, *bQW = bA + kTile,
          *bN = bQW + kTile, *bZ = bN + kTile, *bY = bZ + kTile;
    float *sB = bY + kTile, *sCl = sB + kC, *sL2 = sCl + kC, *sDD = sL2 + kC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * D, *k = (const T *)a.k + hoff * D, *w = (const T *)a.w + hoff * D;
    const T *v = (const T *)a.v + hoff * D, *o = (const T *)a.out + hoff * D, *dout = (const T *)a.dout + hoff * D;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float scale = a.scale;
    const int64_t tok = (int64_t)J * kC * kC;

    if (tid < kC) {
        const int i = row0 + tid;
        sB[tid] = i < L ? a.beta[hoff + i] : 0.f;
        sL2[tid] = i < L ? a.lse[hoff + i] * kLog2e : 0.f;
    }
    gate_prefix(sCl, a.logf ? a.logf + hoff : nullptr, row0, L, tid);
    {   // D_i = do_i . o_i - dlse_i: eight lanes per row, D / 8 columns each
        const int r = tid >> 3, c0 = (tid & 7) * (D / 8), i = row0 + r;
        float s = 0.f;
        if (i < L) {
#pragma unroll
            for (int c = 0; c < D / 8; c += 8) {
                float xo[8], xd[8];
                load8(xd, dout + (int64_t)i * D + c0 + c);
                load8(xo, o + (int64_t)i * D + c0 + c);
#pragma unroll
                for (int t = 0; t < 8; ++t) s += xd[t] * xo[t];
            }
        }
        s = sum8(s);
        if ((tid & 7) == 0) sDD[r] = i < L ? s - (a.dlse ? a.dlse[hoff + i] : 0.f) : 0.f;
    }
    // G = W W^T, Q W^T, N = K W^T and Q K^T, summed over the chunks of the head dimension
    f32x8 aG = zero8(), aQW = zero8(), aN = zero8(), aQK = zero8();
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        in2l(bW, w, D, 64 * c, row0, L, tid);
        in2l(bQ, q, D, 64 * c, row0, L, tid);
        in2l(bK, k, D, 64 * c, row0, L, tid);
        __syncthreads();
        mmx<T, true, true>(aG, nat(bW), tr(bW), lane, wave);
        mmx<T, true, true>(aQW, nat(bQ), tr(bW), lane, wave);
        mmx<T, true, true>(aN, nat(bK), tr(bW), lane, wave);
        mmx<T, true, true>(aQK, nat(bQ), tr(bK), lane, wave);
    }
    store_lds(bG, aG, lane, wave, Id());
    store_lds(bQW, aQW, lane, wave, [](int r, int c, float x) { return c <= r ? x : 0.f; });  // Q W^T, r <= i
    store_lds(bN, aN, lane, wave, [](int r, int c, float x) { return c > r ? x : 0.f; });     // N, r > j
    __syncthreads();
    unit_upper_inverse(bA, bG, sB, tid);
    l2g((float *)(ws + ly.qwm) + tok, kC, bQW, tid);
    l2g((float *)(ws + ly.nn) + tok, kC, bN, tid);
    __syncthreads();
    {
        float *XX = (float *)(ws + ly.xx) + tok, *AA = (float *)(ws + ly.aa) + tok;
#pragma unroll
        for (int e = tid; e < kC * kC / 4; e += kT) {  // keep X, then A = X diag(beta) in place
            const int r = e >> 4, c = (e & 15) * 4;
            f32x4 x = *reinterpret_cast<const f32x4 *>(bA + r * kP + c);
            *reinterpret_cast<f32x4 *>(XX + r * kC + c) = x;
            x[0] *= sB[c]; x[1] *= sB[c + 1]; x[2] *= sB[c + 2]; x[3] *= sB[c + 3];
            *reinterpret_cast<f32x4 *>(bA + r * kP + c) = x;
            *reinterpret_cast<f32x4 *>(AA + r * kC + c) = x;
        }
    }
    __syncthreads();
    f32x8 acc = zero8();
    mmx<T, false, false>(acc, nat(bQW), tr(bA), lane, wave);  // Z = QWm A^T
    store_lds(bZ, acc, lane, wave, Id());
    acc = zero8();
    mmx<T, false, false>(acc, nat(bN), nat(bA), lane, wave);  // Y = N A
    store_lds(bY, acc, lane, wave, Id());
    __syncthreads();
    l2g((float *)(ws + ly.zz) + tok, kC, bZ, tid);
    // diagonal block: P = exp(scale (Q K^T - Z N^T) + cl_i - cl_j - lse_i) for j <= i  (G is dead: P -> bG)
    {
        f32x8 sZN = zero8();
        mmx<T, false, false>(sZN, nat(bZ), tr(bN), lane, wave);
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            const float s = (scale * (aQK[vv] - sZN[vv]) + (sCl[r] - sCl[c])) * kLog2e - sL2[r];
            bG[r * kP + c] = c <= r ? fast_exp2(s) : 0.f;
        }
    }
    // dP = dO V^T over the chunks; dS = P (dP - D_i) -> bQW (Q W^T is stored)
    f32x8 aDP = zero8();
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        in2l(bQ, dout, D, 64 * c, row0, L, tid);
        in2l(bK, v, D, 64 * c, row0, L, tid);
        __syncthreads();
        mmx<T, true, true>(aDP, nat(bQ), tr(bK), lane, wave);
    }
    store_lds(bQW, aDP, lane, wave, [&](int r, int c, float x) { return bG[r * kP + c] * (x - sDD[r]); });
    __syncthreads();
    {
        float *EE = (float *)(ws + ly.ee) + tok;
        for (int e = tid; e < kC * kC; e += kT) EE[e] = scale * bQW[(e >> 6) * kP + (e & 63)];
        float *rs = (float *)(ws + ly.rsd) + row0, *cs = (float *)(ws + ly.csd) + row0;
        if (tid < kC) {
            float s = 0.f;
            for (int c = 0; c < kC; ++c) s += bQW[tid * kP + c];
            rs[tid] = s;
        } else if (tid < 2 * kC) {
            const int c = tid - kC;
            float s = 0.f;
            for (int r = 0; r < kC; ++r) s += bQW[r * kP + c];
            cs[c] = s;
        } else if (tid < 3 * kC) {
            const int r = tid - 2 * kC;
            ((float *)(ws + ly.dd))[row0 + r] = sDD[r];
            ((float *)(ws + ly.cql))[row0 + r] = sCl[r] * kLog2e - sL2[r];
            ((float *)(ws + ly.ckl))[row0 + r] = (sCl[kC - 1] - sCl[r]) * kLog2e;
            if (r == 0) ((float *)(ws + ly.tot))[J] = sCl[kC - 1] * kLog2e;
        }
    }
    // chunks of the head dimension: q^, k^ (fragments), A W (kept for T), V and dO fragments,
    // the diagonal value gradient
    const int64_t fo = (int64_t)J * kC * D;  // this block's 64 x D fragment set
    S *REC = (S *)(ws + ly.urec) + J * ly.rec_elems;
    S *KH1 = REC, *V1 = REC + kC * D, *KH2 = REC + 2 * kC * D;
    S *DO1 = (S *)(ws + ly.do1) + fo, *DO2 = (S *)(ws + ly.do2) + fo;
    float *bAW[2] = {bN, bQW};  // A W of chunk 0 / 1 (N and dS are done with)
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        in2l(bW, w, D, 64 * c, row0, L, tid);
        in2l(bQ, q, D, 64 * c, row0, L, tid);
        in2l(bK, k, D, 64 * c, row0, L, tid);
        __syncthreads();
        {
            f32x8 zw = zero8(), yw = zero8(), aw = zero8();
            mmx<T, false, true>(zw, nat(bZ), nat(bW), lane, wave);
            mmx<T, false, true>(yw, nat(bY), nat(bW), lane, wave);
            mmx<T, false, true>(aw, nat(bA), nat(bW), lane, wave);
            float *QH = (float *)(ws + ly.qh) + (int64_t)row0 * D + 64 * c;
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) {  // each element read and rewritten by the same thread
                const int r = arow(vv, lane, wave), cc = acol(vv, lane, wave);
                QH[(int64_t)r * D + cc] = bQ[r * kP + cc] - zw[vv];  // q^ = q - Z W
                bK[r * kP + cc] -= yw[vv];                            // k^ = k - Y W
            }
            store_lds(bAW[c], aw, lane, wave, Id());
        }
        __syncthreads();
        tile2frag<S, false>(KH1, KCD, 0, 4 * c, bK, tid);  // k^: rows keys, k over d
        tile2frag<S, true>(KH2, 4, 2 * c, 0, bK, tid);     // k^^T: rows d, k over keys
        __syncthreads();
        in2l(bQ, v, D, 64 * c, row0, L, tid);
        in2l(bK, dout, D, 64 * c, row0, L, tid);
        __syncthreads();
        tile2frag<S, false>(V1, KCD, 0, 4 * c, bQ, tid);   // V: rows keys
        tile2frag<S, false>(DO1, KCD, 0, 4 * c, bK, tid);  // dO: rows queries
        if constexpr (sizeof(S) == 4) tile2frag<S, true>(DO2, 4, 2 * c, 0, bK, tid);  // dO^T: rows d (fp32 only)
        acc = zero8();
        mmx<T, false, true>(acc, tr(bG), nat(bK), lane, wave);  // diagonal value gradient P^T dO
        acc2g((float *)(ws + ly.dvd) + (int64_t)row0 * D + 64 * c, D, acc, lane, wave);
    }
    // T - I = -W^T (A W) and its transpose, block (c1, c2) = rows of chunk c1, columns of chunk c2
    S *NT = (S *)(ws + ly.nt) + (int64_t)J * D * D, *NTT = REC + 3 * kC * D;
    for (int c1 = 0; c1 < NCH; ++c1) {
        __syncthreads();
        in2l(bW, w, D, 64 * c1, row0, L, tid);
        __syncthreads();
        for (int c2 = 0; c2 < NCH; ++c2) {
            acc = zero8();
            mmx<T, true, false>(acc, tr(bW), nat(bAW[c2]), lane, wave);
            store_lds(bQ, acc, lane, wave, [](int, int, float x) { return -x; });
            __syncthreads();
            tile2frag<S, false>(NT, KCD, 2 * c1, 4 * c2, bQ, tid);  // (T - I): rows d_out, k over d_in
            tile2frag<S, true>(NTT, KCD, 2 * c2, 4 * c1, bQ, tid);  // (T - I)^T
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// The walks: two waves per query block (down and up walks), each owning 32 of
// its queries; matrix-core operands are fragments loaded from the workspace.
// ---------------------------------------------------------------------------

// Per-wave LDS scratch of the generic (fp32) walks for writing an accumulator tile set
// (rows d, columns the wave's 32 queries) back as fragments with the query index inside
// the lane.
template <typename S>
struct XScr {
    static_assert(sizeof(S) == 4, "the generic walks serve fp32 inputs");
    static constexpr int kStride = 36;  // row stride (elements): rows 16-byte aligned
};

// acc tiles t[dt] (rows d = 32 dt + acc_row(r, h), columns this wave's 32 queries) ->
// fragments (rt = dt, kc = 2 w + 0/1) of a set with rows d and k over the block's 64 queries.
// Only this wave touches x, and a wave's LDS accesses are performed in order.
template <typename S, int D>
__device__ __forceinline__ void store_transposed(S *dst, const f32x16 *t, S *x, int w, int lane) {
    constexpr int XS = XScr<S>::kStride;
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(32 * dt + acc_row(r, h)) * XS + l32] = Elem<S>::from_float(t[dt][r]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int kcl = 0; kcl < 2; ++kcl) {
            const S *src = x + (32 * dt + l32) * XS + 16 * kcl + 4 * h;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(src), hi = *reinterpret_cast<const f32x4 *>(src + 8);
            const float y[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            stfrag<S>(dst, dt, 2 * w + kcl, 4, lane, Elem<S>::from_f32(y));
        }
}

// Down walk (fp32 inputs; bf16: bwd_down_kernel_lds): one workgroup (two waves) per
// (query block I >= 1, head), heaviest first.  q~^T (rows d, the wave's 32 queries) stays in fp32 accumulators:
// q~^T <- q~^T + (T_J - I) q~^T; q~^(J) is stored for the pair (I, J) with rows
// queries (for the logits) and, with Q2, with rows d (for the key walk's sums
// over queries), with the gate sum of the blocks strictly between I and J.
template <typename S, int D, bool Q2>
__global__ __launch_bounds__(128) void bwd_down_kernel(BwdArgs a) {
    typedef typename Elem<S>::Frag Frag;
    constexpr int KCD = D / 16, RTD = D / 32;
    __shared__ __attribute__((aligned(16))) S sx[2][D * XScr<S>::kStride];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, I = nb - 1 - blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *NT = (const S *)(ws + ly.nt);
    const float *tot = (const float *)(ws + ly.tot);
    float *MID = (float *)(ws + ly.mid);
    S *QS1 = (S *)(ws + ly.qs1), *QS2 = (S *)(ws + ly.qs2);
    const int row0 = I * kC;

    f32x16 qt[RTD];
    {
        const float *qh = (const float *)(ws + ly.qh) + (int64_t)(row0 + 32 * w + l32) * D;
#pragma unroll
        for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(qh + 32 * dt + 8 * g4 + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) qt[dt][4 * g4 + e] = x[e];
            }
    }
    float mid = 0.f;
    if (tid == 0) MID[pair_index(I, I - 1)] = 0.f;
    for (int J = I - 1; J >= 0; --J) {
        const int64_t p = pair_index(I, J);
        Frag qf[KCD];
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) qf[kc] = acc_frag<S>(qt[kc >> 1], kc & 1);
        S *q1 = QS1 + p * kC * D;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) stfrag<S>(q1, w, kc, KCD, lane, qf[kc]);
        if constexpr (Q2) store_transposed<S, D>(QS2 + p * kC * D, qt, sx[w], w, lane);
        if (J >= 1) {
            const S *nt = NT + (int64_t)J * D * D;
#pragma unroll
            for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) Elem<S>::mma(qt[dt], ldfrag<S>(nt, dt, kc, KCD, lane), qf[kc]);
            mid += tot[J];
            if (tid == 0) MID[pair_index(I, J - 1)] = mid;
        }
    }
}

// Up walk (fp32 inputs; bf16: bwd_up_kernel_lds, bwd_up_kernel_split): one workgroup
// (two waves) per (query block I >= 1, head), heaviest
// first.  For J = 0 .. I-1: S^T = K^_J q~^T and dP^T = V_J dO^T (rows keys,
// columns the wave's queries), P and dS, then the adjoint (rows d, fp32
// accumulators) G^T <- G^T + (T_J - I)^T G^T + K^_J^T (scale dS^T).  G^(J) is
// stored with rows d for the pair (I, J + 1); G^(I-1) = dq^_I.
template <typename S, int D>
__global__ __launch_bounds__(128) void bwd_up_kernel(BwdArgs a) {
    typedef typename Elem<S>::Frag Frag;
    constexpr int KCD = D / 16, RTD = D / 32;
    __shared__ __attribute__((aligned(16))) S sx[2][D * XScr<S>::kStride];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, I = nb - 1 - blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *RECS = (const S *)(ws + ly.urec), *QS1 = (const S *)(ws + ly.qs1);
    const int64_t RE = ly.rec_elems;
    S *GS2 = (S *)(ws + ly.gs2);
    const float *MID = (const float *)(ws + ly.mid), *CKK = (const float *)(ws + ly.ckl);
    const float scale = a.scale, c2 = scale * kLog2e;
    const int row0 = I * kC, qi = row0 + 32 * w + l32;  // this lane's query (column of the accumulators)
    const float dd = ((const float *)(ws + ly.dd))[qi], cq = ((const float *)(ws + ly.cql))[qi];

    Frag dof[KCD];  // dO with k over d, lane <-> query: the B operand of dP^T
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc)
        dof[kc] = ldfrag<S>((const S *)(ws + ly.do1) + (int64_t)I * kC * D, w, kc, KCD, lane);
    f32x16 gt[RTD];
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt) gt[dt] = f32x16{};
    float rsum = 0.f;
    if constexpr (D == 64) {
    // A step loads k^ and V of block J with the stored q~ at its top (q~ one step ahead),
    // and the operands of the adjoint update while the logits are computed.
    Frag qf[KCD];
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc) qf[kc] = ldfrag<S>(QS1 + pair_index(I, 0) * kC * D, w, kc, KCD, lane);
    for (int J = 0; J < I; ++J) {
        const int64_t p = pair_index(I, J);
        const S *rec = RECS + J * RE;  // k^, V, k^^T, (T - I)^T of block J
        Frag kf[2][KCD], vf[2][KCD];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) {
                kf[kt][kc] = ldfrag<S>(rec, kt, kc, KCD, lane);
                vf[kt][kc] = ldfrag<S>(rec + kC * D, kt, kc, KCD, lane);
            }
        const float mid = MID[p];
        f32x4 ck[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                ck[kt][g4] = *reinterpret_cast<const f32x4 *>(CKK + J * kC + 32 * kt + 8 * g4 + 4 * h);
        Frag qn[KCD];
        if (J + 1 < I) {
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) qn[kc] = ldfrag<S>(QS1 + (p + 1) * kC * D, w, kc, KCD, lane);
        }
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
            dp[kt] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) {
                Elem<S>::mma(s[kt], kf[kt][kc], qf[kc]);
                Elem<S>::mma(dp[kt], vf[kt][kc], dof[kc]);
            }
        }
        const S *ntt = rec + 3 * kC * D;
        Frag tf[RTD][KCD], k2[RTD][4];
#pragma unroll
        for (int dt = 0; dt < RTD; ++dt) {
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) tf[dt][kc] = J >= 1 ? ldfrag<S>(ntt, dt, kc, KCD, lane) : Frag{};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) k2[dt][kc] = ldfrag<S>(rec + 2 * kC * D, dt, kc, 4, lane);
        }
        // P^T and scale dS^T (rows: keys 32 kt + acc_row(r, h); column: this lane's query)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g4 + e;
                    const float P = fast_exp2(c2 * s[kt][r] + cq + ck[kt][g4][e] + mid);
                    const float ds = P * (dp[kt][r] - dd);
                    rsum += ds;
                    s[kt][r] = scale * ds;
                }
        Frag gf[KCD], sf[4];
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) gf[kc] = acc_frag<S>(gt[kc >> 1], kc & 1);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) sf[kc] = acc_frag<S>(s[kc >> 1], kc & 1);
#pragma unroll
        for (int dt = 0; dt < RTD; ++dt) {
            if (J >= 1) {
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) Elem<S>::mma(gt[dt], tf[dt][kc], gf[kc]);
            }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(gt[dt], k2[dt][kc], sf[kc]);
        }
        if (J + 1 < I) {
            store_transposed<S, D>(GS2 + pair_index(I, J + 1) * kC * D, gt, sx[w], w, lane);
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) qf[kc] = qn[kc];
        }
    }
    } else {
    // (d = 128: a step's operands do not fit the registers at once; each is loaded where it is used)
    for (int J = 0; J < I; ++J) {
        const int64_t p = pair_index(I, J);
        const S *rec = RECS + J * RE;  // k^, V, k^^T, (T - I)^T of block J
        const float mid = MID[p];
        Frag qf[KCD];
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) qf[kc] = ldfrag<S>(QS1 + p * kC * D, w, kc, KCD, lane);
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
            dp[kt] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) {
                Elem<S>::mma(s[kt], ldfrag<S>(rec, kt, kc, KCD, lane), qf[kc]);
                Elem<S>::mma(dp[kt], ldfrag<S>(rec + kC * D, kt, kc, KCD, lane), dof[kc]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 ck = *reinterpret_cast<const f32x4 *>(CKK + J * kC + 32 * kt + 8 * g4 + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g4 + e;
                    const float P = fast_exp2(c2 * s[kt][r] + cq + ck[e] + mid);
                    const float ds = P * (dp[kt][r] - dd);
                    rsum += ds;
                    s[kt][r] = scale * ds;
                }
            }
        Frag gf[KCD], sf[4];
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) gf[kc] = acc_frag<S>(gt[kc >> 1], kc & 1);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) sf[kc] = acc_frag<S>(s[kc >> 1], kc & 1);
        const S *ntt = rec + 3 * kC * D;
#pragma unroll
        for (int dt = 0; dt < RTD; ++dt) {
            if (J >= 1) {
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) Elem<S>::mma(gt[dt], ldfrag<S>(ntt, dt, kc, KCD, lane), gf[kc]);
            }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(gt[dt], ldfrag<S>(rec + 2 * kC * D, dt, kc, 4, lane), sf[kc]);
        }
        if (J + 1 < I) store_transposed<S, D>(GS2 + pair_index(I, J + 1) * kC * D, gt, sx[w], w, lane);
    }
    }
    rsum = other_half_sum(rsum);  // lanes l and l ^ 32 hold the other keys of the same query
    float *dqo = (float *)(ws + ly.dqo) + (int64_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = {gt[dt][4 * g4], gt[dt][4 * g4 + 1], gt[dt][4 * g4 + 2], gt[dt][4 * g4 + 3]};
            *reinterpret_cast<f32x4 *>(dqo + 32 * dt + 8 * g4 + 4 * h) = x;
        }
    if (h == 0) ((float *)(ws + ly.rso))[qi] = rsum;
}

// Shared by the LDS-staged walks below.
constexpr int kUpQB = 4;  // query blocks per workgroup
typedef __attribute__((address_space(3))) void lds_void;

// Work item of a walk launch with nu units (query tiles or key blocks) per head over hc
// heads, for a kernel that keeps wpc workgroups on a compute unit.  Workgroups are dealt
// round-robin over gfx950's 8 XCDs, each with its own L2 and 32 compute units: the items
// are numbered XCD by XCD, so that every XCD takes a contiguous range of heads, in groups
// of about one round of its workgroup slots.  Inside a group, rank r (0: the longest walk)
// runs on every head of the group before rank r + 1, so the group's walks read the same
// key or query blocks at about the same time and share them through the XCD's L2.
// Returns the head (gl) and the rank (r).
constexpr int kXcds = 8, kCusPerXcd = 32;
__device__ __forceinline__ void walk_item(int nu, int hc, int wpc, int &gl, int &r) {
    // the grid (nu hc workgroups) is below 2^31, so 32-bit arithmetic suffices
    const unsigned total = (unsigned)nu * (unsigned)hc, x = blockIdx.x;
    const unsigned q = total / kXcds, rem = total % kXcds, k = x % kXcds;
    const unsigned item = k * q + min(k, rem) + x / kXcds;  // XCD k holds items [k q + min(k, rem), ...)
    const unsigned G = (unsigned)max(1, kCusPerXcd * wpc / nu);
    const unsigned gbase = item / (G * (unsigned)nu) * G;  // first head of the item's group
    const unsigned gn = min(G, (unsigned)hc - gbase);
    const unsigned rank = item - gbase * (unsigned)nu;
    gl = (int)(gbase + rank % gn);
    r = (int)(rank / gn);
}

// Copy NLD 16-byte chunks per thread of a contiguous record into LDS (lane l of a wave
// lands at the wave's LDS base + 16 l); completion is tracked by vmcnt.
template <int NTH, int NLD>
__device__ __forceinline__ void dma_record(const void *src, void *dst, int tid) {
    const int wv = tid >> 6;
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
        const char *g = (const char *)src + (size_t)t * NTH * 16 + 16 * tid;
        char *l = (char *)dst + (size_t)t * NTH * 16 + 1024 * wv;
        __builtin_amdgcn_global_load_lds((const void *)g, (lds_void *)l, 16, 0, 0);
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14,
// expcnt left at its maximum): at most n vector-memory operations outstanding and every
// LDS access of the wave returned.
constexpr int vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// Down walk for bf16 inputs: as bwd_down_kernel (without the q~^T copy), but four query
// blocks (eight waves, two per block) share each key block's transition T - I (8 KiB at
// d = 64, 32 KiB at d = 128), copied global -> LDS one step ahead (global_load_lds,
// double-buffered), as in the up walk below.  The tile walks J = Imax - 1 .. 0; a wave
// joins at J = I - 1.  Every step issues the same memory operations on every wave (the
// next copy, the next gate total, the stores of q~ and of the gate sum, to a spare target
// when the wave has nothing to store), so that one wait at the top of a step covers every
// path.
template <int D>
__global__ __launch_bounds__(64 * 2 * kUpQB) void bwd_down_kernel_lds(BwdArgs a) {
    typedef uint16_t S;
    typedef Elem<S>::Frag Frag;
    constexpr int KCD = D / 16, RTD = D / 32, NTH = 64 * 2 * kUpQB;
    constexpr int REC = D * D;               // elements of a transition
    constexpr int NLD = REC * 2 / 16 / NTH;  // DMA chunks per thread and transition
    static_assert(REC * 2 % (16 * NTH) == 0, "transition must split evenly over the workgroup");
    constexpr int NST = KCD + 1;  // global stores of one step: the q~ fragments and the gate sum
    constexpr int BUF = REC * 2;  // bytes per buffer
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int nb = a.nb, hc = a.hc;
    const int ntile = (nb - 1 + kUpQB - 1) / kUpQB;  // query blocks 1 .. nb-1, four per tile
    int gl, tile;
    walk_item(ntile, hc, 2, gl, tile);
    tile = ntile - 1 - tile;
    const int I0 = 1 + kUpQB * tile, Imax = min(nb - 1, I0 + kUpQB - 1);
    const int I = __builtin_amdgcn_readfirstlane(I0 + (w >> 1)), wq = __builtin_amdgcn_readfirstlane(w & 1);
    const bool active = I <= nb - 1;
    const int Ic = active ? I : Imax;  // idle waves carry a valid block and discard it
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *NT = (const S *)(ws + ly.nt);
    const float *tot = (const float *)(ws + ly.tot);
    float *MID = (float *)(ws + ly.mid);
    S *QS1 = (S *)(ws + ly.qs1);
    // the spare fragment set after the last pair's G (written before the up walk fills it)
    S *const spare = (S *)(ws + ly.gs2) + (int64_t)nb * (nb - 1) / 2 * kC * D;
    float *const mspare = (float *)spare;

    auto issue = [&](int J, int B) { dma_record<NTH, NLD>(NT + (int64_t)J * REC, smem + B * BUF, tid); };
    const int Jtop = Imax - 1;
    issue(Jtop, 0);
    f32x16 qt[RTD];
    {
        const float *qh = (const float *)(ws + ly.qh) + (int64_t)(Ic * kC + 32 * wq + l32) * D;
#pragma unroll
        for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(qh + 32 * dt + 8 * g4 + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) qt[dt][4 * g4 + e] = x[e];
            }
    }
    float tcur = tot[Jtop];  // gate total of the step's key block, loaded one step ahead
    float mid = 0.f;         // gate sum over the blocks strictly between I and the step's J
    asm volatile("" ::: "memory");  // the wait below stays after these loads
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
    auto step = [&](int J, auto bsel) {
        constexpr int B = decltype(bsel)::value;
        const S *nt = (const S *)(smem + B * BUF);
        // this wave's copy of T_J - I and its gate-total load have landed (only the previous
        // step's stores may still be in flight); after the barrier every wave's copies have
        // landed and every wave is done with the other buffer
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(NST));
        asm volatile("s_barrier" ::: "memory");
        issue(max(J - 1, 0), 1 - B);
        const float tnext = tot[max(J - 1, 0)];
        asm volatile("" ::: "memory");  // the loads stay ahead of this step's stores
        const bool act = active && J <= I - 1;
        Frag qf[KCD];
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) qf[kc] = acc_frag<S>(qt[kc >> 1], kc & 1);
        S *dst = act ? QS1 + pair_index(I, J) * kC * D : spare;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) stfrag<S>(dst, wq, kc, KCD, lane, qf[kc]);
        // every lane stores the same value (one store instruction, no branch)
        *((act && wq == 0) ? MID + pair_index(I, J) : mspare) = mid;
        if (act && J >= 1) {
#pragma unroll
            for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) Elem<S>::mma(qt[dt], ldfrag<S>(nt, dt, kc, KCD, lane), qf[kc]);
        }
        if (act) mid += tcur;
        tcur = tnext;
    };
    for (int J = Jtop; J >= 0; J -= 2) {
        step(J, std::integral_constant<int, 0>{});
        if (J >= 1) step(J - 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));  // no copy may still be landing in LDS when the workgroup leaves
}

// Up walk for bf16 inputs at head dimension 64: as bwd_up_kernel, but four query
// blocks (eight waves, two per block) share each key block's record (k^, V, k^^T,
// (T - I)^T: 32 KiB), which is copied global -> LDS one step ahead by the DMA path
// (global_load_lds, double-buffered), as in the forward scan; each wave prefetches its
// next stored q~ into registers.  G^(J-1) is stored for the pair (I, J) with rows
// queries, k over d: the rounded fragments that are the update's B operand, so it needs
// no transposition; the key walk gathers G^T from it.
//
// Every step issues the same memory operations on every wave, whether or not the wave
// has work in it (a copy for the next record, a q~ prefetch from a clamped valid pair,
// and the stores of G, to a spare fragment set of the workspace when there is nothing to
// store), so that one wait for all but the last stores at the top of each step covers
// every path and the compiler adds no wait of its own inside the step.
__global__ __launch_bounds__(64 * 2 * kUpQB) void bwd_up_kernel_lds(BwdArgs a) {
    typedef uint16_t S;
    typedef Elem<S>::Frag Frag;
    constexpr int D = 64, KCD = D / 16, RTD = D / 32, NTH = 64 * 2 * kUpQB;
    constexpr int REC = 3 * kC * D + D * D;  // elements of a record
    constexpr int NLD = REC * 2 / 16 / NTH;   // DMA chunks per thread and record
    static_assert(REC * 2 % (16 * NTH) == 0, "record must split evenly over the workgroup");
    constexpr int NST = KCD;  // global stores of one step: G^(J-1)
    // One LDS array: two buffers, each a record followed by 64 key terms of the exponent and 64
    // gate sums (between each of the tile's query blocks and the record's key block, repeated
    // over the lanes).  The copies into LDS are ordered by the explicit waits and barriers of the
    // walk alone.
    constexpr int BUF = REC * 2 + 2 * 4 * kC;  // bytes per buffer
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int nb = a.nb, hc = a.hc;
    const int ntile = (nb - 1 + kUpQB - 1) / kUpQB;  // query blocks 1 .. nb-1, four per tile
    int gl, tile;
    walk_item(ntile, hc, 1, gl, tile);
    tile = ntile - 1 - tile;
    const int I0 = 1 + kUpQB * tile;                 // the tile's first query block
    const int Imax = min(nb - 1, I0 + kUpQB - 1);    // and its last
    // this wave's query block and query half (wave-uniform, so the per-pair scalars are scalar loads)
    const int I = __builtin_amdgcn_readfirstlane(I0 + (w >> 1)), wq = __builtin_amdgcn_readfirstlane(w & 1);
    const bool active = I <= nb - 1;
    const int Ic = active ? I : Imax;  // idle waves read a valid block and discard it
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *RECS = (const S *)(ws + ly.urec), *QS1 = (const S *)(ws + ly.qs1);
    S *GS2 = (S *)(ws + ly.gs2);
    S *const spare = GS2 + (int64_t)nb * (nb - 1) / 2 * kC * D;  // the fragment set after the last pair's
    const float *MID = (const float *)(ws + ly.mid), *CKK = (const float *)(ws + ly.ckl);
    const float scale = a.scale, c2 = scale * kLog2e;
    const int qi = Ic * kC + 32 * wq + l32;
    const float dd = ((const float *)(ws + ly.dd))[qi], cq = ((const float *)(ws + ly.cql))[qi];
    // the gate-sum lane of wave 1: query block I0 + (lane % 4), clamped to the last block
    const int Il = min(I0 + (lane & (kUpQB - 1)), nb - 1);

    // copies of key block J's record (all threads) and its side values (one 4-byte element per
    // lane: key terms from wave 0 and waves 2.. (the same values), gate sums from wave 1) into
    // buffer B.  J <= nb - 1, so every source lies inside the workspace.
    auto issue = [&](int J, int B) {
        unsigned char *buf = smem + B * BUF;
        dma_record<NTH, NLD>(RECS + (int64_t)J * REC, buf, tid);
        const float *src = w == 1 ? MID + pair_index(Il, min(J, Il - 1)) : CKK + J * kC + lane;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(buf + REC * 2 + (w == 1 ? 4 * kC : 0)), 4, 0, 0);
    };
    issue(0, 0);
    // q~ of the pair (I, J) is in qa for even J and in qb for odd J; each step loads the next one
    Frag dof[KCD], qa[KCD], qb[KCD];
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc) {
        dof[kc] = ldfrag<S>((const S *)(ws + ly.do1) + (int64_t)Ic * kC * D, wq, kc, KCD, lane);
        qa[kc] = ldfrag<S>(QS1 + pair_index(Ic, 0) * kC * D, wq, kc, KCD, lane);
    }
    f32x16 gt[RTD];
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt) gt[dt] = f32x16{};
    float rsum = 0.f;
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
    // one step over key block J, whose copies are in buffer B (J % 2); it refills the other one
    auto step = [&](int J, auto bsel) {
        constexpr int B = decltype(bsel)::value;
        const S *rec = (const S *)(smem + B * BUF);
        const float *sck = (const float *)(smem + B * BUF + REC * 2), *smid = sck + kC;
        // this wave's copies of record J and its q~ prefetch have landed (only the previous
        // step's stores may still be in flight) and its LDS accesses of the previous step have
        // returned; after the barrier every wave's copies have landed and the other buffer is free
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(NST));
        asm volatile("s_barrier" ::: "memory");
        issue(min(J + 1, nb - 1), 1 - B);
        asm volatile("" ::: "memory");  // the copies stay ahead of this step's stores
        const bool act = active && J < I;
        Frag(&qf)[KCD] = B ? qb : qa;
        Frag(&qn)[KCD] = B ? qa : qb;
        {
            const int64_t pn = pair_index(Ic, min(J + 1, Ic - 1));
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) qn[kc] = ldfrag<S>(QS1 + pn * kC * D, wq, kc, KCD, lane);
        }
        Frag gf[KCD];  // G^(J-1) (rows: the wave's queries, k over d), rounded: the B operand below
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) gf[kc] = acc_frag<S>(gt[kc >> 1], kc & 1);
        if (act) {
            const float mid = smid[w >> 1];
            f32x16 sv[2], dp[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sv[kt] = f32x16{};
                dp[kt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) {
                    Elem<S>::mma(sv[kt], ldfrag<S>(rec, kt, kc, KCD, lane), qf[kc]);
                    Elem<S>::mma(dp[kt], ldfrag<S>(rec + kC * D, kt, kc, KCD, lane), dof[kc]);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 ck = *reinterpret_cast<const f32x4 *>(sck + 32 * kt + 8 * g4 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        const float P = fast_exp2(c2 * sv[kt][r] + cq + ck[e] + mid);
                        const float ds = P * (dp[kt][r] - dd);
                        rsum += ds;
                        sv[kt][r] = scale * ds;
                    }
                }
            Frag sf[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) sf[kc] = acc_frag<S>(sv[kc >> 1], kc & 1);
#pragma unroll
            for (int dt = 0; dt < RTD; ++dt) {
                if (J >= 1) {
#pragma unroll
                    for (int kc = 0; kc < KCD; ++kc)
                        Elem<S>::mma(gt[dt], ldfrag<S>(rec + 3 * kC * D, dt, kc, KCD, lane), gf[kc]);
                }
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(gt[dt], ldfrag<S>(rec + 2 * kC * D, dt, kc, 4, lane), sf[kc]);
            }
        }
        // G^(J-1) for the pair (I, J) (J >= 1; to the spare set otherwise)
        S *dst = (act && J >= 1) ? GS2 + pair_index(I, J) * kC * D : spare;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) stfrag<S>(dst, wq, kc, KCD, lane, gf[kc]);
    };
    for (int J = 0; J < Imax; J += 2) {
        step(J, std::integral_constant<int, 0>{});
        if (J + 1 < Imax) step(J + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));  // no copy may still be landing in LDS when the workgroup leaves
    if (!active) return;
    rsum = other_half_sum(rsum);
    float *dqo = (float *)(ws + ly.dqo) + (int64_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = {gt[dt][4 * g4], gt[dt][4 * g4 + 1], gt[dt][4 * g4 + 2], gt[dt][4 * g4 + 3]};
            *reinterpret_cast<f32x4 *>(dqo + 32 * dt + 8 * g4 + 4 * h) = x;
        }
    if (h == 0) ((float *)(ws + ly.rso))[qi] = rsum;
}

// Up walk for bf16 inputs at head dimension 128: as bwd_up_kernel_lds, but a record (80
// KiB) is copied in two parts: k^ and V (the operands of the logits, 32 KiB) one step
// ahead into two buffers, and k^^T and (T - I)^T (the operands of the adjoint update, 48
// KiB) into one buffer at the top of the step, landing while the logits and dS are
// computed.  G^(J-1) is stored as at d = 64.  Every step issues the same memory
// operations on every wave, as in the d = 64 walks.
__global__ __launch_bounds__(64 * 2 * kUpQB) void bwd_up_kernel_split(BwdArgs a) {
    typedef uint16_t S;
    typedef Elem<S>::Frag Frag;
    constexpr int D = 128, KCD = D / 16, RTD = D / 32, NTH = 64 * 2 * kUpQB;
    constexpr int RA = 2 * kC * D;            // elements of the first part: k^, V
    constexpr int RB = kC * D + D * D;        // of the second: k^^T, (T - I)^T
    constexpr int NLA = RA * 2 / 16 / NTH, NLB = RB * 2 / 16 / NTH;
    static_assert(RA * 2 % (16 * NTH) == 0 && RB * 2 % (16 * NTH) == 0, "parts must split evenly over the workgroup");
    constexpr int NST = KCD;                  // global stores of one step: G^(J-1)
    constexpr int NAFTER = NLA + 1 + KCD;     // memory operations issued after the second part's copy
    // one LDS array: two buffers of the first part, each followed by 64 key terms and 64 gate
    // sums, then the second part's buffer
    constexpr int ABUF = RA * 2 + 2 * 4 * kC;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * ABUF + RB * 2];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int nb = a.nb, hc = a.hc;
    const int ntile = (nb - 1 + kUpQB - 1) / kUpQB;
    int gl, tile;
    walk_item(ntile, hc, 1, gl, tile);
    tile = ntile - 1 - tile;
    const int I0 = 1 + kUpQB * tile, Imax = min(nb - 1, I0 + kUpQB - 1);
    const int I = __builtin_amdgcn_readfirstlane(I0 + (w >> 1)), wq = __builtin_amdgcn_readfirstlane(w & 1);
    const bool active = I <= nb - 1;
    const int Ic = active ? I : Imax;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *RECS = (const S *)(ws + ly.urec), *QS1 = (const S *)(ws + ly.qs1);
    const int64_t RE = ly.rec_elems;
    S *GS2 = (S *)(ws + ly.gs2);
    S *const spare = GS2 + (int64_t)nb * (nb - 1) / 2 * kC * D;
    const float *MID = (const float *)(ws + ly.mid), *CKK = (const float *)(ws + ly.ckl);
    const float scale = a.scale, c2 = scale * kLog2e;
    const int qi = Ic * kC + 32 * wq + l32;
    const float dd = ((const float *)(ws + ly.dd))[qi], cq = ((const float *)(ws + ly.cql))[qi];
    const int Il = min(I0 + (lane & (kUpQB - 1)), nb - 1);
    const S *sb = (const S *)(smem + 2 * ABUF);  // k^^T (rows d, k over keys), then (T - I)^T

    // first part of record J and its side values (key terms from waves other than 1, gate sums
    // from wave 1) into buffer B; J <= nb - 1
    auto issue_a = [&](int J, int B) {
        unsigned char *buf = smem + B * ABUF;
        dma_record<NTH, NLA>(RECS + (int64_t)J * RE, buf, tid);
        const float *src = w == 1 ? MID + pair_index(Il, min(J, Il - 1)) : CKK + J * kC + lane;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(buf + RA * 2 + (w == 1 ? 4 * kC : 0)), 4, 0, 0);
    };
    issue_a(0, 0);
    Frag dof[KCD], qa[KCD], qb[KCD];
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc) {
        dof[kc] = ldfrag<S>((const S *)(ws + ly.do1) + (int64_t)Ic * kC * D, wq, kc, KCD, lane);
        qa[kc] = ldfrag<S>(QS1 + pair_index(Ic, 0) * kC * D, wq, kc, KCD, lane);
    }
    f32x16 gt[RTD];
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt) gt[dt] = f32x16{};
    float rsum = 0.f;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
    auto step = [&](int J, auto bsel) {
        constexpr int B = decltype(bsel)::value;
        const S *rec = (const S *)(smem + B * ABUF);
        const float *sck = (const float *)(smem + B * ABUF + RA * 2), *smid = sck + kC;
        // this wave's copies of the first part of record J and its q~ prefetch have landed (only
        // the previous step's stores may be in flight); after the barrier every wave's have, and
        // every wave is done with the second-part buffer and the other first-part buffer
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(NST));
        asm volatile("s_barrier" ::: "memory");
        dma_record<NTH, NLB>(RECS + (int64_t)J * RE + RA, smem + 2 * ABUF, tid);
        issue_a(min(J + 1, nb - 1), 1 - B);
        asm volatile("" ::: "memory");
        const bool act = active && J < I;
        Frag(&qf)[KCD] = B ? qb : qa;
        Frag(&qn)[KCD] = B ? qa : qb;
        {
            const int64_t pn = pair_index(Ic, min(J + 1, Ic - 1));
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) qn[kc] = ldfrag<S>(QS1 + pn * kC * D, wq, kc, KCD, lane);
        }
        f32x16 sv[2];
        if (act) {
            const float mid = smid[w >> 1];
            // one key tile at a time (its dP dies before the next tile's products)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x16 dp = {};
                sv[kt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KCD; ++kc) {
                    Elem<S>::mma(sv[kt], ldfrag<S>(rec, kt, kc, KCD, lane), qf[kc]);
                    Elem<S>::mma(dp, ldfrag<S>(rec + kC * D, kt, kc, KCD, lane), dof[kc]);
                }
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 ck = *reinterpret_cast<const f32x4 *>(sck + 32 * kt + 8 * g4 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        const float P = fast_exp2(c2 * sv[kt][r] + cq + ck[e] + mid);
                        const float ds = P * (dp[r] - dd);
                        rsum += ds;
                        sv[kt][r] = scale * ds;
                    }
                }
            }
        }
        // this wave's copies of the second part have landed (the first part's next copy and the
        // q~ prefetch, issued after them, may stay in flight); after the barrier every wave's have
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(NAFTER));
        asm volatile("s_barrier" ::: "memory");
        Frag gf[KCD];  // G^(J-1) (rows: the wave's queries, k over d), rounded: the B operand below
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) gf[kc] = acc_frag<S>(gt[kc >> 1], kc & 1);
        if (act) {
            Frag sf[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) sf[kc] = acc_frag<S>(sv[kc >> 1], kc & 1);
#pragma unroll
            for (int dt = 0; dt < RTD; ++dt) {
                if (J >= 1) {
#pragma unroll
                    for (int kc = 0; kc < KCD; ++kc) Elem<S>::mma(gt[dt], ldfrag<S>(sb + kC * D, dt, kc, KCD, lane), gf[kc]);
                }
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) Elem<S>::mma(gt[dt], ldfrag<S>(sb, dt, kc, 4, lane), sf[kc]);
            }
        }
        // G^(J-1) for the pair (I, J) (J >= 1; to the spare set otherwise)
        S *dst = (act && J >= 1) ? GS2 + pair_index(I, J) * kC * D : spare;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) stfrag<S>(dst, wq, kc, KCD, lane, gf[kc]);
    };
    for (int J = 0; J < Imax; J += 2) {
        step(J, std::integral_constant<int, 0>{});
        if (J + 1 < Imax) step(J + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));  // no copy may still be landing in LDS when the workgroup leaves
    if (!active) return;
    rsum = other_half_sum(rsum);
    float *dqo = (float *)(ws + ly.dqo) + (int64_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < RTD; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = {gt[dt][4 * g4], gt[dt][4 * g4 + 1], gt[dt][4 * g4 + 2], gt[dt][4 * g4 + 3]};
            *reinterpret_cast<f32x4 *>(dqo + 32 * dt + 8 * g4 + 4 * h) = x;
        }
    if (h == 0) ((float *)(ws + ly.rso))[qi] = rsum;
}

// Key walk (fp32 inputs; bf16: bwd_key_kernel_lds): one workgroup per (key block J <= nb-2, head).  Wave w takes the
// logit tile of queries 32 qt .. (qt = w & 1) and keys 32 kt .. (kt = (w >> 1)
// & 1) of every later query block I, recomputes P and dS, and accumulates over
// its 32 queries dV^T = dO^T P and dk^^T = q~^T dS (rows: its group dh = w >> 2
// of head-dimension tiles) and dT = G^T q~ (its rows of dT); the two query
// halves are added at the end.
template <int D>
struct KeyCfg {
    static constexpr int NW = D == 64 ? 4 : 8;  // waves
    static constexpr int NDH = NW / 4;           // groups of head-dimension tiles
    static constexpr int RTW = (D / 32) / NDH;   // dV^T, dk^T row tiles per wave
    static constexpr int NG = 2 * NDH;           // wave groups (kt, dh) splitting the rows of dT
    static constexpr int TRW = (D / 32) / NG;    // dT row tiles per wave
};

template <typename S, int D>
__global__ __launch_bounds__(64 * KeyCfg<D>::NW) void bwd_key_kernel(BwdArgs a) {
    typedef typename Elem<S>::Frag Frag;
    typedef KeyCfg<D> K;
    constexpr int KCD = D / 16, RTD = D / 32, RTW = K::RTW, TRW = K::TRW;
    constexpr int NACC = 2 * RTW + TRW * RTD;  // accumulator tiles per wave
    __shared__ __attribute__((aligned(16))) float sred[K::NW / 2][16 * 65];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int qt = w & 1, kt = (w >> 1) & 1, dh = K::NDH == 1 ? 0 : w >> 2, grp = kt + 2 * dh;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, J = blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *QS1 = (const S *)(ws + ly.qs1), *QS2 = (const S *)(ws + ly.qs2), *GS2 = (const S *)(ws + ly.gs2);
    const S *DO1 = (const S *)(ws + ly.do1), *DO2 = (const S *)(ws + ly.do2);
    const float *MID = (const float *)(ws + ly.mid);
    const float *DD = (const float *)(ws + ly.dd), *CQL = (const float *)(ws + ly.cql);
    const float scale = a.scale, c2 = scale * kLog2e;
    const int key = J * kC + 32 * kt + l32;  // this lane's key (column of the logit tile)
    const float ck = ((const float *)(ws + ly.ckl))[key];

    Frag kf[KCD], vf[KCD];  // k^ and V of key tile kt, k over d: the B operands of S and dP
    {
        const S *rec = (const S *)(ws + ly.urec) + J * ly.rec_elems;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            kf[kc] = ldfrag<S>(rec, kt, kc, KCD, lane);
            vf[kc] = ldfrag<S>(rec + kC * D, kt, kc, KCD, lane);
        }
    }
    f32x16 acc[NACC];  // dV^T (RTW), dk^^T (RTW), dT rows grp * TRW .. (TRW x RTD)
#pragma unroll
    for (int t = 0; t < NACC; ++t) acc[t] = f32x16{};
    float csum = 0.f;
    if constexpr (D == 64) {
    // Every fragment a step needs is loaded at its top, and the next pair's q~ and dO
    // (the first operands of a step) one step ahead, so a step waits for memory once.
    Frag q1[KCD], o1[KCD];
    auto load_first = [&](int I, Frag *q, Frag *o) {
        const int64_t po = pair_index(I, J) * kC * D, bo = (int64_t)I * kC * D;
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            q[kc] = ldfrag<S>(QS1 + po, qt, kc, KCD, lane);
            o[kc] = ldfrag<S>(DO1 + bo, qt, kc, KCD, lane);
        }
    };
    load_first(J + 1, q1, o1);
    for (int I = J + 1; I < nb; ++I) {
        const int64_t p = pair_index(I, J), po = p * kC * D, bo = (int64_t)I * kC * D;
        // (the dk^ operands are loaded apart from the dT ones: indexing a register array with the
        // wave's tile group would compile into selects over the whole array)
        Frag q2[RTD][2], q2k[RTW][2], o2[RTW][2], g2[TRW][2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
            for (int ct = 0; ct < RTD; ++ct) q2[ct][cc] = ldfrag<S>(QS2 + po, ct, 2 * qt + cc, 4, lane);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                q2k[i][cc] = ldfrag<S>(QS2 + po, dh * RTW + i, 2 * qt + cc, 4, lane);
                o2[i][cc] = ldfrag<S>(DO2 + bo, dh * RTW + i, 2 * qt + cc, 4, lane);
            }
#pragma unroll
            for (int i = 0; i < TRW; ++i)
                g2[i][cc] = J >= 1 ? ldfrag<S>(GS2 + po, grp * TRW + i, 2 * qt + cc, 4, lane) : Frag{};
        }
        const float mid = MID[p];
        const int q0 = I * kC + 32 * qt + 4 * h;
        f32x4 ddv[4], cqv[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            ddv[g4] = *reinterpret_cast<const f32x4 *>(DD + q0 + 8 * g4);
            cqv[g4] = *reinterpret_cast<const f32x4 *>(CQL + q0 + 8 * g4);
        }
        Frag q1n[KCD], o1n[KCD];
        if (I + 1 < nb) load_first(I + 1, q1n, o1n);
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            Elem<S>::mma(s, q1[kc], kf[kc]);
            Elem<S>::mma(dp, o1[kc], vf[kc]);
        }
        // P and dS (rows: queries 32 qt + acc_row(r, h) of block I; column: this lane's key)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                const float P = fast_exp2(c2 * s[r] + cqv[g4][e] + ck + mid);
                const float ds = P * (dp[r] - ddv[g4][e]);
                csum += ds;
                s[r] = ds;
                dp[r] = P;
            }
        Frag pf[2], sf[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            pf[cc] = acc_frag<S>(dp, cc);
            sf[cc] = acc_frag<S>(s, cc);
        }
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                Elem<S>::mma(acc[i], o2[i][cc], pf[cc]);
                Elem<S>::mma(acc[RTW + i], q2k[i][cc], sf[cc]);
            }
        if (J >= 1) {
#pragma unroll
            for (int i = 0; i < TRW; ++i)
#pragma unroll
                for (int ct = 0; ct < RTD; ++ct)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) Elem<S>::mma(acc[2 * RTW + i * RTD + ct], g2[i][cc], q2[ct][cc]);
        }
        if (I + 1 < nb) {
#pragma unroll
            for (int kc = 0; kc < KCD; ++kc) {
                q1[kc] = q1n[kc];
                o1[kc] = o1n[kc];
            }
        }
    }
    } else {
    // (d = 128: a step's operands do not fit the registers at once; each is loaded where it is used)
    for (int I = J + 1; I < nb; ++I) {
        const int64_t p = pair_index(I, J), po = p * kC * D, bo = (int64_t)I * kC * D;
        const float mid = MID[p];
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            Elem<S>::mma(s, ldfrag<S>(QS1 + po, qt, kc, KCD, lane), kf[kc]);
            Elem<S>::mma(dp, ldfrag<S>(DO1 + bo, qt, kc, KCD, lane), vf[kc]);
        }
        const int q0 = I * kC + 32 * qt + 4 * h;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 dd = *reinterpret_cast<const f32x4 *>(DD + q0 + 8 * g4);
            const f32x4 cq = *reinterpret_cast<const f32x4 *>(CQL + q0 + 8 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                const float P = fast_exp2(c2 * s[r] + cq[e] + ck + mid);
                const float ds = P * (dp[r] - dd[e]);
                csum += ds;
                s[r] = ds;
                dp[r] = P;
            }
        }
        Frag pf[2], sf[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            pf[cc] = acc_frag<S>(dp, cc);
            sf[cc] = acc_frag<S>(s, cc);
        }
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int dt = dh * RTW + i;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                Elem<S>::mma(acc[i], ldfrag<S>(DO2 + bo, dt, 2 * qt + cc, 4, lane), pf[cc]);
                Elem<S>::mma(acc[RTW + i], ldfrag<S>(QS2 + po, dt, 2 * qt + cc, 4, lane), sf[cc]);
            }
        }
        if (J >= 1) {
#pragma unroll
            for (int i = 0; i < TRW; ++i) {
                const int rt = grp * TRW + i;
                Frag ga[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) ga[cc] = ldfrag<S>(GS2 + po, rt, 2 * qt + cc, 4, lane);
#pragma unroll
                for (int ct = 0; ct < RTD; ++ct)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
                        Elem<S>::mma(acc[2 * RTW + i * RTD + ct], ga[cc],
                                     ldfrag<S>(QS2 + po, ct, 2 * qt + cc, 4, lane));
            }
        }
    }
    }
    csum = other_half_sum(csum);  // lanes l and l ^ 32 hold the other queries of the same key
    // add the query half qt = 1 into qt = 0 (the partner wave w + 1), one tile at a time
    float *red = sred[w >> 1];
    for (int t = 0; t <= NACC; ++t) {
        __syncthreads();
        if (qt == 1) {
            if (t < NACC) {
#pragma unroll
                for (int r = 0; r < 16; ++r) red[r * 65 + lane] = acc[t][r];
            } else {
                red[lane] = csum;
            }
        }
        __syncthreads();
        if (qt == 0) {
            if (t < NACC) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] += red[r * 65 + lane];
            } else {
                csum += red[lane];
            }
        }
    }
    if (qt != 0) return;
    float *dvo = (float *)(ws + ly.dvo) + (int64_t)key * D, *dko = (float *)(ws + ly.dko) + (int64_t)key * D;
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int dt = dh * RTW + i;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * dt + 8 * g4 + 4 * h;
            const f32x4 xv = {acc[i][4 * g4], acc[i][4 * g4 + 1], acc[i][4 * g4 + 2], acc[i][4 * g4 + 3]};
            const f32x4 xk = {scale * acc[RTW + i][4 * g4], scale * acc[RTW + i][4 * g4 + 1],
                              scale * acc[RTW + i][4 * g4 + 2], scale * acc[RTW + i][4 * g4 + 3]};
            *reinterpret_cast<f32x4 *>(dvo + d0) = xv;
            *reinterpret_cast<f32x4 *>(dko + d0) = xk;
        }
    }
    if (J >= 1) {  // dT^T: element (c, r) = dT[r][c]; lane c writes 4 consecutive r
        float *dtt = (float *)(ws + ly.dtt) + (int64_t)J * D * D;
#pragma unroll
        for (int i = 0; i < TRW; ++i) {
            const int rt = grp * TRW + i;
#pragma unroll
            for (int ct = 0; ct < RTD; ++ct)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x16 &x = acc[2 * RTW + i * RTD + ct];
                    const f32x4 y = {x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]};
                    *reinterpret_cast<f32x4 *>(dtt + (int64_t)(32 * ct + l32) * D + 32 * rt + 8 * g4 + 4 * h) = y;
                }
        }
    }
    if (dh == 0 && h == 0) ((float *)(ws + ly.cso))[J * kC + 32 * kt + l32] = csum;
}

// ---------------------------------------------------------------------------
// Block backward: one workgroup per (block J, head); fp32 inputs (bf16: bwd_block_kernel_bf16).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void acc2out(T *g, int D, const f32x8 &acc, int row0, int L, int lane, int wave) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        if (row0 + r < L) g[(int64_t)(row0 + r) * D + c] = Elem<T>::from_float(acc[v]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kT) void bwd_block_kernel(BwdArgs a) {
    constexpr int NCH = D / 64;
    __shared__ __attribute__((aligned(16))) float sm[9 * kTile + 2 * kC];
    float *bE = sm, *bN = bE + kTile, *bZ = bN + kTile, *bX = bZ + kTile, *bA = bX + kTile, *bQW = bA + kTile,
          *b6 = bQW + kTile, *b7 = b6 + kTile, *b8 = b7 + kTile;
    float *sB = b8 + kTile, *sRed = sB + kC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, nb = a.nb, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * D, *k = (const T *)a.k + hoff * D, *w = (const T *)a.w + hoff * D;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const bool hasQ = J >= 1, hasK = J <= nb - 2, hasT = J >= 1 && J <= nb - 2;
    const int64_t tok = (int64_t)J * kC * kC, nat0 = (int64_t)row0 * D;
    const float *dqo = (const float *)(ws + ly.dqo) + nat0, *dko = (const float *)(ws + ly.dko) + nat0;

    if (tid < kC) sB[tid] = row0 + tid < L ? a.beta[hoff + row0 + tid] : 0.f;
    g2l(bE, (const float *)(ws + ly.ee) + tok, kC, tid);  // scale dS of the diagonal block
    g2l(bN, (const float *)(ws + ly.nn) + tok, kC, tid);
    g2l(bZ, (const float *)(ws + ly.zz) + tok, kC, tid);
    g2l(bX, (const float *)(ws + ly.xx) + tok, kC, tid);
    g2l(bA, (const float *)(ws + ly.aa) + tok, kC, tid);
    g2l(bQW, (const float *)(ws + ly.qwm) + tok, kC, tid);
    __syncthreads();
    // ---- token-level quantities
    f32x8 aZ = zero8(), aNn = zero8(), aY = zero8(), aG = zero8(), aA = zero8(), acc;
    mmx<T, false, false>(aZ, nat(bE), nat(bN), lane, wave);    // E N         (dZ = -(E N + dq^ W^T))
    mmx<T, false, false>(aNn, tr(bE), nat(bZ), lane, wave);    // E^T Z       (dN = -E^T Z + dY A^T)
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        in2l(b6, w, D, 64 * c, row0, L, tid);
        if (hasQ) g2l(b7, dqo + 64 * c, D, tid);
        else zero_lds(b7, tid);
        if (hasK) g2l(b8, dko + 64 * c, D, tid);
        else zero_lds(b8, tid);
        __syncthreads();
        mmx<T, false, true>(aZ, nat(b7), tr(b6), lane, wave);  // + dq^ W^T
        mmx<T, false, true>(aY, nat(b8), tr(b6), lane, wave);  // dk^ W^T   (dY = -dk^ W^T)
        mmx<T, true, true>(aG, nat(b6), tr(b6), lane, wave);  // G = W W^T
    }
    if (hasT) {
        // U = W dT and V' = W dT^T (64 x D, for the backward through T = I - W^T A W) and
        // U W^T = W dT W^T; the key walk left dT^T, so dT[c2, c] = (dT^T[c, c2])^T
        const float *dtt = (const float *)(ws + ly.dtt) + (int64_t)J * D * D;
        float *uu = (float *)(ws + ly.uu) + nat0, *vv = (float *)(ws + ly.vv) + nat0;
        for (int c = 0; c < NCH; ++c) {
            f32x8 aU = zero8(), aV = zero8();
            for (int c2 = 0; c2 < NCH; ++c2) {
                __syncthreads();
                in2l(b6, w, D, 64 * c2, row0, L, tid);
                g2l(b7, dtt + (int64_t)(64 * c) * D + 64 * c2, D, tid);   // dT^T block (c, c2)
                g2l(b8, dtt + (int64_t)(64 * c2) * D + 64 * c, D, tid);   // dT^T block (c2, c)
                __syncthreads();
                mmx<T, true, false>(aU, nat(b6), tr(b7), lane, wave);  // W_c2 dT[c2, c]
                mmx<T, true, false>(aV, nat(b6), nat(b8), lane, wave);  // W_c2 dT^T[c2, c]
            }
            acc2g(uu + 64 * c, D, aU, lane, wave);
            acc2g(vv + 64 * c, D, aV, lane, wave);
            __syncthreads();
            store_lds(b7, aU, lane, wave, Id());
            in2l(b6, w, D, 64 * c, row0, L, tid);
            __syncthreads();
            acc = zero8();
            mmx<T, false, true>(acc, nat(b7), tr(b6), lane, wave);  // U_c W_c^T
#pragma unroll
            for (int v = 0; v < 8; ++v) aA[v] -= acc[v];  // dA = -W dT W^T + ...
        }
    }
    __syncthreads();
    store_lds(b6, aY, lane, wave, [](int, int, float x) { return -x; });  // dY
    store_lds(b7, aZ, lane, wave, [](int, int, float x) { return -x; });  // dZ
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 8; ++v) aNn[v] = -aNn[v];
    mmx<T, false, false>(aNn, nat(b6), tr(bA), lane, wave);   // dN = -E^T Z + dY A^T
    mmx<T, false, false>(aA, tr(bN), nat(b6), lane, wave);    // dA += N^T dY
    mmx<T, false, false>(aA, tr(b7), nat(bQW), lane, wave);   // dA += dZ^T QWm
    acc = zero8();
    mmx<T, false, false>(acc, nat(b7), nat(bA), lane, wave);  // dQWm = (dZ A) o [r <= i]
    f32x8 aYv = zero8();
    mmx<T, false, false>(aYv, nat(bN), nat(bA), lane, wave);  // Y = N A
    __syncthreads();
    store_lds(b8, acc, lane, wave, [](int r, int c, float x) { return c <= r ? x : 0.f; });  // dQWm
    store_lds(b6, aNn, lane, wave, [](int r, int c, float x) { return c > r ? x : 0.f; });   // dKW = dN o [r > j]
    store_lds(bN, aYv, lane, wave, Id());                                                    // Y (N is done with)
    // A = X diag(beta): dX = dA diag(beta), dbeta_c += sum_r X_rc dA_rc (dA kept on the upper triangle)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        aA[v] = c >= r ? aA[v] : 0.f;
        b7[r * kP + c] = aA[v] * sB[c];
        bQW[r * kP + c] = bX[r * kP + c] * aA[v];
    }
    __syncthreads();
    float dbeta = 0.f;
    if (tid < kC)
        for (int r = 0; r < kC; ++r) dbeta += bQW[r * kP + tid];
    acc = zero8();
    mmx<T, false, false>(acc, tr(bX), nat(b7), lane, wave);  // X^T dX
    __syncthreads();
    store_lds(bQW, acc, lane, wave, Id());
    __syncthreads();
    f32x8 dTp = zero8();
    mmx<T, false, false>(dTp, nat(bQW), tr(bX), lane, wave);  // (X^T dX) X^T; dT' is its negative
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        const float t = -dTp[v];
        bQW[r * kP + c] = c > r ? t * aG[v] : 0.f;  // dbeta_r += sum_c dT'_rc G_rc
        b7[r * kP + c] = c > r ? sB[r] * t : 0.f;   // dG = diag(beta) dT' on the strict upper triangle
    }
    __syncthreads();
    if (tid >= kC && tid < 2 * kC) {
        float s = 0.f;
        for (int c = 0; c < kC; ++c) s += bQW[(tid - kC) * kP + c];
        sRed[tid - kC] = s;
    }
    __syncthreads();
    if (tid < kC && row0 + tid < L) a.dbeta[hoff + row0 + tid] = dbeta + sRed[tid];
    // ---- chunks of the head dimension.  LDS: E, Y (bN), Z, A, dKW (b6), dG (b7), dQWm (b8);
    //      bX and bQW hold the chunk operands.
    const float *uu = (const float *)(ws + ly.uu) + nat0, *vvp = (const float *)(ws + ly.vv) + nat0;
    for (int c = 0; c < NCH; ++c) {
        f32x8 dQ = zero8(), dK = zero8(), dW = zero8();
        __syncthreads();
        in2l(bX, k, D, 64 * c, row0, L, tid);
        in2l(bQW, q, D, 64 * c, row0, L, tid);
        __syncthreads();
        mmx<T, false, true>(dQ, nat(bE), nat(bX), lane, wave);   // E K
        mmx<T, false, true>(dK, tr(bE), nat(bQW), lane, wave);   // E^T Q
        mmx<T, false, true>(dW, tr(b6), nat(bX), lane, wave);    // dKW^T K
        mmx<T, false, true>(dW, tr(b8), nat(bQW), lane, wave);   // dQWm^T Q
        __syncthreads();
        in2l(bX, w, D, 64 * c, row0, L, tid);
        __syncthreads();
        mmx<T, false, true>(dQ, nat(b8), nat(bX), lane, wave);   // dQWm W
        mmx<T, false, true>(dK, nat(b6), nat(bX), lane, wave);   // dKW W
        mmx<T, false, true>(dW, nat(b7), nat(bX), lane, wave);   // (dG + dG^T) W
        mmx<T, false, true>(dW, tr(b7), nat(bX), lane, wave);
        __syncthreads();
        if (hasQ) g2l(bX, dqo + 64 * c, D, tid);
        else zero_lds(bX, tid);
        if (hasK) g2l(bQW, dko + 64 * c, D, tid);
        else zero_lds(bQW, tid);
        __syncthreads();
        acc = zero8();
        mmx<T, false, false>(acc, tr(bZ), nat(bX), lane, wave);   // Z^T dq^
        mmx<T, false, false>(acc, tr(bN), nat(bQW), lane, wave);  // + Y^T dk^ (= A^T N^T dk^)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int r = arow(v, lane, wave), cc = acol(v, lane, wave);
            dQ[v] += bX[r * kP + cc];
            dK[v] += bQW[r * kP + cc];
            dW[v] -= acc[v];
        }
        if (hasT) {
            __syncthreads();
            g2l(bX, uu + 64 * c, D, tid);
            g2l(bQW, vvp + 64 * c, D, tid);
            __syncthreads();
            acc = zero8();
            mmx<T, false, false>(acc, nat(bA), nat(bQW), lane, wave);  // A W dT^T
            mmx<T, false, false>(acc, tr(bA), nat(bX), lane, wave);    // + A^T W dT
#pragma unroll
            for (int v = 0; v < 8; ++v) dW[v] -= acc[v];
        }
        acc2out((T *)a.dq + hoff * D + 64 * c, D, dQ, row0, L, lane, wave);
        acc2out((T *)a.dk + hoff * D + 64 * c, D, dK, row0, L, lane, wave);
        acc2out((T *)a.dw + hoff * D + 64 * c, D, dW, row0, L, lane, wave);
    }
    {
        const float *dvd = (const float *)(ws + ly.dvd) + nat0, *dvo = (const float *)(ws + ly.dvo) + nat0;
        T *dv = (T *)a.dv + hoff * D;
        for (int e = tid; e < kC * D; e += kT) {
            const int r = e / D;
            if (row0 + r < L) dv[(int64_t)row0 * D + e] = Elem<T>::from_float(dvd[e] + (hasK ? dvo[e] : 0.f));
        }
    }
    if (tid < kC) {
        const int i = row0 + tid;
        const float rs = ((const float *)(ws + ly.rsd))[i] + (hasQ ? ((const float *)(ws + ly.rso))[i] : 0.f);
        const float cs = ((const float *)(ws + ly.csd))[i] + (hasK ? ((const float *)(ws + ly.cso))[i] : 0.f);
        ((float *)(ws + ly.dc))[i] = rs - cs;
    }
}

// ---------------------------------------------------------------------------
// Block backward for bf16 inputs: the same steps as bwd_block_kernel, with every
// 64x64 tile held in LDS already split for the bf16 products.
// ---------------------------------------------------------------------------
// A split tile is two planes of bf16 numbers, hi and lo, with x ~ hi + lo (hi = x rounded,
// lo = the rest rounded: about 16 significant bits; lo = 0 for a tile of bf16 input values).
// Each element is split once, when the tile is written, instead of by every wave that reads it
// in a product.  Rows of 64 elements; the 16-byte chunks of row r are swizzled (chunk c / 8 at
// position (c / 8) ^ (r % 8)), which spreads both the row-wise 16-byte reads of 16 consecutive
// rows and the transposing reads below over the LDS banks.
constexpr int kSP = kC * kC;  // elements per plane; a tile is 2 kSP bf16 (hi plane, then lo)
__device__ __forceinline__ int sidx(int r, int c) { return r * kC + ((((c >> 3) ^ r) & 7) << 3) + (c & 7); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A split tile as a product operand: t false, element (r, c) = tile[r][c]; t true, tile[c][r].
struct SMat {
    const uint16_t *p;
    bool t;
};
__device__ __forceinline__ SMat snat(const uint16_t *p) { return {p, false}; }
__device__ __forceinline__ SMat str(const uint16_t *p) { return {p, true}; }

// Operand fragment of v_mfma_f32_16x16x32_bf16 for k = k0 .. k0 + 31 from one plane: lane
// l = 16 q + i holds index rho0 + i (a row of A, a column of B) and k = k0 + 8 q + e, e = 0..7.
// KC (k runs along the plane's rows, element (rho, k) at [rho][k]): one 16-byte read.
// Otherwise (element at [k][rho]) two transposing reads: ds_read_b64_tr_b16 gives lane 16 g + i
// (in each group of 16 lanes) element i % 4 of the 8-byte chunks addressed by lanes 16 g + 4 t +
// i / 4, t = 0..3, as its elements t; lane 16 g + 4 t + j addresses elements rho0 + 4 j .. + 3 of
// row k0 + 8 g + t (second read: row k0 + 8 g + 4 + t).
template <bool KC>
__device__ __forceinline__ i16x8 sfrag(const uint16_t *pl, int rho0, int k0, int lane) {
    if constexpr (KC) {
        const int q = lane >> 4, i = lane & 15;
        return *reinterpret_cast<const i16x8 *>(pl + sidx(rho0 + i, k0 + 8 * q));
    } else {
        const int g = lane >> 4, t = (lane >> 2) & 3, j = lane & 3;
        const uint16_t *p1 = pl + sidx(k0 + 8 * g + t, rho0 + 4 * j);
        const uint16_t *p2 = pl + sidx(k0 + 8 * g + 4 + t, rho0 + 4 * j);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p2);
        return i16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
}
// A's fragment: rho is A's row, k contiguous unless A is the transposed view.
__device__ __forceinline__ i16x8 afrag(SMat A, int plane, int rho0, int k0, int lane) {
    const uint16_t *pl = A.p + plane * kSP;
    return A.t ? sfrag<false>(pl, rho0, k0, lane) : sfrag<true>(pl, rho0, k0, lane);
}
// B's fragment: rho is B's column; B(k, c) = tile[c][k] (k contiguous) for the transposed view.
__device__ __forceinline__ i16x8 bfrag(SMat B, int plane, int rho0, int k0, int lane) {
    const uint16_t *pl = B.p + plane * kSP;
    return B.t ? sfrag<true>(pl, rho0, k0, lane) : sfrag<false>(pl, rho0, k0, lane);
}

// acc += A * B on split tiles, the output layout of mm; EA, EB: the operand is a tile of bf16
// input values (lo = 0), so its lo products are skipped.  hi*hi + hi*lo + lo*hi otherwise.
template <bool EA, bool EB>
__device__ __forceinline__ void smm(f32x8 &acc, SMat A, SMat B, int lane, int wave) {
    const int r0 = 16 * (wave >> 1), c0 = 32 * (wave & 1);
    f32x4 lo = acc.lo, hi = acc.hi;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int k0 = 32 * st;
        const i16x8 ah = afrag(A, 0, r0, k0, lane);
        i16x8 al;
        if constexpr (!EA) al = afrag(A, 1, r0, k0, lane);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const i16x8 bh = bfrag(B, 0, c0 + 16 * ct, k0, lane);
            i16x8 bl;
            if constexpr (!EB) bl = bfrag(B, 1, c0 + 16 * ct, k0, lane);
            f32x4 &c = ct == 0 ? lo : hi;
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
            if constexpr (!EB) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
            if constexpr (!EA) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
        }
    }
    acc.lo = lo;
    acc.hi = hi;
}

// Element access and writes of split tiles.
__device__ __forceinline__ float sld(const uint16_t *p, int r, int c) {
    const int e = sidx(r, c);
    return bf16_to_f32(p[e]) + bf16_to_f32(p[kSP + e]);
}
__device__ __forceinline__ void sst(uint16_t *p, int r, int c, float x) {
    const int e = sidx(r, c);
    const uint16_t h = to_bf16(x);
    p[e] = h;
    p[kSP + e] = to_bf16(x - bf16_to_f32(h));
}
template <typename F>
__device__ __forceinline__ void sstore(uint16_t *p, const f32x8 &acc, int lane, int wave, F f) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        sst(p, r, c, f(r, c, acc[v]));
    }
}
// Eight consecutive elements (one 16-byte chunk) of row r, split, into both planes.
__device__ __forceinline__ void sput8(uint16_t *p, int r, int c8, const float *x) {
    u32x4 h, l;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        h[t] = pack_bf16(x[2 * t], x[2 * t + 1]);
        l[t] = pack_bf16(x[2 * t] - __uint_as_float(h[t] << 16), x[2 * t + 1] - __uint_as_float(h[t] & 0xffff0000u));
    }
    const int e = sidx(r, c8);
    *reinterpret_cast<u32x4 *>(p + e) = h;
    *reinterpret_cast<u32x4 *>(p + kSP + e) = l;
}
// Global fp32 matrix [64 rows][row stride gs] -> split tile (one chunk per thread).
__device__ __forceinline__ void sg2l(uint16_t *p, const float *g, int gs, int tid) {
    const int r = tid >> 3, c8 = (tid & 7) * 8;
    float x[8];
    load8(x, g + (int64_t)r * gs + c8);
    sput8(p, r, c8, x);
}
// Columns c0 .. c0+63 of bf16 input rows [row0, row0 + 64) (rows >= L read as 0) -> split tile.
__device__ __forceinline__ void sin2l(uint16_t *p, const uint16_t *g, int D, int c0, int row0, int L, int tid) {
    const int r = tid >> 3, c8 = (tid & 7) * 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 h = row0 + r < L ? *reinterpret_cast<const u32x4 *>(g + (int64_t)(row0 + r) * D + c0 + c8) : z;
    const int e = sidx(r, c8);
    *reinterpret_cast<u32x4 *>(p + e) = h;
    *reinterpret_cast<u32x4 *>(p + kSP + e) = z;
}
__device__ __forceinline__ void szero(uint16_t *p, int tid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int r = tid >> 3, c8 = (tid & 7) * 8, e = sidx(r, c8);
    *reinterpret_cast<u32x4 *>(p + e) = z;
    *reinterpret_cast<u32x4 *>(p + kSP + e) = z;
}

// A 64x64 block of a matrix X held as a split tile -> the 2 x 4 fragments of X it covers (bf16:
// the hi plane, i.e. each value rounded to nearest), one (fragment, lane) per thread; as tile2frag.
template <bool TRANS>
__device__ __forceinline__ void stile2frag(uint16_t *dst, int KC, int rt0, int kc0, const uint16_t *p, int tid) {
    const int f = tid >> 6, lane = tid & 63, rtl = f >> 2, kcl = f & 3, h = lane >> 5;
    const int row = 32 * rtl + (lane & 31);
    u32x4 u;
    if constexpr (!TRANS) {
        // k = 16 kcl + frag_k(e, h): elements 0..3 at 16 kcl + 4 h .., 4..7 at 16 kcl + 8 + 4 h ..
        const u32x2 x = *reinterpret_cast<const u32x2 *>(p + sidx(row, 16 * kcl + 4 * h));
        const u32x2 y = *reinterpret_cast<const u32x2 *>(p + sidx(row, 16 * kcl + 8 + 4 * h));
        u = u32x4{x.x, x.y, y.x, y.y};
    } else {
        uint16_t x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[sidx(16 * kcl + frag_k(e, h), row)];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = (uint32_t)x[2 * t] | ((uint32_t)x[2 * t + 1] << 16);
    }
    stfrag<uint16_t>(dst, rt0 + rtl, kc0 + kcl, KC, lane, __builtin_bit_cast(i16x8, u));
}
// An fp32 64x64 tile without padding, columns swizzled by the row, so that one thread per row
// or one per column walking the tile hits 64 different banks.
__device__ __forceinline__ int fidx(int r, int c) { return r * kC + ((c ^ r) & 63); }

// Prep for bf16 inputs: the steps of bwd_prep_kernel with split tiles.  G and X stay fp32 for
// the triangular inverse (their space then holds P and A as split tiles); the diagonal dS is an
// fp32 tile, for the exact row and column sums; the matrices kept for the block backward go to
// the workspace straight from the accumulators.
template <int D>
__global__ __launch_bounds__(kT) void bwd_prep_kernel_bf16(BwdArgs a) {
    typedef uint16_t T;
    constexpr int NCH = D / 64, KCD = D / 16, TS = 2 * kSP;
    __shared__ __attribute__((aligned(16))) float sf[2 * kTile];  // G, then P (split); X, then A (split)
    __shared__ __attribute__((aligned(16))) uint16_t sm[7 * TS];
    __shared__ float sB[kC], sCl[kC], sL2[kC], sDD[kC];
    float *fG = sf, *fX = sf + kTile;
    uint16_t *bP = (uint16_t *)fG, *bA = (uint16_t *)fX;
    uint16_t *bW = sm, *bQ = bW + TS, *bK = bQ + TS, *bQW = bK + TS, *bN = bQW + TS, *bZ = bN + TS, *bY = bZ + TS;
    float *fS = (float *)bQW;  // the diagonal dS (fp32, fidx order), once Q W^T is done with
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * D, *k = (const T *)a.k + hoff * D, *w = (const T *)a.w + hoff * D;
    const T *v = (const T *)a.v + hoff * D, *o = (const T *)a.out + hoff * D, *dout = (const T *)a.dout + hoff * D;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float scale = a.scale;
    const int64_t tok = (int64_t)J * kC * kC;

    if (tid < kC) {
        const int i = row0 + tid;
        sB[tid] = i < L ? a.beta[hoff + i] : 0.f;
        sL2[tid] = i < L ? a.lse[hoff + i] * kLog2e : 0.f;
    }
    gate_prefix(sCl, a.logf ? a.logf + hoff : nullptr, row0, L, tid);
    {   // D_i = do_i . o_i - dlse_i: eight lanes per row, D / 8 columns each
        const int r = tid >> 3, c0 = (tid & 7) * (D / 8), i = row0 + r;
        float s = 0.f;
        if (i < L) {
#pragma unroll
            for (int c = 0; c < D / 8; c += 8) {
                float xo[8], xd[8];
                load8(xd, dout + (int64_t)i * D + c0 + c);
                load8(xo, o + (int64_t)i * D + c0 + c);
#pragma unroll
                for (int t = 0; t < 8; ++t) s += xd[t] * xo[t];
            }
        }
        s = sum8(s);
        if ((tid & 7) == 0) sDD[r] = i < L ? s - (a.dlse ? a.dlse[hoff + i] : 0.f) : 0.f;
    }
    // G = W W^T, Q W^T, N = K W^T and Q K^T, summed over the chunks of the head dimension
    f32x8 aG = zero8(), aQW = zero8(), aN = zero8(), aQK = zero8();
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        sin2l(bW, w, D, 64 * c, row0, L, tid);
        sin2l(bQ, q, D, 64 * c, row0, L, tid);
        sin2l(bK, k, D, 64 * c, row0, L, tid);
        __syncthreads();
        smm<true, true>(aG, snat(bW), str(bW), lane, wave);
        smm<true, true>(aQW, snat(bQ), str(bW), lane, wave);
        smm<true, true>(aN, snat(bK), str(bW), lane, wave);
        smm<true, true>(aQK, snat(bQ), str(bK), lane, wave);
    }
#pragma unroll
    for (int vv = 0; vv < 8; ++vv) {
        const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
        aQW[vv] = c <= r ? aQW[vv] : 0.f;  // Q W^T, r <= i
        aN[vv] = c > r ? aN[vv] : 0.f;     // N, r > j
    }
    store_lds(fG, aG, lane, wave, Id());
    sstore(bQW, aQW, lane, wave, Id());
    sstore(bN, aN, lane, wave, Id());
    acc2g((float *)(ws + ly.qwm) + tok, kC, aQW, lane, wave);
    acc2g((float *)(ws + ly.nn) + tok, kC, aN, lane, wave);
    __syncthreads();
    unit_upper_inverse(fX, fG, sB, tid);
    __syncthreads();
    {   // X and A = X diag(beta) to the workspace; A, split, into X's space
        const int r = tid >> 3, c8 = (tid & 7) * 8;
        float *XX = (float *)(ws + ly.xx) + tok + r * kC + c8, *AA = (float *)(ws + ly.aa) + tok + r * kC + c8;
        f32x4 x0 = *reinterpret_cast<const f32x4 *>(fX + r * kP + c8);
        f32x4 x1 = *reinterpret_cast<const f32x4 *>(fX + r * kP + c8 + 4);
        *reinterpret_cast<f32x4 *>(XX) = x0;
        *reinterpret_cast<f32x4 *>(XX + 4) = x1;
        float x[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[t] = x0[t] * sB[c8 + t];
            x[4 + t] = x1[t] * sB[c8 + 4 + t];
        }
        *reinterpret_cast<f32x4 *>(AA) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4 *>(AA + 4) = f32x4{x[4], x[5], x[6], x[7]};
        __syncthreads();  // every thread has read its part of X
        sput8(bA, r, c8, x);
    }
    __syncthreads();
    f32x8 acc = zero8();
    smm<false, false>(acc, snat(bQW), str(bA), lane, wave);  // Z = QWm A^T
    sstore(bZ, acc, lane, wave, Id());
    acc2g((float *)(ws + ly.zz) + tok, kC, acc, lane, wave);
    acc = zero8();
    smm<false, false>(acc, snat(bN), snat(bA), lane, wave);  // Y = N A
    sstore(bY, acc, lane, wave, Id());
    __syncthreads();
    // diagonal block: P = exp(scale (Q K^T - Z N^T) + cl_i - cl_j - lse_i) for j <= i (G is dead: P -> bP)
    f32x8 pv;
    {
        f32x8 sZN = zero8();
        smm<false, false>(sZN, snat(bZ), str(bN), lane, wave);
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            const float s = (scale * (aQK[vv] - sZN[vv]) + (sCl[r] - sCl[c])) * kLog2e - sL2[r];
            pv[vv] = c <= r ? fast_exp2(s) : 0.f;
        }
        sstore(bP, pv, lane, wave, Id());
    }
    // dP = dO V^T over the chunks; dS = P (dP - D_i) -> fS (Q W^T is stored)
    f32x8 aDP = zero8();
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        sin2l(bQ, dout, D, 64 * c, row0, L, tid);
        sin2l(bK, v, D, 64 * c, row0, L, tid);
        __syncthreads();
        smm<true, true>(aDP, snat(bQ), str(bK), lane, wave);
    }
#pragma unroll
    for (int vv = 0; vv < 8; ++vv) {
        const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
        const float ds = pv[vv] * (aDP[vv] - sDD[r]);
        fS[fidx(r, c)] = ds;
        aDP[vv] = scale * ds;
    }
    acc2g((float *)(ws + ly.ee) + tok, kC, aDP, lane, wave);
    __syncthreads();
    {
        float *rs = (float *)(ws + ly.rsd) + row0, *cs = (float *)(ws + ly.csd) + row0;
        if (tid < kC) {
            float s = 0.f;
            for (int c = 0; c < kC; ++c) s += fS[fidx(tid, c)];
            rs[tid] = s;
        } else if (tid < 2 * kC) {
            const int c = tid - kC;
            float s = 0.f;
            for (int r = 0; r < kC; ++r) s += fS[fidx(r, c)];
            cs[c] = s;
        } else if (tid < 3 * kC) {
            const int r = tid - 2 * kC;
            ((float *)(ws + ly.dd))[row0 + r] = sDD[r];
            ((float *)(ws + ly.cql))[row0 + r] = sCl[r] * kLog2e - sL2[r];
            ((float *)(ws + ly.ckl))[row0 + r] = (sCl[kC - 1] - sCl[r]) * kLog2e;
            if (r == 0) ((float *)(ws + ly.tot))[J] = sCl[kC - 1] * kLog2e;
        }
    }
    // chunks of the head dimension: q^, k^ (fragments), A W (kept for T), V and dO fragments,
    // the diagonal value gradient
    const int64_t fo = (int64_t)J * kC * D;  // this block's 64 x D fragment set
    T *REC = (T *)(ws + ly.urec) + J * ly.rec_elems;
    T *KH1 = REC, *V1 = REC + kC * D, *KH2 = REC + 2 * kC * D;
    T *DO1 = (T *)(ws + ly.do1) + fo;
    uint16_t *bAW[2] = {bN, bQW};  // A W of chunk 0 / 1 (N and dS are done with)
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        sin2l(bW, w, D, 64 * c, row0, L, tid);
        sin2l(bQ, q, D, 64 * c, row0, L, tid);
        sin2l(bK, k, D, 64 * c, row0, L, tid);
        __syncthreads();
        {
            f32x8 zw = zero8(), yw = zero8(), aw = zero8();
            smm<false, true>(zw, snat(bZ), snat(bW), lane, wave);
            smm<false, true>(yw, snat(bY), snat(bW), lane, wave);
            smm<false, true>(aw, snat(bA), snat(bW), lane, wave);
            float *QH = (float *)(ws + ly.qh) + (int64_t)row0 * D + 64 * c;
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) {  // each element read and rewritten by the same thread
                const int r = arow(vv, lane, wave), cc = acol(vv, lane, wave);
                QH[(int64_t)r * D + cc] = sld(bQ, r, cc) - zw[vv];  // q^ = q - Z W
                sst(bK, r, cc, sld(bK, r, cc) - yw[vv]);            // k^ = k - Y W
            }
            sstore(bAW[c], aw, lane, wave, Id());
        }
        __syncthreads();
        stile2frag<false>(KH1, KCD, 0, 4 * c, bK, tid);  // k^: rows keys, k over d
        stile2frag<true>(KH2, 4, 2 * c, 0, bK, tid);     // k^^T: rows d, k over keys
        __syncthreads();
        sin2l(bQ, v, D, 64 * c, row0, L, tid);
        sin2l(bK, dout, D, 64 * c, row0, L, tid);
        __syncthreads();
        stile2frag<false>(V1, KCD, 0, 4 * c, bQ, tid);   // V: rows keys
        stile2frag<false>(DO1, KCD, 0, 4 * c, bK, tid);  // dO: rows queries
        acc = zero8();
        smm<false, true>(acc, str(bP), snat(bK), lane, wave);  // diagonal value gradient P^T dO
        acc2g((float *)(ws + ly.dvd) + (int64_t)row0 * D + 64 * c, D, acc, lane, wave);
    }
    // T - I = -W^T (A W) and its transpose, block (c1, c2) = rows of chunk c1, columns of chunk c2
    T *NT = (T *)(ws + ly.nt) + (int64_t)J * D * D, *NTT = REC + 3 * kC * D;
    for (int c1 = 0; c1 < NCH; ++c1) {
        __syncthreads();
        sin2l(bW, w, D, 64 * c1, row0, L, tid);
        __syncthreads();
        for (int c2 = 0; c2 < NCH; ++c2) {
            acc = zero8();
            smm<true, false>(acc, str(bW), snat(bAW[c2]), lane, wave);
            sstore(bQ, acc, lane, wave, [](int, int, float x) { return -x; });
            __syncthreads();
            stile2frag<false>(NT, KCD, 2 * c1, 4 * c2, bQ, tid);  // (T - I): rows d_out, k over d_in
            stile2frag<true>(NTT, KCD, 2 * c2, 4 * c1, bQ, tid);  // (T - I)^T
            __syncthreads();
        }
    }
}

template <int D>
__global__ __launch_bounds__(kT) void bwd_block_kernel_bf16(BwdArgs a) {
    typedef uint16_t T;
    constexpr int NCH = D / 64;
    constexpr int TS = 2 * kSP;  // elements of a split tile
    __shared__ __attribute__((aligned(16))) uint16_t sm[9 * TS];
    __shared__ float sB[kC], sRed[kC];
    uint16_t *bE = sm, *bN = bE + TS, *bZ = bN + TS, *bX = bZ + TS, *bA = bX + TS, *bQW = bA + TS, *b6 = bQW + TS,
             *b7 = b6 + TS, *b8 = b7 + TS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, nb = a.nb, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * D, *k = (const T *)a.k + hoff * D, *w = (const T *)a.w + hoff * D;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const bool hasQ = J >= 1, hasK = J <= nb - 2, hasT = J >= 1 && J <= nb - 2;
    const int64_t tok = (int64_t)J * kC * kC, nat0 = (int64_t)row0 * D;
    const float *dqo = (const float *)(ws + ly.dqo) + nat0, *dko = (const float *)(ws + ly.dko) + nat0;

    if (tid < kC) sB[tid] = row0 + tid < L ? a.beta[hoff + row0 + tid] : 0.f;
    sg2l(bE, (const float *)(ws + ly.ee) + tok, kC, tid);  // scale dS of the diagonal block
    sg2l(bN, (const float *)(ws + ly.nn) + tok, kC, tid);
    sg2l(bZ, (const float *)(ws + ly.zz) + tok, kC, tid);
    sg2l(bX, (const float *)(ws + ly.xx) + tok, kC, tid);
    sg2l(bA, (const float *)(ws + ly.aa) + tok, kC, tid);
    sg2l(bQW, (const float *)(ws + ly.qwm) + tok, kC, tid);
    __syncthreads();
    // ---- token-level quantities
    f32x8 aZ = zero8(), aNn = zero8(), aY = zero8(), aG = zero8(), aA = zero8(), acc;
    smm<false, false>(aZ, snat(bE), snat(bN), lane, wave);  // E N         (dZ = -(E N + dq^ W^T))
    smm<false, false>(aNn, str(bE), snat(bZ), lane, wave);  // E^T Z       (dN = -E^T Z + dY A^T)
    for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        sin2l(b6, w, D, 64 * c, row0, L, tid);
        if (hasQ) sg2l(b7, dqo + 64 * c, D, tid);
        else szero(b7, tid);
        if (hasK) sg2l(b8, dko + 64 * c, D, tid);
        else szero(b8, tid);
        __syncthreads();
        smm<false, true>(aZ, snat(b7), str(b6), lane, wave);  // + dq^ W^T
        smm<false, true>(aY, snat(b8), str(b6), lane, wave);  // dk^ W^T   (dY = -dk^ W^T)
        smm<true, true>(aG, snat(b6), str(b6), lane, wave);   // G = W W^T
    }
    if (hasT) {
        // U = W dT and V' = W dT^T (64 x D, for the backward through T = I - W^T A W) and
        // U W^T = W dT W^T; the key walk left dT^T, so dT[c2, c] = (dT^T[c, c2])^T
        const float *dtt = (const float *)(ws + ly.dtt) + (int64_t)J * D * D;
        float *uu = (float *)(ws + ly.uu) + nat0, *vv = (float *)(ws + ly.vv) + nat0;
        for (int c = 0; c < NCH; ++c) {
            f32x8 aU = zero8(), aV = zero8();
            for (int c2 = 0; c2 < NCH; ++c2) {
                __syncthreads();
                sin2l(b6, w, D, 64 * c2, row0, L, tid);
                sg2l(b7, dtt + (int64_t)(64 * c) * D + 64 * c2, D, tid);  // dT^T block (c, c2)
                sg2l(b8, dtt + (int64_t)(64 * c2) * D + 64 * c, D, tid);  // dT^T block (c2, c)
                __syncthreads();
                smm<true, false>(aU, snat(b6), str(b7), lane, wave);   // W_c2 dT[c2, c]
                smm<true, false>(aV, snat(b6), snat(b8), lane, wave);  // W_c2 dT^T[c2, c]
            }
            acc2g(uu + 64 * c, D, aU, lane, wave);
            acc2g(vv + 64 * c, D, aV, lane, wave);
            __syncthreads();
            sstore(b7, aU, lane, wave, Id());
            sin2l(b6, w, D, 64 * c, row0, L, tid);
            __syncthreads();
            acc = zero8();
            smm<false, true>(acc, snat(b7), str(b6), lane, wave);  // U_c W_c^T
#pragma unroll
            for (int v = 0; v < 8; ++v) aA[v] -= acc[v];  // dA = -W dT W^T + ...
        }
    }
    __syncthreads();
    sstore(b6, aY, lane, wave, [](int, int, float x) { return -x; });  // dY
    sstore(b7, aZ, lane, wave, [](int, int, float x) { return -x; });  // dZ
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 8; ++v) aNn[v] = -aNn[v];
    smm<false, false>(aNn, snat(b6), str(bA), lane, wave);   // dN = -E^T Z + dY A^T
    smm<false, false>(aA, str(bN), snat(b6), lane, wave);    // dA += N^T dY
    smm<false, false>(aA, str(b7), snat(bQW), lane, wave);   // dA += dZ^T QWm
    acc = zero8();
    smm<false, false>(acc, snat(b7), snat(bA), lane, wave);  // dQWm = (dZ A) o [r <= i]
    f32x8 aYv = zero8();
    smm<false, false>(aYv, snat(bN), snat(bA), lane, wave);  // Y = N A
    __syncthreads();
    sstore(b8, acc, lane, wave, [](int r, int c, float x) { return c <= r ? x : 0.f; });  // dQWm
    sstore(b6, aNn, lane, wave, [](int r, int c, float x) { return c > r ? x : 0.f; });   // dKW = dN o [r > j]
    sstore(bN, aYv, lane, wave, Id());                                                    // Y (N is done with)
    // A = X diag(beta): dX = dA diag(beta), dbeta_c += sum_r X_rc dA_rc (dA kept on the upper triangle)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        aA[v] = c >= r ? aA[v] : 0.f;
        sst(b7, r, c, aA[v] * sB[c]);
        sst(bQW, r, c, sld(bX, r, c) * aA[v]);
    }
    __syncthreads();
    float dbeta = 0.f;
    if (tid < kC)
        for (int r = 0; r < kC; ++r) dbeta += sld(bQW, r, tid);
    acc = zero8();
    smm<false, false>(acc, str(bX), snat(b7), lane, wave);  // X^T dX
    __syncthreads();
    sstore(bQW, acc, lane, wave, Id());
    __syncthreads();
    f32x8 dTp = zero8();
    smm<false, false>(dTp, snat(bQW), str(bX), lane, wave);  // (X^T dX) X^T; dT' is its negative
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        const float t = -dTp[v];
        sst(bQW, r, c, c > r ? t * aG[v] : 0.f);  // dbeta_r += sum_c dT'_rc G_rc
        sst(b7, r, c, c > r ? sB[r] * t : 0.f);   // dG = diag(beta) dT' on the strict upper triangle
    }
    __syncthreads();
    if (tid >= kC && tid < 2 * kC) {
        float s = 0.f;
        for (int c = 0; c < kC; ++c) s += sld(bQW, tid - kC, c);
        sRed[tid - kC] = s;
    }
    __syncthreads();
    if (tid < kC && row0 + tid < L) a.dbeta[hoff + row0 + tid] = dbeta + sRed[tid];
    // ---- chunks of the head dimension.  LDS: E, Y (bN), Z, A, dKW (b6), dG (b7), dQWm (b8);
    //      bX and bQW hold the chunk operands.
    const float *uu = (const float *)(ws + ly.uu) + nat0, *vvp = (const float *)(ws + ly.vv) + nat0;
    for (int c = 0; c < NCH; ++c) {
        f32x8 dQ = zero8(), dK = zero8(), dW = zero8();
        __syncthreads();
        sin2l(bX, k, D, 64 * c, row0, L, tid);
        sin2l(bQW, q, D, 64 * c, row0, L, tid);
        __syncthreads();
        smm<false, true>(dQ, snat(bE), snat(bX), lane, wave);  // E K
        smm<false, true>(dK, str(bE), snat(bQW), lane, wave);  // E^T Q
        smm<false, true>(dW, str(b6), snat(bX), lane, wave);   // dKW^T K
        smm<false, true>(dW, str(b8), snat(bQW), lane, wave);  // dQWm^T Q
        __syncthreads();
        sin2l(bX, w, D, 64 * c, row0, L, tid);
        __syncthreads();
        smm<false, true>(dQ, snat(b8), snat(bX), lane, wave);  // dQWm W
        smm<false, true>(dK, snat(b6), snat(bX), lane, wave);  // dKW W
        smm<false, true>(dW, snat(b7), snat(bX), lane, wave);  // (dG + dG^T) W
        smm<false, true>(dW, str(b7), snat(bX), lane, wave);
        __syncthreads();
        if (hasQ) sg2l(bX, dqo + 64 * c, D, tid);
        else szero(bX, tid);
        if (hasK) sg2l(bQW, dko + 64 * c, D, tid);
        else szero(bQW, tid);
        __syncthreads();
        acc = zero8();
        smm<false, false>(acc, str(bZ), snat(bX), lane, wave);   // Z^T dq^
        smm<false, false>(acc, str(bN), snat(bQW), lane, wave);  // + Y^T dk^ (= A^T N^T dk^)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int r = arow(v, lane, wave), cc = acol(v, lane, wave);
            dQ[v] += sld(bX, r, cc);
            dK[v] += sld(bQW, r, cc);
            dW[v] -= acc[v];
        }
        if (hasT) {
            __syncthreads();
            sg2l(bX, uu + 64 * c, D, tid);
            sg2l(bQW, vvp + 64 * c, D, tid);
            __syncthreads();
            acc = zero8();
            smm<false, false>(acc, snat(bA), snat(bQW), lane, wave);  // A W dT^T
            smm<false, false>(acc, str(bA), snat(bX), lane, wave);    // + A^T W dT
#pragma unroll
            for (int v = 0; v < 8; ++v) dW[v] -= acc[v];
        }
        acc2out((T *)a.dq + hoff * D + 64 * c, D, dQ, row0, L, lane, wave);
        acc2out((T *)a.dk + hoff * D + 64 * c, D, dK, row0, L, lane, wave);
        acc2out((T *)a.dw + hoff * D + 64 * c, D, dW, row0, L, lane, wave);
    }
    {
        const float *dvd = (const float *)(ws + ly.dvd) + nat0, *dvo = (const float *)(ws + ly.dvo) + nat0;
        T *dv = (T *)a.dv + hoff * D;
        for (int e = tid; e < kC * D; e += kT) {
            const int r = e / D;
            if (row0 + r < L) dv[(int64_t)row0 * D + e] = Elem<T>::from_float(dvd[e] + (hasK ? dvo[e] : 0.f));
        }
    }
    if (tid < kC) {
        const int i = row0 + tid;
        const float rs = ((const float *)(ws + ly.rsd))[i] + (hasQ ? ((const float *)(ws + ly.rso))[i] : 0.f);
        const float cs = ((const float *)(ws + ly.csd))[i] + (hasK ? ((const float *)(ws + ly.cso))[i] : 0.f);
        ((float *)(ws + ly.dc))[i] = rs - cs;
    }
}

// dlogf_t = sum_{t' >= t} dc_t' for one head: 512 threads, contiguous chunks, fixed order.
__global__ __launch_bounds__(kT) void bwd_gate_kernel(BwdArgs a) {
    __shared__ float part[kT];
    const int tid = threadIdx.x, gl = blockIdx.x, L = a.L;
    const int64_t hoff = (int64_t)(a.g0 + gl) * L;
    const float *dc = (const float *)((const char *)a.ws + (int64_t)gl * a.ly.head + a.ly.dc);
    const int ch = (L + kT - 1) / kT, t0 = tid * ch, t1 = min(L, t0 + ch);
    float s = 0.f;
    for (int t = t1 - 1; t >= t0; --t) s += dc[t];
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {  // exclusive suffix sums of the chunk totals, in place
        float run = 0.f;
        for (int u = kT - 1; u >= 0; --u) {
            const float x = part[u];
            part[u] = run;
            run += x;
        }
    }
    __syncthreads();
    float run = part[tid];
    for (int t = t1 - 1; t >= t0; --t) {
        run += dc[t];
        a.dlogf[hoff + t] = run;
    }
}

// Key walk for bf16 inputs: as bwd_key_kernel (the same waves: query half qt = w & 1,
// key half kt = (w >> 1) & 1, head-dimension group dh = w >> 2), but each step's
// operands -- the pair's q~ (rows queries) and G, the query block's dO (rows queries),
// its exponent terms and the pair's gate sum: 24.8 KiB at d = 64, 48.8 KiB at d = 128 --
// are copied global -> LDS one step ahead (global_load_lds, double-buffered) and read by
// every wave from there.  The fragments with k over queries -- q~^T, G^T and dO^T (rows
// d) -- are gathered from those copies with transposing LDS reads, so the down and up
// walks store q~ and G in one orientation only and dO^T is not stored at all.  At d = 128
// the registers do not hold k^ and V of the key tile besides the accumulators: they are
// read from an LDS copy.
template <int D>
__global__ __launch_bounds__(64 * KeyCfg<D>::NW) void bwd_key_kernel_lds(BwdArgs a) {
    typedef uint16_t S;
    typedef Elem<S>::Frag Frag;
    typedef KeyCfg<D> K;
    constexpr int KCD = D / 16, RTD = D / 32, RTW = K::RTW, NTH = 64 * K::NW;
    static_assert(K::TRW == 1, "one row tile of dT per wave");
    constexpr int NACC = 2 * RTW + RTD;      // dV^T, dk^^T (RTW each), dT row tile grp (RTD column tiles)
    constexpr bool KVL = D == 128;           // k^, V from LDS
    constexpr int NSET = 3;                  // fragment sets per buffer: q~, G, dO
    constexpr int FR = kC * D;               // elements of a 64 x D fragment set
    constexpr int NLD = FR * 2 / 16 / NTH;   // 16-byte copies per thread and fragment set
    static_assert(FR * 2 % (16 * NTH) == 0, "a fragment set must split evenly over the workgroup");
    // a buffer: q~, G, dO (rows queries), then 64 floats each of the query
    // terms dd and cq and of the gate sum (the same value 64 times); with KVL, k^ and V of the
    // key block after the two buffers
    constexpr int BUF = NSET * FR * 2 + 3 * 4 * kC;
    constexpr int KVB = KVL ? 2 * FR * 2 : 0;
    static_assert(K::NW / 2 * 16 * 65 * 4 <= 2 * BUF, "the final reduction reuses the buffers");
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF + KVB];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int qt = w & 1, kt = (w >> 1) & 1, dh = w >> 2, grp = kt + 2 * dh;
    const int nb = a.nb, hc = a.hc;
    int gl, J;  // head and key block; J = 0 (the longest walk) first
    walk_item(nb - 1, hc, K::NW == 4 ? 2 : 1, gl, J);
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const S *QS1 = (const S *)(ws + ly.qs1), *GS2 = (const S *)(ws + ly.gs2);
    const S *DO1 = (const S *)(ws + ly.do1);
    const float *MID = (const float *)(ws + ly.mid);
    const float *DD = (const float *)(ws + ly.dd), *CQL = (const float *)(ws + ly.cql);
    const float scale = a.scale, c2 = scale * kLog2e;
    const int key = J * kC + 32 * kt + l32;  // this lane's key (column of the logit tile)
    const float ck = ((const float *)(ws + ly.ckl))[key];

    // copies of query block I's step into buffer B (I <= nb - 1, so every source is in the
    // workspace; for J = 0 the G^T slot holds no adjoint and is not used)
    auto issue = [&](int I, int B) {
        unsigned char *buf = smem + B * BUF;
        const int64_t po = pair_index(I, J) * FR, bo = (int64_t)I * FR;
        dma_record<NTH, NLD>(QS1 + po, buf, tid);
        dma_record<NTH, NLD>(GS2 + po, buf + FR * 2, tid);
        dma_record<NTH, NLD>(DO1 + bo, buf + 2 * FR * 2, tid);
        const float *src = w == 0 ? DD + I * kC + lane : w == 1 ? CQL + I * kC + lane : MID + pair_index(I, J);
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(buf + NSET * FR * 2 + 4 * kC * min(w, 2)), 4, 0,
                                         0);
    };
    const S *rec = (const S *)(ws + ly.urec) + J * ly.rec_elems;  // k^ (rows keys, k over d), then V
    const S *skv = (const S *)(smem + 2 * BUF);
    if constexpr (KVL) dma_record<NTH, 2 * NLD>(rec, smem + 2 * BUF, tid);
    issue(nb - 1, 0);
    // k^ and V of key tile kt, k over d: the B operands of S and dP (registers, or the LDS copy)
    Frag kf[KVL ? 1 : KCD], vf[KVL ? 1 : KCD];
    if constexpr (!KVL) {
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            kf[kc] = ldfrag<S>(rec, kt, kc, KCD, lane);
            vf[kc] = ldfrag<S>(rec + kC * D, kt, kc, KCD, lane);
        }
    }
    f32x16 acc[NACC];
#pragma unroll
    for (int t = 0; t < NACC; ++t) acc[t] = f32x16{};
    float csum = 0.f;
    // q~^T fragment (rows d = 32 ct + lane % 32, k over queries 16 kq ..) gathered from the q~ copy
    // (fragments of rows queries, k over d) with two transposing LDS reads.  ds_read_b64_tr_b16
    // works on groups of 16 lanes: lane 16 g + i receives element i % 4 of the 8-byte chunks that
    // lanes 16 g + 4 t + i / 4 (t = 0..3) address, as its elements t.  Element t of the first read
    // must be q~[16 kq + 4 (lane / 32) + t][d] (the second: 8 queries on), so lane s = 16 g + 4 t + m
    // addresses the four consecutive d = 32 ct + 16 (g & 1) + 4 m .. of query 16 kq + 4 (g >> 1) + t,
    // which sit together in the q~ fragment of d chunk 2 ct + (g & 1) at lane (query % 32) +
    // 32 (m & 1), elements 4 (m >> 1) ..
    // The reads are issued by inline assembly and waited for by an explicit lgkmcnt(0) tied to
    // their results (the compiler would otherwise wait for every copy in flight before each
    // one); LDS operations complete in order, so the compiler's own counts stay safe.
    const int tg = lane >> 4, tt = (lane >> 2) & 3, tm = lane & 3;
    const int troff = ((tg & 1) * 64 + 4 * (tg >> 1) + tt + 32 * (tm & 1)) * 8 + 4 * (tm >> 1);
    struct TrF {
        u32x2 lo, hi;
    };
    auto tr_issue = [&](const S *sq, int ct, int kq) {
        const S *p = sq + (((kq >> 1) * KCD + 2 * ct) * 64 + 16 * (kq & 1)) * 8 + troff;
        const unsigned la = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) S *)p;
        TrF t;
        asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:128"  // queries + 8
                     : "=&v"(t.lo), "=&v"(t.hi)
                     : "v"(la));
        return t;
    };
    auto tr_wait2 = [](TrF &a, TrF &b) {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a.lo), "+v"(a.hi), "+v"(b.lo), "+v"(b.hi));
    };
    auto tr_frag = [](const TrF &t) { return __builtin_bit_cast(Frag, u32x4{t.lo.x, t.lo.y, t.hi.x, t.hi.y}); };
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
    // one step over query block I, whose copies are in buffer B ((nb - 1 - I) % 2); it refills the
    // other.  The walk runs I = nb - 1 .. J + 1, so that the key walks of a head start on the same
    // query block and read its dO and query terms at about the same time.
    auto step = [&](int I, auto bsel) {
        constexpr int B = decltype(bsel)::value;
        const unsigned char *buf = smem + B * BUF;
        const S *sq = (const S *)buf, *sg = sq + FR, *so1 = sq + 2 * FR;
        const float *sdd = (const float *)(buf + NSET * FR * 2), *scq = sdd + kC, *smid = scq + kC;
        // this wave's copies of step I have landed and its LDS reads of the previous step have
        // returned; after the barrier every wave's copies have landed and the other buffer is free
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
        asm volatile("s_barrier" ::: "memory");
        issue(max(I - 1, J + 1), 1 - B);
        asm volatile("" ::: "memory");
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) {
            const Frag kb = KVL ? ldfrag<S>(skv, kt, kc, KCD, lane) : kf[KVL ? 0 : kc];
            const Frag vb = KVL ? ldfrag<S>(skv + FR, kt, kc, KCD, lane) : vf[KVL ? 0 : kc];
            Elem<S>::mma(s, ldfrag<S>(sq, qt, kc, KCD, lane), kb);
            Elem<S>::mma(dp, ldfrag<S>(so1, qt, kc, KCD, lane), vb);
        }
        const float mid = smid[0];
        // P and dS (rows: queries 32 qt + acc_row(r, h) of block I; column: this lane's key)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 ddv = *reinterpret_cast<const f32x4 *>(sdd + 32 * qt + 8 * g4 + 4 * h);
            const f32x4 cqv = *reinterpret_cast<const f32x4 *>(scq + 32 * qt + 8 * g4 + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                const float P = fast_exp2(c2 * s[r] + cqv[e] + ck + mid);
                const float ds = P * (dp[r] - ddv[e]);
                csum += ds;
                s[r] = ds;
                dp[r] = P;
            }
        }
        Frag pf[2], sf[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            pf[cc] = acc_frag<S>(dp, cc);
            sf[cc] = acc_frag<S>(s, cc);
        }
        // dV^T += dO^T P^T (dO^T gathered from the dO copy)
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            TrF t0 = tr_issue(so1, dh * RTW + i, 2 * qt), t1 = tr_issue(so1, dh * RTW + i, 2 * qt + 1);
            tr_wait2(t0, t1);
            const Frag ob[2] = {tr_frag(t0), tr_frag(t1)};
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) Elem<S>::mma(acc[i], ob[cc], pf[cc]);
        }
        // G^T (rows d of tile grp, k over queries) and the first column tile of q~^T
        Frag ga[2];
        TrF qn0 = tr_issue(sq, 0, 2 * qt), qn1 = tr_issue(sq, 0, 2 * qt + 1);
        {
            TrF g0 = tr_issue(sg, grp, 2 * qt), g1 = tr_issue(sg, grp, 2 * qt + 1);
            tr_wait2(g0, g1);
            ga[0] = tr_frag(g0);
            ga[1] = tr_frag(g1);
        }
        tr_wait2(qn0, qn1);
        // per column tile of q~^T: dT (row tile grp) and, for the wave's own tiles, dk^; the next
        // tile's reads are in flight during this tile's products
#pragma unroll
        for (int ct = 0; ct < RTD; ++ct) {
            const Frag q2[2] = {tr_frag(qn0), tr_frag(qn1)};
            if (ct + 1 < RTD) {
                qn0 = tr_issue(sq, ct + 1, 2 * qt);
                qn1 = tr_issue(sq, ct + 1, 2 * qt + 1);
            }
            if (ct / RTW == dh) {  // wave-uniform
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) Elem<S>::mma(acc[RTW + ct % RTW], q2[cc], sf[cc]);
            }
            if (J >= 1) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) Elem<S>::mma(acc[2 * RTW + ct], ga[cc], q2[cc]);
            }
            if (ct + 1 < RTD) tr_wait2(qn0, qn1);
        }
    };
    for (int I = nb - 1; I > J; I -= 2) {
        step(I, std::integral_constant<int, 0>{});
        if (I - 1 > J) step(I - 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));  // the last (unused) copy has landed
    csum = other_half_sum(csum);  // lanes l and l ^ 32 hold the other queries of the same key
    // add the query half qt = 1 (wave w + 1) into qt = 0 (wave w), one tile at a time, through
    // the buffers (free now)
    float *red = (float *)smem + (w >> 1) * 16 * 65;
    for (int t = 0; t <= NACC; ++t) {
        __syncthreads();
        if (qt == 1) {
            if (t < NACC) {
#pragma unroll
                for (int r = 0; r < 16; ++r) red[r * 65 + lane] = acc[t][r];
            } else {
                red[lane] = csum;
            }
        }
        __syncthreads();
        if (qt == 0) {
            if (t < NACC) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] += red[r * 65 + lane];
            } else {
                csum += red[lane];
            }
        }
    }
    if (qt != 0) return;
    float *dvo = (float *)(ws + ly.dvo) + (int64_t)key * D, *dko = (float *)(ws + ly.dko) + (int64_t)key * D;
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * (dh * RTW + i) + 8 * g4 + 4 * h;
            const f32x4 xv = {acc[i][4 * g4], acc[i][4 * g4 + 1], acc[i][4 * g4 + 2], acc[i][4 * g4 + 3]};
            const f32x4 xk = {scale * acc[RTW + i][4 * g4], scale * acc[RTW + i][4 * g4 + 1],
                              scale * acc[RTW + i][4 * g4 + 2], scale * acc[RTW + i][4 * g4 + 3]};
            *reinterpret_cast<f32x4 *>(dvo + d0) = xv;
            *reinterpret_cast<f32x4 *>(dko + d0) = xk;
        }
    if (J >= 1) {  // dT^T: element (c, r) = dT[r][c]; lane c writes 4 consecutive r
        float *dtt = (float *)(ws + ly.dtt) + (int64_t)J * D * D;
#pragma unroll
        for (int ct = 0; ct < RTD; ++ct)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x16 &x = acc[2 * RTW + ct];
                const f32x4 y = {x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]};
                *reinterpret_cast<f32x4 *>(dtt + (int64_t)(32 * ct + l32) * D + 32 * grp + 8 * g4 + 4 * h) = y;
            }
    }
    if (dh == 0 && h == 0) ((float *)(ws + ly.cso))[J * kC + 32 * kt + l32] = csum;
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs &a0, hipStream_t st) {
    BwdArgs a = a0;
    const int G = a.B * a.H;
    for (int g0 = 0; g0 < G; g0 += a.hc_max) {
        a.g0 = g0;
        a.hc = min(a.hc_max, G - g0);
        if constexpr (sizeof(T) == 2) hipLaunchKernelGGL(bwd_prep_kernel_bf16<D>, dim3(a.nb, a.hc), dim3(kT), 0, st, a);
        else hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3(a.nb, a.hc), dim3(kT), 0, st, a);
        if (a.nb > 1) {
            const dim3 walks((unsigned)((a.nb - 1) * a.hc));
            if constexpr (sizeof(T) == 2) {
                // bf16: the LDS-staged walks (four query blocks per workgroup for the down and up walks)
                const dim3 tiles((unsigned)((a.nb - 1 + kUpQB - 1) / kUpQB * a.hc));
                hipLaunchKernelGGL(bwd_down_kernel_lds<D>, tiles, dim3(64 * 2 * kUpQB), 0, st, a);
                if constexpr (D == 64) hipLaunchKernelGGL(bwd_up_kernel_lds, tiles, dim3(64 * 2 * kUpQB), 0, st, a);
                else hipLaunchKernelGGL(bwd_up_kernel_split, tiles, dim3(64 * 2 * kUpQB), 0, st, a);
                hipLaunchKernelGGL(bwd_key_kernel_lds<D>, walks, dim3(64 * KeyCfg<D>::NW), 0, st, a);
            } else {
                hipLaunchKernelGGL((bwd_down_kernel<T, D, true>), walks, dim3(128), 0, st, a);
                hipLaunchKernelGGL((bwd_up_kernel<T, D>), walks, dim3(128), 0, st, a);
                hipLaunchKernelGGL((bwd_key_kernel<T, D>), walks, dim3(64 * KeyCfg<D>::NW), 0, st, a);
            }
        }
        if constexpr (sizeof(T) == 2) hipLaunchKernelGGL(bwd_block_kernel_bf16<D>, dim3(a.nb, a.hc), dim3(kT), 0, st, a);
        else hipLaunchKernelGGL((bwd_block_kernel<T, D>), dim3(a.nb, a.hc), dim3(kT), 0, st, a);
        if (a.dlogf) hipLaunchKernelGGL(bwd_gate_kernel, dim3(a.hc), dim3(kT), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t st) {
    if (a.d == 64) return bf16 ? launch_bwd_t<uint16_t, 64>(a, st) : launch_bwd_t<float, 64>(a, st);
    if (a.d == 128) return bf16 ? launch_bwd_t<uint16_t, 128>(a, st) : launch_bwd_t<float, 128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace path
