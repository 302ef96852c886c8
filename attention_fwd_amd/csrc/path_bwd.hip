// path_bwd.hip -- backward pass of PaTH attention (gradients of q, k, v, w,
// beta and the log forget gate), gfx950.
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
//   T_J  = H_s ... H_e          = I - W^T A W                (d x d, dense)
//   diagonal logits  s_ij = scale (Q K^T - Z N^T)_ij + gate,  j <= i
// For query block I and key block J < I the logits are scale q~ . k^ with the
// query carried down q~^(J-1) = T_J q~^(J), q~^(I-1) = q^.  The adjoint of
// q~^(J) obeys G^(J) = G^(J-1) T_J + scale dS_IJ K^_J (rows), running upward
// while q~ runs downward, so:
//   prep (per block): the quantities above (X, A, Q W^T o mask, N and Z kept
//     for the block backward), the diagonal block's dS, its value gradient,
//     and copies of v and do;
//   query-major walk (per query block I): a down walk J = I-1 .. 0 storing
//     q~^(J) for every pair (its own kernel: one product per step, so several
//     workgroups per compute unit), then the up walk J = 0 .. I-1 storing
//     G^(J-1), P and dS for every pair and ending with dq^_I = G^(I-1);
//   key-major walk (per key block J): over I > J, dV_J += P^T dO_I,
//     dk^_J += scale dS^T q~, dT_J += G^(J-1)^T q~ -- sums owned by one
//     workgroup, so no atomics; P and dS come from the query-major walk;
//   block backward (per block): the matrix-form chain rule through the
//     formulas above (including the triangular inverse: dT' = -X^T dX X^T)
//     gives dq, dk, dw, dbeta; dv adds the two value sums; the gate's
//     per-token adjoint dc_t = rowsum_t(dS) - colsum_t(dS);
//   gate: dlogf_t = sum_{t' >= t} dc_t' (one workgroup per head).
// Every contraction is a 64x64x64 fp32 product on the matrix cores
// (v_mfma_f32_16x16x4f32, eight waves sharing each product) with operands in
// LDS; the arithmetic is fp32 for either input type.  The walks exchange q~,
// G, P and dS of every pair through the workspace in the input type: fp32,
// or bf16 for bf16 inputs (the forward's own scan feeds q~ to its logit
// products in bf16 too); the column sums of dS the gate needs stay fp32.
// Head dimension 64.
#include <hip/hip_runtime.h>

#include "path_bwd.h"
#include "path_common.h"

namespace path {
namespace {

constexpr int kC = 64;   // tokens per block
constexpr int kD = 64;   // head dimension
constexpr int kP = 68;   // LDS row stride of a 64x64 fp32 tile: rows 16-byte aligned, columns conflict-free
constexpr int kT = 512;  // threads per workgroup (8 waves, two per SIMD)
constexpr int kTile = kC * kP;

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
// product and each SIMD holds two waves.  The contraction runs in four
// blocks of sixteen k; in block g, MFMA t (0..3) takes k = 16g + 4q + t from
// lane group q = lane / 16, the same order for both operands.  An operand
// whose k index is contiguous in LDS (A stored by rows, B stored by columns)
// is read with one 16-byte load per four MFMAs; otherwise with four single
// loads, whose sixteen lanes walk a row and so hit distinct banks.
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

// Global fp32 tile [64][64] (row stride 64) <-> LDS.
__device__ __forceinline__ void g2l(float *buf, const float *g, int tid) {
#pragma unroll
    for (int e = tid; e < kC * kD / 4; e += kT) {
        const int r = e >> 4, c = (e & 15) * 4;
        *reinterpret_cast<f32x4 *>(buf + r * kP + c) = *reinterpret_cast<const f32x4 *>(g + r * kD + c);
    }
}
// One thread's share of a 64x64 fp32 tile, so the next step's tiles can be
// fetched from global memory while the current step computes.
struct Stage {
    f32x4 v[kC * kD / 4 / kT];
};
__device__ __forceinline__ void gload(Stage &t, const float *g, int tid) {
#pragma unroll
    for (int u = 0; u < kC * kD / 4 / kT; ++u) {
        const int e = tid + u * kT, r = e >> 4, c = (e & 15) * 4;
        t.v[u] = *reinterpret_cast<const f32x4 *>(g + r * kD + c);
    }
}
__device__ __forceinline__ void lstore(float *buf, const Stage &t, int tid) {
#pragma unroll
    for (int u = 0; u < kC * kD / 4 / kT; ++u) {
        const int e = tid + u * kT, r = e >> 4, c = (e & 15) * 4;
        *reinterpret_cast<f32x4 *>(buf + r * kP + c) = t.v[u];
    }
}
// The same for a 64x64 tile stored as bf16 (the walks' scratch for bf16 inputs):
// 8 KiB, one 16-byte load of eight elements per thread.
struct Stage16 {
    u32x4 v;
};
__device__ __forceinline__ void gload(Stage16 &t, const uint16_t *g, int tid) {
    t.v = *reinterpret_cast<const u32x4 *>(g + tid * 8);
}
__device__ __forceinline__ void lstore(float *buf, const Stage16 &t, int tid) {
    const int r = tid >> 3, c = (tid & 7) * 8;
    f32x4 lo, hi;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lo[2 * u] = __uint_as_float(t.v[u] << 16);
        lo[2 * u + 1] = __uint_as_float(t.v[u] & 0xffff0000u);
        hi[2 * u] = __uint_as_float(t.v[2 + u] << 16);
        hi[2 * u + 1] = __uint_as_float(t.v[2 + u] & 0xffff0000u);
    }
    *reinterpret_cast<f32x4 *>(buf + r * kP + c) = lo;
    *reinterpret_cast<f32x4 *>(buf + r * kP + c + 4) = hi;
}
template <typename SC>
struct StageOf {
    typedef Stage T;
};
template <>
struct StageOf<uint16_t> {
    typedef Stage16 T;
};

// LDS fp32 tile -> global 64x64 tile of the scratch type, eight consecutive
// elements per thread (one 16-byte store for bf16, two for fp32).
__device__ __forceinline__ void l2g_sc(float *g, const float *buf, int tid) {
    const int r = tid >> 3, c = (tid & 7) * 8;
    *reinterpret_cast<f32x4 *>(g + r * kD + c) = *reinterpret_cast<const f32x4 *>(buf + r * kP + c);
    *reinterpret_cast<f32x4 *>(g + r * kD + c + 4) = *reinterpret_cast<const f32x4 *>(buf + r * kP + c + 4);
}
__device__ __forceinline__ void l2g_sc(uint16_t *g, const float *buf, int tid) {
    const int r = tid >> 3, c = (tid & 7) * 8;
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(buf + r * kP + c), hi = *reinterpret_cast<const f32x4 *>(buf + r * kP + c + 4);
    u32x4 u;
    u[0] = pack_bf16(lo[0], lo[1]);
    u[1] = pack_bf16(lo[2], lo[3]);
    u[2] = pack_bf16(hi[0], hi[1]);
    u[3] = pack_bf16(hi[2], hi[3]);
    *reinterpret_cast<u32x4 *>(g + r * kD + c) = u;
}

__device__ __forceinline__ void zero_lds(float *buf, int tid) {
    for (int e = tid; e < kTile; e += kT) buf[e] = 0.f;
}
__device__ __forceinline__ void acc2g(float *g, const f32x8 &acc, int lane, int wave) {
#pragma unroll
    for (int v = 0; v < 8; ++v) g[arow(v, lane, wave) * kD + acol(v, lane, wave)] = acc[v];
}

// Eight consecutive elements of an input tensor as fp32 (one 16-byte load for
// bf16, two for fp32); the tensors are 16-byte aligned and rows are 64 elements.
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

// Input tensor rows [row0, row0 + 64) of one head (rows >= L read as 0) -> LDS fp32;
// each thread converts eight consecutive elements of one row.
template <typename T>
__device__ __forceinline__ void in2l(float *buf, const T *g, int row0, int L, int tid) {
    const int r = tid >> 3, c = (tid & 7) * 8;  // 512 threads = 64 rows x 8 groups
    float x[8];
    if (row0 + r < L) {
        load8(x, g + (int64_t)(row0 + r) * kD + c);
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = 0.f;
    }
    f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
    *reinterpret_cast<f32x4 *>(buf + r * kP + c) = lo;
    *reinterpret_cast<f32x4 *>(buf + r * kP + c + 4) = hi;
}

__device__ __forceinline__ int64_t pair_index(int I, int J) { return (int64_t)I * (I - 1) / 2 + J; }

// X = (I + diag(beta) su(G))^-1 by back substitution: eight lanes per column
// (64 columns x 8 = 512 threads), each summing every eighth term of a row's
// dot product.  The lanes of a column are one aligned group of eight in one
// wave, so X[r][c], written by the group's first lane, is read back by the
// others in program order.
__device__ __forceinline__ void unit_upper_inverse(float *X, const float *G, const float *beta, int tid) {
    const int c = tid >> 3, p = tid & 7;
    for (int r = c + 1 + p; r < kC; r += 8) X[r * kP + c] = 0.f;
    if (p == 0) X[c * kP + c] = 1.f;
    for (int r = c - 1; r >= 0; --r) {
        float s = 0.f;
        for (int t = r + 1 + p; t <= c; t += 8) s += G[r * kP + t] * X[t * kP + c];
        s = sum8(s);
        if (p == 0) X[r * kP + c] = -beta[r] * s;
    }
}

// LDS tile -> global fp32 tile [64][64].
__device__ __forceinline__ void l2g(float *g, const float *buf, int tid) {
#pragma unroll
    for (int e = tid; e < kC * kD / 4; e += kT) {
        const int r = e >> 4, c = (e & 15) * 4;
        *reinterpret_cast<f32x4 *>(g + r * kD + c) = *reinterpret_cast<const f32x4 *>(buf + r * kP + c);
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
// Prep: one workgroup per (block J, head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void bwd_prep_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float sm[9 * kTile + 4 * kC];
    float *bW = sm, *bQ = bW + kTile, *bK = bQ + kTile, *bG = bK + kTile, *bA = bG + kTile, *bQW = bA + kTile,
          *bN = bQW + kTile, *bZ = bN + kTile, *bY = bZ + kTile;
    float *sB = bY + kTile, *sCl = sB + kC, *sL2 = sCl + kC, *sDD = sL2 + kC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * kD, *k = (const T *)a.k + hoff * kD, *w = (const T *)a.w + hoff * kD;
    const T *v = (const T *)a.v + hoff * kD, *o = (const T *)a.out + hoff * kD, *dout = (const T *)a.dout + hoff * kD;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float scale = a.scale;

    in2l(bW, w, row0, L, tid);
    in2l(bQ, q, row0, L, tid);
    in2l(bK, k, row0, L, tid);
    if (tid < kC) {
        const int i = row0 + tid;
        sB[tid] = i < L ? a.beta[hoff + i] : 0.f;
        sL2[tid] = i < L ? a.lse[hoff + i] * kLog2e : 0.f;
    }
    gate_prefix(sCl, a.logf ? a.logf + hoff : nullptr, row0, L, tid);
    {   // D_i = do_i . o_i - dlse_i: eight lanes per row, 8 columns each
        const int r = tid >> 3, c0 = (tid & 7) * 8, i = row0 + r;
        float s = 0.f;
        if (i < L) {
            float xo[8], xd[8];
            load8(xd, dout + (int64_t)i * kD + c0);
            load8(xo, o + (int64_t)i * kD + c0);
#pragma unroll
            for (int t = 0; t < 8; ++t) s += xd[t] * xo[t];
        }
        s = sum8(s);
        if ((tid & 7) == 0) sDD[r] = i < L ? s - (a.dlse ? a.dlse[hoff + i] : 0.f) : 0.f;
    }
    __syncthreads();
    f32x8 acc = zero8();
    mm(acc, nat(bW), tr(bW), lane, wave);  // G = W W^T
    store_lds(bG, acc, lane, wave, [](int, int, float x) { return x; });
    __syncthreads();
    unit_upper_inverse(bA, bG, sB, tid);
    __syncthreads();
    float *XX = (float *)(ws + ly.xx) + (int64_t)J * kC * kC, *AA = (float *)(ws + ly.aa) + (int64_t)J * kC * kC;
#pragma unroll
    for (int e = tid; e < kC * kC / 4; e += kT) {  // keep X, then A = X diag(beta) in place
        const int r = e >> 4, c = (e & 15) * 4;
        f32x4 x = *reinterpret_cast<const f32x4 *>(bA + r * kP + c);
        *reinterpret_cast<f32x4 *>(XX + r * kC + c) = x;
        x[0] *= sB[c]; x[1] *= sB[c + 1]; x[2] *= sB[c + 2]; x[3] *= sB[c + 3];
        *reinterpret_cast<f32x4 *>(bA + r * kP + c) = x;
        *reinterpret_cast<f32x4 *>(AA + r * kC + c) = x;
    }
    acc = zero8();
    mm(acc, nat(bQ), tr(bW), lane, wave);  // Q W^T, keep r <= i
    store_lds(bQW, acc, lane, wave, [](int r, int c, float x) { return c <= r ? x : 0.f; });
    acc = zero8();
    mm(acc, nat(bK), tr(bW), lane, wave);  // N = K W^T, keep r > j
    store_lds(bN, acc, lane, wave, [](int r, int c, float x) { return c > r ? x : 0.f; });
    __syncthreads();
    l2g((float *)(ws + ly.qwm) + (int64_t)J * kC * kC, bQW, tid);
    l2g((float *)(ws + ly.nn) + (int64_t)J * kC * kC, bN, tid);
    acc = zero8();
    mm(acc, nat(bQW), tr(bA), lane, wave);  // Z = QWm A^T
    store_lds(bZ, acc, lane, wave, [](int, int, float x) { return x; });
    acc = zero8();
    mm(acc, nat(bN), nat(bA), lane, wave);  // Y = N A
    store_lds(bY, acc, lane, wave, [](int, int, float x) { return x; });
    __syncthreads();
    l2g((float *)(ws + ly.zz) + (int64_t)J * kC * kC, bZ, tid);
    float *QH = (float *)(ws + ly.qh) + row0 * kD, *KH = (float *)(ws + ly.kh) + row0 * kD;
    {
        acc = zero8();
        mm(acc, nat(bZ), nat(bW), lane, wave);  // q^ = q - Z W
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            QH[r * kD + c] = bQ[r * kP + c] - acc[vv];
        }
        acc = zero8();
        mm(acc, nat(bY), nat(bW), lane, wave);  // k^ = k - Y W
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            KH[r * kD + c] = bK[r * kP + c] - acc[vv];
        }
        acc = zero8();
        mm(acc, nat(bA), nat(bW), lane, wave);  // A W (into bQW, free after Z)
    }
    __syncthreads();
    store_lds(bQW, acc, lane, wave, [](int, int, float x) { return x; });
    __syncthreads();
    {
        float *TT = (float *)(ws + ly.tt) + (int64_t)J * kD * kD, *TTt = (float *)(ws + ly.ttt) + (int64_t)J * kD * kD;
        acc = zero8();
        mm(acc, tr(bW), nat(bQW), lane, wave);  // T = I - W^T (A W)
        f32x8 acct = zero8();
        mm(acct, tr(bQW), nat(bW), lane, wave);  // T^T = I - (A W)^T W
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            TT[r * kD + c] = (r == c ? 1.f : 0.f) - acc[vv];
            TTt[r * kD + c] = (r == c ? 1.f : 0.f) - acct[vv];
        }
    }
    // diagonal block: P = exp(scale (Q K^T - Z N^T) + cl_i - cl_j - lse_i) for j <= i
    f32x8 sQK = zero8(), sZN = zero8();
    mm(sQK, nat(bQ), tr(bK), lane, wave);
    mm(sZN, nat(bZ), tr(bN), lane, wave);
    __syncthreads();  // bG, bY free: P -> bG, v -> bY, do -> bA
    {
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            const float s = (scale * (sQK[vv] - sZN[vv]) + (sCl[r] - sCl[c])) * kLog2e - sL2[r];
            bG[r * kP + c] = c <= r ? fast_exp2(s) : 0.f;
        }
    }
    in2l(bY, v, row0, L, tid);
    in2l(bA, dout, row0, L, tid);
    __syncthreads();
    acc = zero8();
    mm(acc, nat(bA), tr(bY), lane, wave);  // dP = dO V^T
    store_lds(bZ, acc, lane, wave, [&](int r, int c, float x) { return bG[r * kP + c] * (x - sDD[r]); });
    __syncthreads();
    {
        float *EE = (float *)(ws + ly.ee) + (int64_t)J * kC * kC;
        for (int e = tid; e < kC * kC; e += kT) EE[e] = scale * bZ[(e >> 6) * kP + (e & 63)];
        T *VF = (T *)(ws + ly.vf) + row0 * kD, *DOF = (T *)(ws + ly.dof) + row0 * kD;  // exact copies of v, do
        for (int e = tid; e < kC * kD; e += kT) {
            VF[e] = Elem<T>::from_float(bY[(e >> 6) * kP + (e & 63)]);
            DOF[e] = Elem<T>::from_float(bA[(e >> 6) * kP + (e & 63)]);
        }
        acc = zero8();
        mm(acc, tr(bG), nat(bA), lane, wave);  // diagonal value gradient P^T dO
        acc2g((float *)(ws + ly.dvd) + row0 * kD, acc, lane, wave);
        float *rs = (float *)(ws + ly.rsd) + row0, *cs = (float *)(ws + ly.csd) + row0;
        if (tid < kC) {
            float s = 0.f;
            for (int c = 0; c < kC; ++c) s += bZ[tid * kP + c];
            rs[tid] = s;
        } else if (tid < 2 * kC) {
            const int c = tid - kC;
            float s = 0.f;
            for (int r = 0; r < kC; ++r) s += bZ[r * kP + c];
            cs[c] = s;
        } else if (tid < 3 * kC) {
            const int r = tid - 2 * kC;
            ((float *)(ws + ly.l2))[row0 + r] = sL2[r];
            ((float *)(ws + ly.dd))[row0 + r] = sDD[r];
            ((float *)(ws + ly.clq))[row0 + r] = sCl[r];
            ((float *)(ws + ly.ckk))[row0 + r] = sCl[kC - 1] - sCl[r];
            if (r == 0) ((float *)(ws + ly.tot))[J] = sCl[kC - 1];
        }
    }
}

// ---------------------------------------------------------------------------
// Query-major up walk: one workgroup per (query block I >= 1, head); heaviest first.
// ---------------------------------------------------------------------------
// Down walk of the query blocks: one workgroup per (query block I >= 1, head),
// q~^(J-1) = T_J q~^(J) from q~^(I-1) = q^ down to J = 0, each q~^(J) stored for
// the pair (I, J), with the gate sum of the blocks strictly between I and J.
// One product per step on two LDS tiles, so four workgroups share a compute
// unit and hide each other's latency.
template <typename SC>
__global__ __launch_bounds__(kT, 4) void bwd_down_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float sm[2 * kTile];
    float *bQt = sm, *bT = bQt + kTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, I = nb - 1 - blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float *TT = (const float *)(ws + ly.tt), *tot = (const float *)(ws + ly.tot);
    float *MID = (float *)(ws + ly.mid);
    SC *QS = (SC *)(ws + ly.qs);
    const int row0 = I * kC;

    g2l(bQt, (const float *)(ws + ly.qh) + row0 * kD, tid);
    float mid = 0.f;
    if (tid == 0) MID[pair_index(I, I - 1)] = 0.f;
    Stage rT;
    if (I - 1 >= 1) gload(rT, TT + (int64_t)(I - 1) * kD * kD, tid);
    for (int J = I - 1; J >= 1; --J) {  // bQt holds q~^(J)
        lstore(bT, rT, tid);
        __syncthreads();
        l2g_sc(QS + pair_index(I, J) * kC * kD, bQt, tid);
        if (J - 1 >= 1) gload(rT, TT + (int64_t)(J - 1) * kD * kD, tid);  // next step's transition
        f32x8 acc = zero8();
        mm(acc, nat(bQt), tr(bT), lane, wave);  // q~^(J-1) = T_J q~^(J) (rows: Q~ T^T)
        __syncthreads();
        store_lds(bQt, acc, lane, wave, [](int, int, float x) { return x; });
        mid += tot[J];
        if (tid == 0) MID[pair_index(I, J - 1)] = mid;
    }
    __syncthreads();
    l2g_sc(QS + pair_index(I, 0) * kC * kD, bQt, tid);
}

template <typename SC>
__global__ __launch_bounds__(kT) void bwd_query_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float sm[8 * kTile + 4 * kC];
    float *bQt = sm, *bT = bQt + kTile, *bK = bT + kTile, *bV = bK + kTile, *bDO = bV + kTile, *bG = bDO + kTile,
          *bS = bG + kTile, *bP = bS + kTile;
    float *sL2 = bP + kTile, *sDD = sL2 + kC, *sCq = sDD + kC, *sCk = sCq + kC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, I = nb - 1 - blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float *TTt = (const float *)(ws + ly.ttt), *KH = (const float *)(ws + ly.kh);
    const SC *VF = (const SC *)(ws + ly.vf);
    const float *MID = (const float *)(ws + ly.mid);
    float *CSP = (float *)(ws + ly.csp);
    SC *QS = (SC *)(ws + ly.qs), *GS = (SC *)(ws + ly.gs), *PS = (SC *)(ws + ly.ps), *DS = (SC *)(ws + ly.ds);
    const float scale = a.scale;
    const int row0 = I * kC;

    Stage rT, rK;
    typename StageOf<SC>::T rQ, rV;
    // up: adjoint G
    {
        typename StageOf<SC>::T rD;
        gload(rD, (const SC *)(ws + ly.dof) + row0 * kD, tid);
        lstore(bDO, rD, tid);
    }
    if (tid < kC) {
        sL2[tid] = ((const float *)(ws + ly.l2))[row0 + tid];
        sDD[tid] = ((const float *)(ws + ly.dd))[row0 + tid];
        sCq[tid] = ((const float *)(ws + ly.clq))[row0 + tid];
    }
    f32x8 accG = zero8();
    float rsum = 0.f;
    gload(rQ, QS + pair_index(I, 0) * kC * kD, tid);
    gload(rK, KH, tid);
    gload(rV, VF, tid);
    float rck = tid < kC ? ((const float *)(ws + ly.ckk))[tid] : 0.f, rmid = MID[pair_index(I, 0)];
    for (int J = 0; J < I; ++J) {
        const int64_t p = pair_index(I, J);
        lstore(bQt, rQ, tid);
        lstore(bK, rK, tid);
        lstore(bV, rV, tid);
        if (J >= 1) lstore(bT, rT, tid);
        if (tid < kC) sCk[tid] = rck;
        const float midJ = rmid;
        __syncthreads();
        if (J >= 1) l2g_sc(GS + p * kC * kD, bG, tid);  // G^(J-1) (in bG since the last step) for the key-major walk
        if (J + 1 < I) {  // next step's tiles, in flight while this step computes
            gload(rQ, QS + (p + 1) * kC * kD, tid);
            gload(rK, KH + (int64_t)(J + 1) * kC * kD, tid);
            gload(rV, VF + (int64_t)(J + 1) * kC * kD, tid);
            gload(rT, TTt + (int64_t)(J + 1) * kD * kD, tid);
            if (tid < kC) rck = ((const float *)(ws + ly.ckk))[(J + 1) * kC + tid];
            rmid = MID[p + 1];
        }
        f32x8 s = zero8(), dp = zero8();
        mm(s, nat(bQt), tr(bK), lane, wave);
        mm(dp, nat(bDO), tr(bV), lane, wave);
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
            const int r = arow(vv, lane, wave), c = acol(vv, lane, wave);
            const float P = fast_exp2((scale * s[vv] + sCq[r] + sCk[c] + midJ) * kLog2e - sL2[r]);
            bP[r * kP + c] = P;
            bS[r * kP + c] = P * (dp[vv] - sDD[r]);
        }
        __syncthreads();
        l2g_sc(PS + p * kC * kC, bP, tid);  // P and dS for the key-major walk
        l2g_sc(DS + p * kC * kC, bS, tid);
        {   // column sums of this pair's dS (fp32) for the gate, summed over I by the key-major walk
            const int cc = tid >> 3, p0 = tid & 7;
            float t = 0.f;
#pragma unroll
            for (int r = p0; r < kC; r += 8) t += bS[r * kP + cc];
            t = sum8(t);
            if (p0 == 0) CSP[p * kC + cc] = t;
        }
        f32x8 gt = zero8(), xs = zero8();
        if (J >= 1) mm(gt, nat(bG), tr(bT), lane, wave);  // bT holds T_J^T here
        mm(xs, nat(bS), nat(bK), lane, wave);
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) accG[vv] = gt[vv] + scale * xs[vv];
        {   // row sums of dS: eight lanes per row, eight columns each
            const f32x4 *row = reinterpret_cast<const f32x4 *>(bS + (tid >> 3) * kP + (tid & 7) * 8);
            const float t = ((row[0][0] + row[0][1]) + (row[0][2] + row[0][3])) +
                            ((row[1][0] + row[1][1]) + (row[1][2] + row[1][3]));
            rsum += sum8(t);
        }
        __syncthreads();
        store_lds(bG, accG, lane, wave, [](int, int, float x) { return x; });
    }
    acc2g((float *)(ws + ly.dqo) + row0 * kD, accG, lane, wave);
    if ((tid & 7) == 0) ((float *)(ws + ly.rso))[row0 + (tid >> 3)] = rsum;
}

// ---------------------------------------------------------------------------
// Key-major walk: one workgroup per (key block J <= nb-2, head); heaviest first.
// The query-major walk left P, dS, q~ and G of every pair, so this walk only
// sums over the query blocks: dV_J += P^T dO_I, dk^_J += scale dS^T q~,
// dT_J += G^(J-1)^T q~, and the column sums of dS for the gate.
// ---------------------------------------------------------------------------
template <typename SC>
__global__ __launch_bounds__(kT) void bwd_key_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float sm[5 * kTile];
    float *bQt = sm, *bDO = bQt + kTile, *bG = bDO + kTile, *bP = bG + kTile, *bS = bP + kTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, J = blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float *CSP = (const float *)(ws + ly.csp);
    const SC *DOF = (const SC *)(ws + ly.dof);
    const SC *QS = (const SC *)(ws + ly.qs), *GS = (const SC *)(ws + ly.gs), *PS = (const SC *)(ws + ly.ps),
             *DS = (const SC *)(ws + ly.ds);
    const float scale = a.scale;

    f32x8 dV = zero8(), dK = zero8(), dT = zero8();
    float csum = 0.f;
    typename StageOf<SC>::T rO, rQ, rG, rP, rS;
    float rcs = 0.f;
    auto fetch = [&](int I) {
        const int64_t p = pair_index(I, J);
        gload(rQ, QS + p * kC * kD, tid);
        gload(rO, DOF + (int64_t)I * kC * kD, tid);
        if (J >= 1) gload(rG, GS + p * kC * kD, tid);
        gload(rP, PS + p * kC * kC, tid);
        gload(rS, DS + p * kC * kC, tid);
        if (tid < kC) rcs = CSP[p * kC + tid];
    };
    fetch(J + 1);
    for (int I = J + 1; I < nb; ++I) {
        lstore(bQt, rQ, tid);
        lstore(bDO, rO, tid);
        if (J >= 1) lstore(bG, rG, tid);
        lstore(bP, rP, tid);
        lstore(bS, rS, tid);
        __syncthreads();
        if (tid < kC) csum += rcs;
        if (I + 1 < nb) fetch(I + 1);  // next step's tiles, in flight while this step computes
        mm(dV, tr(bP), nat(bDO), lane, wave);
        mm(dK, tr(bS), nat(bQt), lane, wave);
        if (J >= 1) mm(dT, tr(bG), nat(bQt), lane, wave);
        __syncthreads();
    }
    const int row0 = J * kC;
#pragma unroll
    for (int vv = 0; vv < 8; ++vv) dK[vv] *= scale;
    acc2g((float *)(ws + ly.dko) + row0 * kD, dK, lane, wave);
    acc2g((float *)(ws + ly.dvo) + row0 * kD, dV, lane, wave);
    acc2g((float *)(ws + ly.dt) + (int64_t)J * kD * kD, dT, lane, wave);
    if (tid < kC) ((float *)(ws + ly.cso))[row0 + tid] = csum;
}

// The key-major walk for bf16 inputs: its five tiles arrive in bf16 and every
// product reads both operands with single loads (A transposed, B by rows), so
// the tiles stay bf16 in LDS (8 KiB each, row stride 64: the sixteen lanes of
// a read walk a row) and are widened as they are read.  At 40 KiB of LDS two
// workgroups share a compute unit.
__device__ __forceinline__ float h2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// acc += X^T Y for 64x64 bf16 tiles in LDS (row stride 64), fp32 products.
__device__ __forceinline__ void mm_tn_h(f32x8 &acc, const uint16_t *X, const uint16_t *Y, int lane, int wave) {
    const int r = 16 * (wave >> 1) + (lane & 15), c0 = 32 * (wave & 1) + (lane & 15), q = lane >> 4;
    f32x4 lo = acc.lo, hi = acc.hi;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int k0 = 16 * g + 4 * q;
        float x[4], y0[4], y1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[t] = h2f(X[(k0 + t) * 64 + r]);
            y0[t] = h2f(Y[(k0 + t) * 64 + c0]);
            y1[t] = h2f(Y[(k0 + t) * 64 + c0 + 16]);
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

__global__ __launch_bounds__(kT, 2) void bwd_key_kernel_h(BwdArgs a) {
    constexpr int kTh = kC * 64;  // elements of one bf16 tile
    __shared__ __attribute__((aligned(16))) uint16_t sm[5 * kTh];
    uint16_t *bQt = sm, *bDO = bQt + kTh, *bG = bDO + kTh, *bP = bG + kTh, *bS = bP + kTh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = a.nb, hc = a.hc;
    const int gl = blockIdx.x % hc, J = blockIdx.x / hc;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const float *CSP = (const float *)(ws + ly.csp);
    const uint16_t *DOF = (const uint16_t *)(ws + ly.dof), *QS = (const uint16_t *)(ws + ly.qs),
                   *GS = (const uint16_t *)(ws + ly.gs), *PS = (const uint16_t *)(ws + ly.ps),
                   *DS = (const uint16_t *)(ws + ly.ds);
    const float scale = a.scale;

    f32x8 dV = zero8(), dK = zero8(), dT = zero8();
    float csum = 0.f, rcs = 0.f;
    u32x4 rO, rQ, rG, rP, rS;  // eight bf16 per thread and tile: row tid / 8, columns 8 (tid % 8) ..
    auto fetch = [&](int I) {
        const int64_t p = pair_index(I, J);
        rQ = *reinterpret_cast<const u32x4 *>(QS + p * kC * kD + tid * 8);
        rO = *reinterpret_cast<const u32x4 *>(DOF + (int64_t)I * kC * kD + tid * 8);
        if (J >= 1) rG = *reinterpret_cast<const u32x4 *>(GS + p * kC * kD + tid * 8);
        rP = *reinterpret_cast<const u32x4 *>(PS + p * kC * kC + tid * 8);
        rS = *reinterpret_cast<const u32x4 *>(DS + p * kC * kC + tid * 8);
        if (tid < kC) rcs = CSP[p * kC + tid];
    };
    fetch(J + 1);
    for (int I = J + 1; I < nb; ++I) {
        *reinterpret_cast<u32x4 *>(bQt + tid * 8) = rQ;
        *reinterpret_cast<u32x4 *>(bDO + tid * 8) = rO;
        if (J >= 1) *reinterpret_cast<u32x4 *>(bG + tid * 8) = rG;
        *reinterpret_cast<u32x4 *>(bP + tid * 8) = rP;
        *reinterpret_cast<u32x4 *>(bS + tid * 8) = rS;
        __syncthreads();
        if (tid < kC) csum += rcs;
        if (I + 1 < nb) fetch(I + 1);  // next step's tiles, in flight while this step computes
        mm_tn_h(dV, bP, bDO, lane, wave);              // P^T dO
        mm_tn_h(dK, bS, bQt, lane, wave);              // dS^T q~
        if (J >= 1) mm_tn_h(dT, bG, bQt, lane, wave);  // G^T q~
        __syncthreads();
    }
    const int row0 = J * kC;
#pragma unroll
    for (int vv = 0; vv < 8; ++vv) dK[vv] *= scale;
    acc2g((float *)(ws + ly.dko) + row0 * kD, dK, lane, wave);
    acc2g((float *)(ws + ly.dvo) + row0 * kD, dV, lane, wave);
    acc2g((float *)(ws + ly.dt) + (int64_t)J * kD * kD, dT, lane, wave);
    if (tid < kC) ((float *)(ws + ly.cso))[row0 + tid] = csum;
}

// ---------------------------------------------------------------------------
// Block backward: one workgroup per (block J, head).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void acc2out(T *g, const f32x8 &acc, int row0, int L, int lane, int wave) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int r = arow(v, lane, wave), c = acol(v, lane, wave);
        if (row0 + r < L) g[(int64_t)(row0 + r) * kD + c] = Elem<T>::from_float(acc[v]);
    }
}

template <typename T>
__global__ __launch_bounds__(kT) void bwd_block_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float sm[9 * kTile + 2 * kC];
    float *bW = sm, *bQ = bW + kTile, *bK = bQ + kTile, *bX = bK + kTile, *bA = bX + kTile, *bQW = bA + kTile,
          *b6 = bQW + kTile, *bN = b6 + kTile, *b8 = bN + kTile;
    float *sB = b8 + kTile, *sRed = sB + kC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int J = blockIdx.x, gl = blockIdx.y, g = a.g0 + gl, L = a.L, nb = a.nb, row0 = J * kC;
    const int64_t hoff = (int64_t)g * L;
    const T *q = (const T *)a.q + hoff * kD, *k = (const T *)a.k + hoff * kD, *w = (const T *)a.w + hoff * kD;
    const BwdLayout &ly = a.ly;
    char *ws = (char *)a.ws + (int64_t)gl * ly.head;
    const bool hasQ = J >= 1, hasK = J <= nb - 2, hasT = J >= 1 && J <= nb - 2;
    auto id = [](int, int, float x) { return x; };

    in2l(bW, w, row0, L, tid);
    in2l(bQ, q, row0, L, tid);
    in2l(bK, k, row0, L, tid);
    if (tid < kC) sB[tid] = row0 + tid < L ? a.beta[hoff + row0 + tid] : 0.f;
    {   // the block's UT quantities, as prep computed them
        const int64_t o = (int64_t)J * kC * kC;
        g2l(bX, (const float *)(ws + ly.xx) + o, tid);
        g2l(bA, (const float *)(ws + ly.aa) + o, tid);
        g2l(bQW, (const float *)(ws + ly.qwm) + o, tid);
        g2l(bN, (const float *)(ws + ly.nn) + o, tid);
        g2l(b6, (const float *)(ws + ly.zz) + o, tid);
        g2l(b8, (const float *)(ws + ly.ee) + o, tid);  // E = scale dS of the diagonal block
    }
    f32x8 acc;
    __syncthreads();
    f32x8 dQ = zero8(), dK = zero8(), dZ = zero8(), dN = zero8(), dW = zero8(), dA = zero8();
    mm(dQ, nat(b8), nat(bK), lane, wave);   // E K
    mm(dK, tr(b8), nat(bQ), lane, wave);    // E^T Q
    mm(dZ, nat(b8), nat(bN), lane, wave);   // (E N), negated below
    mm(dN, tr(b8), nat(b6), lane, wave);    // (E^T Z), negated below
    __syncthreads();
    if (hasQ) g2l(b8, (const float *)(ws + ly.dqo) + row0 * kD, tid);  // dq^ from the query-major walk
    else zero_lds(b8, tid);
    __syncthreads();
    mm(dZ, nat(b8), tr(bW), lane, wave);    // + dq^ W^T
    mm(dW, tr(b6), nat(b8), lane, wave);    // Z^T dq^ (negated below)
    {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int r = arow(v, lane, wave), c = acol(v, lane, wave);
            dQ[v] += b8[r * kP + c];
            dZ[v] = -dZ[v];
            dN[v] = -dN[v];
            dW[v] = -dW[v];
        }
    }
    __syncthreads();
    if (hasK) g2l(b8, (const float *)(ws + ly.dko) + row0 * kD, tid);  // dk^ from the key-major walk
    else zero_lds(b8, tid);
    __syncthreads();
    {
#pragma unroll
        for (int v = 0; v < 8; ++v) dK[v] += b8[arow(v, lane, wave) * kP + acol(v, lane, wave)];
    }
    acc = zero8();
    mm(acc, nat(b8), tr(bW), lane, wave);  // dY = -dk^ W^T
    store_lds(b6, acc, lane, wave, [](int, int, float x) { return -x; });
    acc = zero8();
    mm(acc, tr(bN), nat(b8), lane, wave);  // R = N^T dk^ (into bQ; q is read again later)
    __syncthreads();
    store_lds(bQ, acc, lane, wave, id);
    __syncthreads();
    mm(dN, nat(b6), tr(bA), lane, wave);   // += dY A^T
    mm(dA, tr(bN), nat(b6), lane, wave);   // N^T dY
    acc = zero8();
    mm(acc, tr(bA), nat(bQ), lane, wave);  // A^T R = Y^T dk^
#pragma unroll
    for (int v = 0; v < 8; ++v) dW[v] -= acc[v];
    __syncthreads();
    store_lds(b6, dN, lane, wave, [](int r, int c, float x) { return c > r ? x : 0.f; });  // dKW = dN o [r > j]
    in2l(bQ, q, row0, L, tid);
    __syncthreads();
    mm(dK, nat(b6), nat(bW), lane, wave);  // += dKW W
    mm(dW, tr(b6), nat(bK), lane, wave);   // += dKW^T K
    __syncthreads();
    store_lds(b6, dZ, lane, wave, id);
    __syncthreads();
    acc = zero8();
    mm(acc, nat(b6), nat(bA), lane, wave);  // dQWm = (dZ A) o [r <= i]
    mm(dA, tr(b6), nat(bQW), lane, wave);   // += dZ^T QWm
    store_lds(bN, acc, lane, wave, [](int r, int c, float x) { return c <= r ? x : 0.f; });
    __syncthreads();
    mm(dQ, nat(bN), nat(bW), lane, wave);   // += dQWm W
    mm(dW, tr(bN), nat(bQ), lane, wave);    // += dQWm^T Q
    __syncthreads();
    if (hasT) {  // T = I - W^T A W
        g2l(b6, (const float *)(ws + ly.dt) + (int64_t)J * kD * kD, tid);
        acc = zero8();
        mm(acc, nat(bA), nat(bW), lane, wave);  // A W
        __syncthreads();
        store_lds(bN, acc, lane, wave, id);
        acc = zero8();
        mm(acc, nat(bW), nat(b6), lane, wave);  // W dT
        store_lds(bQW, acc, lane, wave, id);
        __syncthreads();
        acc = zero8();
        mm(acc, nat(bQW), tr(bW), lane, wave);  // W dT W^T
#pragma unroll
        for (int v = 0; v < 8; ++v) dA[v] -= acc[v];
        acc = zero8();
        mm(acc, nat(bN), tr(b6), lane, wave);   // A W dT^T
        mm(acc, tr(bA), nat(bQW), lane, wave);  // + A^T W dT
#pragma unroll
        for (int v = 0; v < 8; ++v) dW[v] -= acc[v];
        __syncthreads();
    }
    // A = X diag(beta): dX = dA diag(beta), dbeta_c += sum_r X_rc dA_rc (dA kept on the upper triangle)
    {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int r = arow(v, lane, wave), c = acol(v, lane, wave);
            dA[v] = c >= r ? dA[v] : 0.f;
            b6[r * kP + c] = dA[v] * sB[c];
            bQW[r * kP + c] = bX[r * kP + c] * dA[v];
        }
    }
    __syncthreads();
    float dbeta = 0.f;
    if (tid < kC)
        for (int r = 0; r < kC; ++r) dbeta += bQW[r * kP + tid];
    acc = zero8();
    mm(acc, tr(bX), nat(b6), lane, wave);  // X^T dX
    __syncthreads();
    store_lds(bN, acc, lane, wave, id);
    __syncthreads();
    f32x8 dTp = zero8(), G = zero8();
    mm(dTp, nat(bN), tr(bX), lane, wave);  // (X^T dX) X^T; dT' is its negative
    mm(G, nat(bW), tr(bW), lane, wave);
    {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int r = arow(v, lane, wave), c = acol(v, lane, wave);
            const float t = -dTp[v];
            bQW[r * kP + c] = c > r ? t * G[v] : 0.f;    // dbeta_r += sum_c dT'_rc U_rc
            b6[r * kP + c] = c > r ? sB[r] * t : 0.f;    // dG = diag(beta) dT' on the strict upper triangle
        }
    }
    __syncthreads();
    if (tid >= kC && tid < 2 * kC) {
        float s = 0.f;
        for (int c = 0; c < kC; ++c) s += bQW[(tid - kC) * kP + c];
        sRed[tid - kC] = s;
    }
    mm(dW, nat(b6), nat(bW), lane, wave);  // += (dG + dG^T) W
    mm(dW, tr(b6), nat(bW), lane, wave);
    __syncthreads();
    if (tid < kC && row0 + tid < L) a.dbeta[hoff + row0 + tid] = dbeta + sRed[tid];
    acc2out((T *)a.dq + hoff * kD, dQ, row0, L, lane, wave);
    acc2out((T *)a.dk + hoff * kD, dK, row0, L, lane, wave);
    acc2out((T *)a.dw + hoff * kD, dW, row0, L, lane, wave);
    {
        const float *dvd = (const float *)(ws + ly.dvd) + row0 * kD, *dvo = (const float *)(ws + ly.dvo) + row0 * kD;
        T *dv = (T *)a.dv + hoff * kD;
        for (int e = tid; e < kC * kD; e += kT) {
            const int r = e >> 6;
            if (row0 + r < L)
                dv[(int64_t)(row0 + r) * kD + (e & 63)] = Elem<T>::from_float(dvd[e] + (hasK ? dvo[e] : 0.f));
        }
    }
    if (tid < kC) {
        const int i = row0 + tid;
        const float rs = ((const float *)(ws + ly.rsd))[i] + (hasQ ? ((const float *)(ws + ly.rso))[i] : 0.f);
        const float cs = ((const float *)(ws + ly.csd))[i] + (hasK ? ((const float *)(ws + ly.cso))[i] : 0.f);
        ((float *)(ws + ly.dc))[i] = rs - cs;
    }
}

// dlogf_t = sum_{t' >= t} dc_t' for one head: 256 threads, contiguous chunks, fixed order.
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

}  // namespace

hipError_t launch_bwd(const BwdArgs &a0, bool bf16, hipStream_t st) {
    BwdArgs a = a0;
    const int G = a.B * a.H;
    for (int g0 = 0; g0 < G; g0 += a.hc_max) {
        a.g0 = g0;
        a.hc = min(a.hc_max, G - g0);
        const dim3 blk(kT);
        if (bf16) hipLaunchKernelGGL(bwd_prep_kernel<uint16_t>, dim3(a.nb, a.hc), blk, 0, st, a);
        else hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(a.nb, a.hc), blk, 0, st, a);
        if (a.nb > 1) {
            if (bf16) {
                hipLaunchKernelGGL(bwd_down_kernel<uint16_t>, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
                hipLaunchKernelGGL(bwd_query_kernel<uint16_t>, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
                hipLaunchKernelGGL(bwd_key_kernel_h, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
            } else {
                hipLaunchKernelGGL(bwd_down_kernel<float>, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
                hipLaunchKernelGGL(bwd_query_kernel<float>, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
                hipLaunchKernelGGL(bwd_key_kernel<float>, dim3((a.nb - 1) * a.hc), blk, 0, st, a);
            }
        }
        if (bf16) hipLaunchKernelGGL(bwd_block_kernel<uint16_t>, dim3(a.nb, a.hc), blk, 0, st, a);
        else hipLaunchKernelGGL(bwd_block_kernel<float>, dim3(a.nb, a.hc), blk, 0, st, a);
        if (a.dlogf) hipLaunchKernelGGL(bwd_gate_kernel, dim3(a.hc), blk, 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace path
