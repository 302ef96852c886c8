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
// unmasked 64 x 64 tile.
//
// The walk is first made with the softmax reference max fixed at 0 ("bounded
// walk"; all bf16 inputs, fp32 without the forget gate): a step is then its
// 32 products of logits and query transform (plus, with the gate, 4 that add
// the gate bias), exp2 of the logits, column sums, bf16 probabilities and the
// 16 products of P V, with no max, no check and no branch.  Floating point
// makes that exact unless a probability overflows or every relevant one
// underflows, which an end-of-walk test per query detects; such waves are
// walked again by a second launch with the running max ("checked walk", the
// only walk for fp32 with the gate).  A checked step issues its matrix-core
// products first (in bf16 the running max and the gate bias folded into the
// logit product as one more k-chunk), then takes the column maxima of all 64
// keys with a single check for the rare rescale, and only then runs the vector
// work interleaved with the products of P V.  The last step of a walk (key
// block 0) skips the query transform.  A workgroup is 4 waves = 4 consecutive query
// blocks sharing each key-block record (khat, V^T, -M: 24 KiB bf16 at d = 64),
// double-buffered in LDS; two workgroups share a CU.
#include <type_traits>

#include "path_common.h"
#include "path_kernels.h"
#include "path_layout.h"

namespace path {
namespace {

// Four consecutive elements (8 bytes of bf16 / 16 bytes of fp32) as fp32.
template <typename S>
__device__ __forceinline__ void load4(const S *p, float *x) {
    if constexpr (sizeof(S) == 2) {
        const u32x2 u = *(const u32x2 *)p;
        x[0] = bf16_to_f32(u.x & 0xffff);
        x[1] = bf16_to_f32(u.x >> 16);
        x[2] = bf16_to_f32(u.y & 0xffff);
        x[3] = bf16_to_f32(u.y >> 16);
    } else {
        const f32x4 v = *(const f32x4 *)p;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// Copy one key-block record (REC elements, 16-byte chunks spread over the
// workgroup) and, with the forget gate, its 64 tail sums from global memory
// straight into LDS (global_load_lds: lane l of a wave lands at the wave's
// LDS base + 16 l).  Completion is tracked by vmcnt.
template <typename S, int REC, int NLD, int NW, bool FOX>
__device__ __forceinline__ void issue_record(const S *src, const float *tail, S *dst, float *dtail, int wv, int lane) {
    // chunk t of thread tid is 16-byte chunk t * NT + tid: a uniform base plus
    // the same per-lane offset for every t, so the addressing needs one VGPR
    constexpr int NT = 64 * NW;
    const int tid = 64 * wv + lane;
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
        const char *g = (const char *)src + (size_t)t * NT * 16;
        char *l = (char *)dst + (size_t)t * NT * 16 + 1024 * wv;  // the wave's LDS base (uniform)
        __builtin_amdgcn_global_load_lds((const void *)(g + 16 * tid), (lds_void *)l, 16, 0, 0);
    }
    if (FOX && wv == 0) __builtin_amdgcn_global_load_lds((const void *)(tail + lane), (lds_void *)dtail, 4, 0, 0);
}

// Launch shape per element type and head dimension: NW waves per workgroup,
// CT 32-query column tiles per wave (a workgroup covers NW * CT / 2 query
// blocks that share every key-block record), NB key-block records in LDS.
// d = 64: 4 waves x 64 queries, two records, two workgroups per CU.  d = 128:
// a record is 64 KiB (bf16), and the query state of 64 columns (q-tilde, O:
// 256 fp32 accumulators) no longer fits a wave's registers, so waves take 32
// queries and 8 of them share the records; fp32 records (128 KiB) are
// single-buffered.
template <typename S, int D>
struct FwdCfg {
    static constexpr int NW = D == 64 ? 4 : (sizeof(S) == 2 ? 8 : 4);
    static constexpr int CT = D == 64 ? 2 : 1;
    static constexpr int NB = (D == 128 && sizeof(S) == 4) ? 1 : 2;
    static constexpr int QB = NW * CT / 2;  // query blocks per workgroup
    static constexpr int WG_PER_CU = D == 128 ? 1 : 2;
};

// The running max m of the online softmax is folded into the logit product
// (bf16, no forget gate): the product gets one more 16-wide k-chunk whose A
// rows are (1, 1, 0, ..., 0) and whose B column is (-m_hi, -m_lo, 0, ..., 0),
// with m_hi, m_lo bf16 and m = m_hi + m_lo exactly, so the accumulator holds
// s - m and each probability is a single exp2.  Only k = 0, 1 (fragment
// elements 0, 1 of lane half 0) are non-zero.
__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(to_bf16(x)); }
__device__ __forceinline__ i16x8 fold_ones(int h) {
    const u32x4 u = {h == 0 ? 0x3F803F80u : 0u, 0u, 0u, 0u};
    return __builtin_bit_cast(i16x8, u);
}
// With the forget gate the extra k-chunk also carries the gate bias: on the key
// side elements 2, 3 (lane half 0) hold the row's tail t_j = c_end(J) - c_j as
// (t_hi, t_lo), on the query side elements 0, 1 hold the query's offset o =
// off_i - m_i (the gate sum from the end of block J to the query, less the
// reference max) as (o_hi, o_lo) and elements 2, 3 hold (1, 1), so the product
// holds s + off_i + t_j - m_i; each pair represents its value to ~2^-17 of it.
__device__ __forceinline__ i16x8 fold_keys(int h, float t) {
    const float th = bf16_round(t);
    const u32x4 u = {h == 0 ? 0x3F803F80u : 0u, h == 0 ? pack_bf16(th, t - th) : 0u, 0u, 0u};
    return __builtin_bit_cast(i16x8, u);
}
__device__ __forceinline__ i16x8 fold_query(int h, float o) {
    const float oh = bf16_round(o);
    const u32x4 u = {h == 0 ? pack_bf16(oh, o - oh) : 0u, h == 0 ? 0x3F803F80u : 0u, 0u, 0u};
    return __builtin_bit_cast(i16x8, u);
}
// Split m0 into two bf16 pieces; m becomes their (exact) sum, frag the B column.
__device__ __forceinline__ void fold_split(float m0, int h, float &m, i16x8 &frag) {
    const float hi = bf16_round(m0), lo = bf16_round(m0 - hi);
    m = hi + lo;
    const u32x4 u = {h == 0 ? pack_bf16(-hi, -lo) : 0u, 0u, 0u, 0u};
    frag = __builtin_bit_cast(i16x8, u);
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt left at their maxima so they are not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// Same with lgkmcnt(0): this wave's LDS reads have returned as well.
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding global load, including the record copies
// meant to stay in flight); the caller waits for what it needs first.  The
// memory clobber keeps the compiler from moving loads or stores across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Per-wave state of the scan: query-side accumulators (transposed), output,
// logit buffers (NS of them), and the online-softmax statistics (log2 units).
template <int D, int CT, int NS>
struct WaveState {
    static constexpr int DT = D / 32;
    f32x16 qt[DT][CT], o[DT][CT], s[NS][2][CT];
    float m[CT], lp[CT], off[CT];
    float mref[CT];  // the diagonal block's max: a lower bound of the final max (skipping)
    i16x8 mb[CT];  // folded max (and gate offset): B column of the extra k-chunk
};

constexpr float kTau = 8.f;  // the running max is refreshed only when it grows by more than 2^kTau
constexpr float kSkipLog2 = 64.f;  // skipped key blocks contribute below 2^-64 of the running max each
constexpr int kCusPerXcd = 32;  // gfx950: 256 compute units in 8 XCDs

// Matrix-core part of step J into logit buffer SB: bf16 copy of qt as the B
// operand, S^T = khat qt^T for all 64 keys, and qt <- P_J qt.
// TAIL (with FOLD): the forget-gate bias goes into the extra k-chunk too (tail:
// the block's 64 tail sums in LDS).
template <typename S, int D, int CT, int NS, bool FOLD, int SB, bool XF = true, bool TAIL = false>
__device__ __forceinline__ void step_mma(WaveState<D, CT, NS> &w, const S *rec, const float *tail, int lane, int h) {
    typedef Elem<S> E;
    typedef typename E::Frag Frag;
    constexpr int KCH = D / 16, DT = D / 32;
    const S *sk = rec;
    const S *sm = rec + 2 * kBlk * D;
    Frag qb[CT][KCH];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kc = 0; kc < KCH; ++kc) qb[ct][kc] = acc_frag<S>(w.qt[kc >> 1][ct], kc & 1);
    if constexpr (TAIL) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) w.mb[ct] = fold_query(h, w.off[ct] - w.m[ct]);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const i16x8 ka = TAIL ? fold_keys(h, tail[32 * hf + (lane & 31)]) : fold_ones(h);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            w.s[SB][hf][ct] = f32x16{};
            if constexpr (FOLD)
                w.s[SB][hf][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, w.mb[ct], w.s[SB][hf][ct], 0, 0, 0);
        }
    }
    if constexpr (sizeof(S) == 2 && CT == 1) {
        // Every A fragment of the step -- the logits' khat, then the transform's -M (qt <- P_J qt;
        // XF false: block 0, whose transform no later block uses) -- in one sequence, each read
        // PF fragments ahead of its product so that the LDS read has returned when the product
        // issues.  The logit fragments alternate between the two key halves, so consecutive
        // products accumulate into different tiles (each tile still sums its k-chunks in order).
        constexpr int NL = 2 * KCH, NF = NL + (XF ? KCH * DT : 0), PF = 4;
        auto src = [&](int i) -> const Frag * {
            if (i < NL) return (const Frag *)(sk + (((i & 1) * KCH + (i >> 1)) * 64 + lane) * 8);
            const int j = i - NL;
            return (const Frag *)(sm + (((j % DT) * KCH + j / DT) * 64 + lane) * 8);
        };
        Frag ring[PF];
#pragma unroll
        for (int i = 0; i < PF && i < NF; ++i) ring[i] = *src(i);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const Frag af = ring[i % PF];
            if (i + PF < NF) ring[i % PF] = *src(i + PF);
            if (i < NL) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) E::mma(w.s[SB][i & 1][ct], af, qb[ct][i >> 1]);
            } else {
                const int j = i - NL;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) E::mma(w.qt[j % DT][ct], af, qb[ct][j / DT]);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the read PF products ahead
        }
    } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kc = 0; kc < KCH; ++kc) {
                const Frag af = *(const Frag *)(sk + ((hf * KCH + kc) * 64 + lane) * 8);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) E::mma(w.s[SB][hf][ct], af, qb[ct][kc]);
            }
        // qt <- P_J qt (XF false: block 0, whose transform no later block uses)
        if constexpr (XF)
#pragma unroll
        for (int kc = 0; kc < KCH; ++kc)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const Frag af = *(const Frag *)(sm + ((dt * KCH + kc) * 64 + lane) * 8);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) E::mma(w.qt[dt][ct], af, qb[ct][kc]);
            }
    }
}

// Column maxima of logit buffer SB (with the forget-gate tail bias added) and,
// rarely, the rescale when the running max grew by more than 2^kTau.
template <typename S, int D, int CT, int NS, bool FOX, bool FOLD, int SB>
__device__ __forceinline__ void step_check(WaveState<D, CT, NS> &w, const float *tail, int h) {
    constexpr int DT = D / 32;
    float mx[CT];
    bool grow = false;
    constexpr bool ADD = FOX && !FOLD;  // gate tail added here (folded into the product otherwise)
    f32x4 tl[2][4];  // forget-gate tail of the key rows this lane holds: rows 32 hf + 8 g + 4 h + e
    if (ADD) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int g = 0; g < 4; ++g) tl[hf][g] = *(const f32x4 *)(tail + 32 * hf + 8 * g + 4 * h);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        float x = -INFINITY;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (ADD) w.s[SB][hf][ct][r] += tl[hf][r >> 2][r & 3];
                x = fmaxf(x, w.s[SB][hf][ct][r]);
            }
        mx[ct] = ADD ? other_half_max(x) + w.off[ct] : other_half_max(x);
        grow = grow || (mx[ct] > (FOLD ? kTau : w.m[ct] + kTau));
    }
    if (__any(grow)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float mnew;
            if constexpr (FOLD)
                fold_split(w.m[ct] + fmaxf(mx[ct], 0.f), h, mnew, w.mb[ct]);
            else
                mnew = fmaxf(w.m[ct], mx[ct]);
            const float dlt = mnew - w.m[ct];
            const float alpha = fast_exp2(-dlt);
            w.m[ct] = mnew;
            w.lp[ct] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) w.o[dt][ct][r] *= alpha;
            if constexpr (FOLD) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int r = 0; r < 16; ++r) w.s[SB][hf][ct][r] -= dlt;
            }
        }
    }
}

// Vector part of step J from logit buffer SB: probabilities, their column
// sums, and O^T += V^T P^T.  BND: bounded walk, the reference max is 0.
template <typename S, int D, int CT, int NS, bool FOX, bool FOLD, int SB, bool BND = false>
__device__ __forceinline__ void step_softmax_pv(WaveState<D, CT, NS> &w, const S *rec, float fbJ, int lane) {
    typedef Elem<S> E;
    typedef typename E::Frag Frag;
    constexpr int DT = D / 32;
    const S *sv = rec + kBlk * D;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        Frag pf[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x16 &x = w.s[SB][hf][ct];
            if constexpr (FOLD || (BND && !FOX)) {  // the accumulator already holds the logit - m (BND: m = 0)
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r]);
            } else if constexpr (FOX) {
                const float sh = w.m[ct] - w.off[ct];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r] - sh);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r] - w.m[ct]);
            }
            float ps0 = x[0], ps1 = x[1];
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                ps0 += x[r];
                ps1 += x[r + 1];
            }
            w.lp[ct] += ps0 + ps1;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) pf[ct][cc] = acc_frag<S>(x, cc);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const Frag af = *(const Frag *)(sv + ((dt * 4 + 2 * hf + cc) * 64 + lane) * 8);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) E::mma(w.o[dt][ct], af, pf[ct][cc]);
            }
    }
    if (FOX) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) w.off[ct] += fbJ;
    }
}

// MODE: kChecked walks with the running max; kBounded walks with the
// reference max fixed at 0 and flags the workgroups whose result it cannot
// keep; kRedo repeats the checked walk for the flagged workgroups only.
enum { kChecked = 0, kBounded = 1, kRedo = 2 };

template <typename S, int D, bool FOX, int MODE>
__global__ __launch_bounds__(64 * (FwdCfg<S, D>::NW), (FwdCfg<S, D>::WG_PER_CU)) void path_fwd_kernel(FwdArgs a) {
    static_assert(D == 64 || D == 128, "forward kernel: head dimension 64 or 128");
    typedef FwdCfg<S, D> F;
    constexpr int NW = F::NW, NB = F::NB, NT = 64 * NW, CT = F::CT, QB = F::QB;
    constexpr int REC = 2 * kBlk * D + D * D;  // elements per key-block record
    constexpr int DT = D / 32;
    constexpr int VEC = 16 / (int)sizeof(S);   // elements per 16-byte load
    constexpr int NLD = REC / VEC / NT;        // 16-byte loads per thread per record
    constexpr bool kFold = sizeof(S) == 2;  // running max (and gate bias) folded into the logit product
    // bounded walk: without the gate nothing is folded; with it (bf16) the gate bias is
    constexpr bool kFoldB = FOX && sizeof(S) == 2;
    static_assert(MODE == kChecked || !FOX || sizeof(S) == 2, "the bounded walk with the forget gate is bf16 only");
    static_assert(REC % (VEC * NT) == 0, "record must split evenly over the workgroup");
    __shared__ __attribute__((aligned(32))) S srec[NB][REC];
    __shared__ __attribute__((aligned(16))) float stail[NB][kBlk];
    // skipping: this wave needs no more key blocks.  Two slots: step it reads slot it & 1 after
    // its barrier and every wave writes its verdict for step it + 1 into the other slot, so a
    // wave that runs ahead never changes flags that a slower wave of the same step still reads.
    __shared__ int sdone[2][NW];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    const int nb = (int)lay.nb;
    const int ntile = (nb + QB - 1) / QB;
    int *redo = (int *)((char *)a.ws + lay.off_redo);

    // Work item: heads are kept together on one XCD (workgroups are dealt
    // round-robin over the 8 XCDs, each with its own L2 and kCusPerXcd compute
    // units).  An XCD takes its heads in groups of G, about two rounds of its
    // workgroup slots; inside a group the tiles run longest first across the
    // group's heads, so the records of a few heads are shared through L2 while
    // the longest walks of the last heads still start early (ordering head by
    // head instead left the last heads' longest walks running alone at the end;
    // groups of one round were about 1% slower, of half a round 3% slower).
    const int64_t total = (int64_t)ntile * lay.bh;
    int64_t g = blockIdx.x;
    const int64_t item = (total % 8 == 0) ? (g % 8) * (total / 8) + g / 8 : g;
    const int64_t G = max(1, (2 * kCusPerXcd * F::WG_PER_CU) / ntile);
    const int64_t gbase = item / (G * ntile) * G;  // first head of the item's group
    const int64_t gn = min(G, lay.bh - gbase);     // heads in the group (the last one may be short)
    const int64_t rank = item - gbase * ntile;     // position inside the group
    const int64_t bh = gbase + rank % gn;
    const int tile = ntile - 1 - (int)(rank / gn);

    const int I = QB * tile + (wv * CT) / 2;     // this wave's query block
    const int c0 = 32 * ((wv * CT) % 2);         // first query column of this wave inside the block
    const int Jtop = min(QB * tile + QB - 1, nb - 1) - 1;
    if (Jtop < 0) return;
    // redo flags: one per wave of the bounded walk (workgroup g, wave wv)
    int *wflag = redo + g * NW;
    bool redo_me = true;
    if constexpr (MODE == kRedo) {
        int any = 0;
#pragma unroll
        for (int v2 = 0; v2 < NW; ++v2) any |= wflag[v2];
        if (!any) return;  // uniform: the bounded walk's results stand
        redo_me = wflag[wv] != 0;
    }
    const bool active = I >= 1 && I < nb && redo_me;  // block 0 is complete after prep

    const S *recs = (const S *)((const char *)a.ws + lay.off_rec) + bh * lay.nb * REC;
    const float *fk = (const float *)((const char *)a.ws + lay.off_fk) + bh * lay.lp;
    const float *fb = (const float *)((const char *)a.ws + lay.off_fb) + bh * lay.nb;

    // ---- per-wave state: qhat (pre-scaled by scale * log2(e): logits are in
    // log2 units), the diagonal block's output, max and sum.  In the bounded
    // walk the reference max is 0, so the diagonal block's sum and output are
    // taken at scale 2^m (0 or inf when that under- or overflows, which the
    // end-of-walk test catches).
    WaveState<D, CT, 1> w;
    auto init_state = [&](auto bounded) {
        constexpr bool BND = decltype(bounded)::value;
        if (!active) return;
        const S *qh = (const S *)((const char *)a.ws + lay.off_qhat) + (bh * lay.lp + (int64_t)I * kBlk) * D;
        const S *od = (const S *)a.out + (bh * a.L + (int64_t)I * kBlk) * D;
        const float *md = (const float *)((const char *)a.ws + lay.off_mdiag) + bh * lay.lp + (int64_t)I * kBlk;
        const float *ld = (const float *)((const char *)a.ws + lay.off_ldiag) + bh * lay.lp + (int64_t)I * kBlk;
        const float *fq = (const float *)((const char *)a.ws + lay.off_fq) + bh * lay.lp + (int64_t)I * kBlk;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int i = c0 + 32 * ct + l32;
            const bool valid = (int64_t)I * kBlk + i < a.L;
            const int io = valid ? i : 0;  // rows past L read row 0 of the block, then drop it
            float ls = ld[i];
            w.m[ct] = md[i];
            w.mref[ct] = md[i];
            if constexpr (BND) {
                ls *= fast_exp2(w.m[ct]);
                w.m[ct] = 0.f;
            } else if constexpr (kFold) {
                // switch the reference to the nearest two-piece bf16 value
                const float m0 = w.m[ct];
                fold_split(m0, h, w.m[ct], w.mb[ct]);
                ls *= fast_exp2(m0 - w.m[ct]);
            }
            w.lp[ct] = h == 0 ? ls : 0.f;
            w.off[ct] = FOX ? fq[i] : 0.f;
            const float os = valid ? ls : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * dt + 8 * g4 + 4 * h;  // 4 contiguous rows of the tile
                    float qv[4], ov[4];
                    load4<S>(qh + (int64_t)i * D + d, qv);
                    load4<S>(od + (int64_t)io * D + d, ov);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w.qt[dt][ct][4 * g4 + e] = qv[e];
                        w.o[dt][ct][4 * g4 + e] = ov[e] * os;
                    }
                }
        }
    };

    // ---- skipping negligible key blocks (with the forget gate, on request).  With
    // every transition a contraction (0 <= beta ||w||^2 <= 2, checked per block
    // by prep), a logit of query i against any key of block J or earlier is at
    // most ||qhat_i|| * max_j ||k_j|| plus the forget-gate bias of the block
    // boundary (off_i, log2 units; the bias only falls further back).  Once
    // that bound is more than kSkipLog2 below the running max for every query
    // of a wave, the remaining blocks add less than L 2^-kSkipLog2 of the
    // normaliser, far below fp32 resolution, and the wave stops; the workgroup
    // leaves the walk when all its waves have.
    const bool skip = FOX && a.skip;
    bool wdone = !active;
    float qbound[CT];
    auto setup_skip = [&]() {
        const float *kn = (const float *)((const char *)a.ws + lay.off_kn) + bh * lay.nb;
        float km = 0.f;
        for (int j = lane; j <= Jtop; j += 64) km = fmaxf(km, kn[j]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) km = fmaxf(km, __shfl_xor(km, o));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float ss = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += w.qt[dt][ct][r] * w.qt[dt][ct][r];
            qbound[ct] = sqrtf(other_half_sum(ss)) * (1.f + 0x1p-10f) * km;  // rounded up; inf if not contractive
        }
        if (lane == 0) sdone[0][wv] = wdone;
    };
    // reference: the running max (checked walk) or the diagonal block's max, a lower bound of the
    // final max (bounded walk, whose m stays 0)
    auto negligible = [&](auto bounded) {
        bool ok = true;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            ok = ok && (qbound[ct] + w.off[ct] - (decltype(bounded)::value ? w.mref[ct] : w.m[ct]) < -kSkipLog2);
        return __all(ok);
    };

    // ---- key-block records are copied global -> LDS by the DMA path (completion
    // tracked by vmcnt; wave 0 has one more copy per record with the forget gate)
    // wait until at most n records' copies of this wave are in flight (lgkmcnt(0) too)
    auto wait_records = [&](auto n) {
        if (FOX && wv == 0)
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((NLD + 1) * decltype(n)::value));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(NLD * decltype(n)::value));
    };
    auto rec_ptr = [&](int J) { return recs + (int64_t)J * REC; };
    auto tail_ptr = [&](int J) { return fk + (int64_t)J * kBlk; };
    // The first NB - 1 records' copies, issued before the query state is loaded
    // so that the two memory latencies overlap.
    auto prologue = [&]() {
#pragma unroll
        for (int k = 0; k < (NB > 1 ? NB - 1 : 1); ++k)
            if (Jtop - k >= 0)
                issue_record<S, REC, NLD, NW, FOX>(rec_ptr(Jtop - k), tail_ptr(Jtop - k), srec[k], stail[k], wv, lane);
    };
    // One walk over the key blocks J = Jtop .. 0.  All waves in step; NB - 1
    // records ahead (a single buffer is refilled after every wave is done with
    // it).  The last step waits for every copy, so no copy is in flight after
    // a full walk.
    auto walk = [&](auto bounded) {
        constexpr bool BND = decltype(bounded)::value;
        // one step; false when the walk stops early (skipping)
        auto body = [&](int J, auto xform) -> bool {
            constexpr bool XF = decltype(xform)::value;
            // unsigned: the read buffer it % NB and the refilled one (it + NB - 1) % NB
            // are then provably different, so the compiler does not make the
            // reads of this record wait for the copies of the next one
            const unsigned it = (unsigned)(Jtop - J);
            const int buf = (int)(it % NB);
            // wait for this wave's copies of record J; the copies of the NB - 2 newer
            // records issued after it may stay in flight
            if (NB > 2 && J >= 1)
                wait_records(std::integral_constant<int, (NB > 2 ? NB - 2 : 0)>{});
            else
                wait_records(std::integral_constant<int, 0>{});
            barrier_only();  // every wave's copies have landed; buffer (it + NB - 1) % NB is free
            if (skip) {
                bool all = true;
#pragma unroll
                for (int v2 = 0; v2 < NW; ++v2) all = all && sdone[it & 1][v2];
                if (all) return false;  // uniform: slot it & 1 is not written again before the next barrier
            }
            if (NB > 1 && J - (NB - 1) >= 0) {
                const int jn = J - (NB - 1);
                issue_record<S, REC, NLD, NW, FOX>(rec_ptr(jn), tail_ptr(jn), srec[(it + NB - 1) % NB],
                                                   stail[(it + NB - 1) % NB], wv, lane);
            }
            if (active && J < I && !wdone) {
                if constexpr (BND) {
                    step_mma<S, D, CT, 1, kFoldB, 0, XF, kFoldB>(w, srec[buf], stail[buf], lane, h);
                    step_softmax_pv<S, D, CT, 1, FOX, kFoldB, 0, true>(w, srec[buf], FOX ? fb[J] : 0.f, lane);
                } else {
                    step_mma<S, D, CT, 1, kFold, 0, XF, FOX && kFold>(w, srec[buf], stail[buf], lane, h);
                    step_check<S, D, CT, 1, FOX, kFold, 0>(w, stail[buf], h);
                    step_softmax_pv<S, D, CT, 1, FOX, kFold, 0>(w, srec[buf], FOX ? fb[J] : 0.f, lane);
                }
            }
            if (skip) {  // bound for blocks J - 1 and earlier (off now sits at the J-1 / J boundary)
                wdone = wdone || negligible(std::integral_constant<bool, BND>{});
                if (lane == 0) sdone[(it + 1) & 1][wv] = wdone;
            }
            if (NB == 1 && J >= 1) {
                __syncthreads();  // every wave is done with the buffer
                issue_record<S, REC, NLD, NW, FOX>(rec_ptr(J - 1), tail_ptr(J - 1), srec[0], stail[0], wv, lane);
            }
            return true;
        };
        bool go = true;
        for (int J = Jtop; J >= 1 && go; --J) go = body(J, std::true_type{});
        if (go) body(0, std::false_type{});  // block 0 without the query transform
    };

    // ---- epilogue
    auto finish = [&]() {
        if (!active) return;
        S *go = (S *)a.out + (bh * a.L + (int64_t)I * kBlk) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int i = c0 + 32 * ct + l32;
            const float lsum = other_half_sum(w.lp[ct]);
            if ((int64_t)I * kBlk + i >= a.L) continue;
            const float inv = 1.f / lsum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * dt + 8 * g4 + 4 * h;
                    S *p = go + (int64_t)i * D + d;
                    const f32x16 &c = w.o[dt][ct];
                    if constexpr (sizeof(S) == 2) {
                        u32x2 u = {pack_bf16(c[4 * g4] * inv, c[4 * g4 + 1] * inv),
                                   pack_bf16(c[4 * g4 + 2] * inv, c[4 * g4 + 3] * inv)};
                        *(u32x2 *)p = u;
                    } else {
                        f32x4 v = {c[4 * g4] * inv, c[4 * g4 + 1] * inv, c[4 * g4 + 2] * inv, c[4 * g4 + 3] * inv};
                        *(f32x4 *)p = v;
                    }
                }
            if (a.lse && h == 0) a.lse[bh * a.L + (int64_t)I * kBlk + i] = (w.m[ct] + __log2f(lsum)) * kLn2;
        }
    };

    if constexpr (MODE == kBounded) {
        // ---- bounded walk.  Without the forget gate, each query first walks
        // with the reference max fixed at 0: no folded max, no per-block max
        // check, no rescale.  The result is exact to fp32 unless a probability
        // overflowed or every relevant one underflowed, so it is kept when, for
        // every valid query, the sum lies in [2^-60, 2^120] (each probability is
        // at most the sum, so all are finite, also in bf16; terms lost below
        // 2^-126 add at most L 2^-126 <= 2^-66 of the sum) and the output
        // accumulators are finite.  Otherwise the wave leaves `out` as the prep
        // kernel wrote it and flags itself, and a second launch repeats the walk
        // with the running max for the flagged waves.  The bounded walk needs no
        // more than the logits being within about +-100 (log2 units) of 0, which
        // holds for any inputs of moderate norm.
        prologue();
        init_state(std::true_type{});
        if (skip) setup_skip();
        walk(std::true_type{});
        // no record copy may still be landing in LDS when the workgroup leaves early
        if (skip) __builtin_amdgcn_s_waitcnt(0);
        bool ok = true;
        if (active) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const float lsum = other_half_sum(w.lp[ct]);
                bool r = lsum >= 0x1p-60f && lsum <= 0x1p120f;  // false for NaN
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) r = r && __builtin_isfinite(w.o[dt][ct][e]);
                const bool valid = (int64_t)I * kBlk + c0 + 32 * ct + l32 < a.L;
                ok = ok && (r || !valid);
            }
        }
        const bool keep = __all(ok);
        if (lane == 0) wflag[wv] = keep ? 0 : 1;
        if (keep) finish();
        return;
    }
    // ---- checked walk: the running max is tracked block by block (refreshed
    // when it grows by more than 2^kTau)
    prologue();
    init_state(std::false_type{});
    if (skip) setup_skip();
    walk(std::false_type{});

    // no record copy may still be landing in LDS when the workgroup leaves early
    if (skip) __builtin_amdgcn_s_waitcnt(0);
    finish();
}

}  // namespace

// The bounded walk, then the checked walk of the waves it flagged (workgroups
// without a flagged wave leave at once); fp32 with the forget gate: the checked
// walk only.
template <typename S, int D, bool FOX>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
    typedef FwdCfg<S, D> F;
    const FwdLayout lay = fwd_layout(a.B, a.H, a.L, D, sizeof(S));
    const int64_t ntile = (lay.nb + F::QB - 1) / F::QB;
    dim3 grid((unsigned)(ntile * lay.bh));
    if constexpr (FOX && sizeof(S) == 4) {
        hipLaunchKernelGGL((path_fwd_kernel<S, D, true, kChecked>), grid, dim3(64 * F::NW), 0, st, a);
    } else {
        hipLaunchKernelGGL((path_fwd_kernel<S, D, FOX, kBounded>), grid, dim3(64 * F::NW), 0, st, a);
        hipLaunchKernelGGL((path_fwd_kernel<S, D, FOX, kRedo>), grid, dim3(64 * F::NW), 0, st, a);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs &a, bool bf16, hipStream_t st) {
    if (bf16) return a.fox ? launch_fwd_t<uint16_t, D, true>(a, st) : launch_fwd_t<uint16_t, D, false>(a, st);
    return a.fox ? launch_fwd_t<float, D, true>(a, st) : launch_fwd_t<float, D, false>(a, st);
}

hipError_t launch_fwd(const FwdArgs &a, bool bf16, hipStream_t st) {
    if (a.d == 64) return launch_fwd_d<64>(a, bf16, st);
    if (a.d == 128) return launch_fwd_d<128>(a, bf16, st);
    return hipErrorInvalidValue;
}

}  // namespace path
