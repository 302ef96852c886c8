// path_common.h -- device-side building blocks shared by the PaTH kernels
// (gfx950 / CDNA4 only).
//
// Matrix-core tiles.  Every contraction in the library is expressed with the
// 32x32 MFMA shapes: v_mfma_f32_32x32x16_bf16 for bf16 operands and
// v_mfma_f32_32x32x2f32 for fp32 operands.  For both, with lane l, half
// h = l / 32 and accumulator register r (0..15), the 32x32 fp32 accumulator
// holds element (row, col) = (8*(r/4) + 4*h + r%4, l%32).
//
// A "fragment" is a 32-row x 16-k slab of an A operand (or 16-k x 32-col of a
// B operand) held as 8 elements per lane: lane l owns row (col) l%32 and the
// k indices
//     k(e, h) = 8*(e/4) + 4*h + e%4,   e = 0..7.
// This k order is not the natural one, but a contraction does not care how k
// is permuted as long as A and B agree; with this order the 16 accumulator
// registers of a 32x32 tile, split as r = 8*c + e, ARE the two B fragments
// (c = 0, 1) of that tile read with its rows as the contraction index.  So an
// accumulator can feed the next product without any data movement, and tiles
// stored in memory in fragment order are read with one 16- or 32-byte load
// per lane.  For bf16 a fragment is one MFMA (k = 16); for fp32 it is eight
// MFMAs of k = 2 (element e of every lane forms the e-th one, lane half h
// supplying k = h), which yields exactly the same k(e, h) map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace path {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> two packed bf16 (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)(pack_bf16(x, 0.f) & 0xffffu); }

// Element type traits: storage type, fragment register type, MFMA.
template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 stored as raw 16-bit
    typedef i16x8 Frag;  // 8 bf16 = 4 VGPRs = 16 bytes
    static constexpr int kFragBytes = 16;
    __device__ __forceinline__ static void mma(f32x16 &c, const Frag &a, const Frag &b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // Fragment from 8 fp32 values (rounded to bf16).
    __device__ __forceinline__ static Frag from_f32(const float *x) {
        u32x4 u;
        u.x = pack_bf16(x[0], x[1]);
        u.y = pack_bf16(x[2], x[3]);
        u.z = pack_bf16(x[4], x[5]);
        u.w = pack_bf16(x[6], x[7]);
        return __builtin_bit_cast(Frag, u);
    }
    __device__ __forceinline__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
    __device__ __forceinline__ static uint16_t from_float(float x) { return to_bf16(x); }
};

template <>
struct Elem<float> {
    typedef f32x8 Frag;  // 8 fp32 = 8 VGPRs = 32 bytes
    static constexpr int kFragBytes = 32;
    __device__ __forceinline__ static void mma(f32x16 &c, const Frag &a, const Frag &b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
    }
    __device__ __forceinline__ static Frag from_f32(const float *x) {
        Frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = x[e];
        return f;
    }
    __device__ __forceinline__ static float to_f32(float x) { return x; }
    __device__ __forceinline__ static float from_float(float x) { return x; }
};

// B fragment c (0/1) of a 32x32 accumulator tile: its registers 8c .. 8c+7.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag acc_frag(const f32x16 &acc, int c) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = acc[8 * c + e];
    return Elem<T>::from_f32(x);
}

// Row of a 32x32 accumulator tile held in register r by lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// k offset (0..15) inside a fragment of element e for lane half h.
__device__ __forceinline__ int frag_k(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

// Value of the other lane half with the same l % 32: {x[l%32], x[l%32+32]}.
__device__ __forceinline__ float other_half_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sums over aligned groups of 4 / 8 lanes via DPP; every lane of a group gets a
// bitwise identical result (each step adds a commutative pair).
__device__ __forceinline__ float sum4(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad xor 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad xor 2
    return x;
}
__device__ __forceinline__ float sum8(float x) {
    x = sum4(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
    return x;
}

}  // namespace path
