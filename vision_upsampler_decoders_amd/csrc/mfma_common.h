// Device helpers shared by the MFMA kernels (polyphase.hip, polyrw.hip):
// fragment types, the MFMA step per element type, raw buffer resources,
// wave-uniform values, register transposes and paired 16-bit rounding.
#pragma once

#include <type_traits>

#include "ctconv_internal.h"

namespace ctconv {
namespace mfma {

// Fragments live in registers as native 4 x 32-bit vectors (16 bytes); the
// 1-byte-aligned variant gives plain, possibly unaligned, 16-byte accesses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_u __attribute__((ext_vector_type(4), aligned(1)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <class TR>
struct Mma;

template <>
struct Mma<TBF16> {
    __device__ static inline void step(f32x4& acc, const u32x4 a, const u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

template <>
struct Mma<TF16> {
    __device__ static inline void step(f32x4& acc, const u32x4 a, const u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
};

template <>
struct Mma<TF32> {
    // Lane group g holds channels 4g..4g+3 of the 16-channel step in one
    // 16-byte fragment; MFMA number e consumes element e of every group, so
    // the four MFMAs together reduce over all 16 channels.
    __device__ static inline void step(f32x4& acc, const u32x4 a, const u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]),
                                                   acc, 0, 0, 0);
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_u __attribute__((ext_vector_type(2), aligned(1)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Fourth word of a raw (stride 0) buffer resource on gfx9-family chips:
// 32-bit data format, no swizzle; byte offsets are range-checked against the
// resource's size and out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;

// Values that are the same in every lane, pinned to scalar registers: buffer
// resources and scalar offsets must be, and a value the compiler cannot prove
// uniform would otherwise cost a loop over the distinct lane values.
__device__ inline uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline void* uniform_ptr(const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    return reinterpret_cast<void*>(((uint64_t)uniform((uint32_t)(u >> 32)) << 32) |
                                   uniform((uint32_t)u));
}

__device__ inline void store16_unaligned(void* p, const u32x4 v) {
    *reinterpret_cast<u32x4_u*>(p) = v;
}

// 8 channels x 4 positions of 16-bit elements -> 4 rows of 8 channels
// (v_perm_b32 gathers one half-word from each of two channels per dword).
__device__ inline void transpose_block(const u32x2 (&in)[8], u32x4 (&out)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const unsigned sel = (p & 1) ? 0x07060302u : 0x05040100u;
        u32x4 d;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            d[c] = __builtin_amdgcn_perm(in[2 * c + 1][p >> 1], in[2 * c][p >> 1], sel);
        out[p] = d;
    }
}

// 4 channels x 2 positions of 32-bit elements -> 2 rows of 4 channels.
__device__ inline void transpose_block(const u32x2 (&in)[4], u32x4 (&out)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) out[p] = u32x4{in[0][p], in[1][p], in[2][p], in[3][p]};
}

// Two fp32 values rounded to the 16-bit storage type and packed into one
// dword (low half first): one packed conversion instruction for bf16.
template <class TR>
__device__ inline uint32_t pack2(float f0, float f1) {
    if constexpr (std::is_same_v<TR, TBF16>) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f0, f1}, bf16x2));
    } else {
        return (uint32_t)TR::from_f32(f0) | ((uint32_t)TR::from_f32(f1) << 16);
    }
}

}  // namespace mfma
}  // namespace ctconv
