// mfma_common.h -- gfx950 matrix-core helpers shared by the prefill and
// decode kernels: operand vector types, the 32x32x16 bf16/fp16 MFMA, rounding
// of fp32 pairs to the element type, and the LDS transpose read.
//
// Layouts (v_mfma_f32_32x32x16_{bf16,f16}, wave64), with l the lane:
//   A[i][k]: lane l holds row i = l%32, k = 8*(l/32) + e for e = 0..7
//   B[k][j]: lane l holds column j = l%32, k = 8*(l/32) + e
//   C[i][j]: lane l holds column j = l%32, rows i = 8*(r/4) + 4*(l/32) + r%4,
//            r = 0..15 the accumulator register.
// (v_mfma_f32_16x16x32_{bf16,f16}):
//   A[i][k]: lane l holds row i = l%16, k = 8*(l/16) + e
//   B[k][j]: lane l holds column j = l%16, k = 8*(l/16) + e
//   C[i][j]: lane l holds column j = l%16, rows i = 4*(l/16) + r, r = 0..3.
// ds_read_b64_tr_b16: within each group of 16 lanes, source lane L reads 4
// elements at its own address; lane i of the group receives element (i%4) of
// source lane 4*e + i/4 as its element e (a 4x16 -> 16x4 transpose).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <bool kBf16> struct Mma;

template <> struct Mma<true> {
    using vec8 = bf16x8;
    static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(i16x8 a, i16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // Two floats -> two rounded elements packed in 32 bits (low = a), and the
    // rounded values back as floats.
    static __device__ __forceinline__ uint32_t pack(float a, float b, float& ra, float& rb) {
        bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        ra = __uint_as_float(u << 16);
        rb = __uint_as_float(u & 0xffff0000u);
        return u;
    }
    static __device__ __forceinline__ uint32_t pack_out(float a, float b) {
        bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
        return __builtin_bit_cast(uint32_t, v);
    }
    // acc + (both rounded elements of a packed pair), products by 1 are exact.
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
    }
};

template <> struct Mma<false> {
    using vec8 = f16x8;
    static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(i16x8 a, i16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b, float& ra, float& rb) {
        f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
        ra = static_cast<float>(v[0]);
        rb = static_cast<float>(v[1]);
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ uint32_t pack_out(float a, float b) {
        f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const f16x2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
    }
};

// Word 3 of a raw (unswizzled, untyped) buffer resource on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

// A raw buffer over [base, base + bytes): loads at or past the end return
// zeros, so tile edges need no branch and memory past the end is never read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             static_cast<int>(bytes), kBufferWord3);
}

__device__ __forceinline__ i16x8 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// The same load with the non-temporal hint, for data read exactly once (a
// streaming pass over a key/value cache): the lines are not kept in the
// caches for reuse, which raises sustained read bandwidth.
__device__ __forceinline__ i16x8 load16_stream(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// Row maximum for the online normaliser: IEEE maximum, which propagates a
// NaN (v_maximum3_f32 on gfx950, no per-input quieting as maxNum needs).  A
// NaN score only occurs in a row that must end NaN anyway: the NaN maximum
// raises nothing and the row's p and l become NaN.
__device__ __forceinline__ float max_nan(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Combine a value with the one in lane l ^ 32 (the other half of the wave)
// through v_permlane32_swap: with both operands x, the first result holds
// x[l] in lanes 0..31 and x[l - 32] above, the second x[l + 32] below and
// x[l] above.  Both lanes of a pair get bit-identical results.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return max_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i16x4 tr_read(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3)))*)(
            (__attribute__((address_space(3))) uint16_t*)(p)));
}

// Eight bytes by the 8-bit transpose read: lane 8h + i of each 16-lane group
// receives byte i of the 8 bytes that lanes 2k + h (k = 0..7) point at, in
// k order (a layout checked on the GPU).
__device__ __forceinline__ uint2 tr_read8(const uint8_t* p) {
    typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (i32x2 __attribute__((address_space(3)))*)((__attribute__((address_space(3))) uint8_t*)(p)));
    return make_uint2(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]));
}

}  // namespace mfma
}  // namespace sdpa
