// device_common.h -- small device helpers: storage-type conversion, base-2
// exponent, wave reductions.  gfx950 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace sdpa {

// The causal offset of batch entry b, given its clamped key length.
__device__ __forceinline__ int64_t causal_delta(const Params& p, int64_t kv_len) {
    return p.delta_end ? kv_len - p.Lq : p.delta;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Storage types.  bfloat16 travels as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

template <typename T> struct Elem;

template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
        static_cast<float*>(p)[i] = x;
    }
};

template <> struct Elem<_Float16> {
    static __device__ __forceinline__ float load(const void* p, int64_t i) {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
        static_cast<_Float16*>(p)[i] = static_cast<_Float16>(x);   // round to nearest even
    }
};

template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const void* p, int64_t i) {
        const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
        return __uint_as_float(u);
    }
    static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
        static_cast<__bf16*>(p)[i] = static_cast<__bf16>(x);         // round to nearest even
    }
};

// 2^x on the transcendental unit: exact 0 for -inf, +inf for +inf, NaN for NaN.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// IEEE maxNum: a NaN operand is ignored (NaN reaches the output through exp2).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Butterfly sum: every lane ends with the same bits (each step adds the same
// two numbers on both partners, and addition is commutative).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace sdpa
