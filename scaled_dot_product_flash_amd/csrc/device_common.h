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

// First key a causal row i may see under a local window of W keys (ONNX
// GroupQueryAttention README, "Attributes"): j > i + delta - W; 0 without one.
__device__ __forceinline__ int64_t window_lo(const Params& p, int64_t i, int64_t delta) {
    if (!p.causal || p.window <= 0) return 0;
    const int64_t lo = i + delta - p.window + 1;
    return lo < 0 ? 0 : lo;
}

// First key row i of entry b may see under the window and the document
// mask (llm.istanbul "05_attention": keys before the document start are
// hidden); 0 without either.
__device__ __forceinline__ int64_t first_key(const Params& p, int b, int64_t i, int64_t delta) {
    int64_t lo = window_lo(p, i, delta);
    if (p.doc_start) {
        const int64_t d = p.doc_start[static_cast<int64_t>(b) * p.Lq + i];
        lo = d > lo ? d : lo;
    }
    return lo;
}

// Softcap on a raw score s = q.k (before scaling): the scaled score becomes
// c * tanh(scale * s / c), i.e. in raw units back * tanh(s * k2 / 2) with
// k2 = 2 * log2(e) * scale / c and back = c / scale, through
// tanh(x) = 1 - 2 / (2^(2 x log2 e) + 1): exact +-1 at +-inf, NaN stays NaN.
__device__ __forceinline__ float softcap_raw(float s, float k2, float back) {
    const float e = __builtin_amdgcn_exp2f(s * k2);
    return back * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
}

// Folds the sink term of query head h into a row's final state, in natural
// units (scores scale * q.k + mask): m is the reference of the accumulated
// terms (-inf when none) and l their sum relative to it.  Returns the factor
// for the accumulator; m and l become those of the full denominator
// (GroupQueryAttention README, "Inputs": a per-head smooth factor added to
// the softmax denominator).  Differences are taken before scaling, so a
// reference anywhere in the float range cannot overflow.  A -inf sink is no
// term; a NaN or +inf sink makes l NaN.
__device__ __forceinline__ float fold_sink(const Params& p, int h, float& m, float& l) {
    if (!p.sink) return 1.f;
    const float s = p.head_sink ? p.head_sink[h] : 0.f;
    if (s == kNegInf) return 1.f;
    const float M = fmaxf(m, s);
    const float f = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m - M) * kLog2e);
    l = l * f + __builtin_amdgcn_exp2f((s - M) * kLog2e);
    m = M;
    return f;
}

// LSE of a row whose reference m (natural units) and sum l are final and
// l > 0: m + ln l.
__device__ __forceinline__ float row_lse(float m, float l) {
    return fmaf(__builtin_amdgcn_logf(l), kLn2, m);
}

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
