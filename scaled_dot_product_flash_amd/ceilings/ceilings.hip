// ceilings.hip -- what this part reaches on plain loops, as context for the
// attention kernels' roofline fractions (the fractions themselves are taken
// against MI355X's published peaks: 2516.6 TFLOP/s dense bf16, 8 TB/s HBM).
//
//   sdpa_ceiling_mfma_bf16  independent chains of v_mfma_f32_32x32x16_bf16,
//                           four waves per workgroup, no memory traffic;
//   sdpa_ceiling_read       a streaming read of a device buffer (16-byte
//                           loads, four in flight per lane);
//   sdpa_ceiling_copy       a streaming copy of one device buffer into another.
//
// Measurement support only: the attention library does not use these.  Every
// entry point returns the hipError_t of its launch (0 = launched) and checks
// its arguments on the host first (-1 = rejected, nothing launched).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kChains = 4;     // independent accumulators per wave
constexpr int kPerIter = 32;   // MFMAs per wave per loop trip

// Each wave: iters * kPerIter matrix ops of 32x32x16 (32768 flop each).  The
// operands are lane-dependent so nothing folds; one float per lane is
// written so the chains stay live.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * static_cast<float>(lane + i));
        b[i] = static_cast<__bf16>(0.002f * static_cast<float>(lane - i));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kPerIter / kChains; ++r)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte load (the data is used once).
__device__ inline u32x4 ld_once(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Grid-stride streaming read: every lane keeps four 16-byte loads in flight
// and folds them with XOR; one word per lane is written at the end.  (Swept
// on MI355X: non-temporal loads and 32 workgroups per CU read fastest,
// about 6.3 TB/s.)
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ out) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    u32x4 x = {0u, 0u, 0u, 0u};
    size_t i = tid;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = ld_once(src + i), b = ld_once(src + i + stride),
                    c = ld_once(src + i + 2 * stride), d = ld_once(src + i + 3 * stride);
        x ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) x ^= ld_once(src + i);
    out[tid] = x.x ^ x.y ^ x.z ^ x.w;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n16) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = tid;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = ld_once(src + i), b = ld_once(src + i + stride),
                    c = ld_once(src + i + 2 * stride), d = ld_once(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(ld_once(src + i), dst + i);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

// out: float[n_wg * 256] on the device.  Flops = n_wg * 4 * iters * 32 * 32768.
int sdpa_ceiling_mfma_bf16(int n_wg, int iters, float* out, void* stream) {
    if (n_wg <= 0 || iters <= 0 || !out) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_wg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return static_cast<int>(hipGetLastError());
}

// src: `bytes` device bytes (a multiple of 16, 16-byte aligned); out:
// uint32[n_wg * 256] on the device.
int sdpa_ceiling_read(const void* src, size_t bytes, uint32_t* out, int n_wg, void* stream) {
    if (!src || !out || n_wg <= 0 || bytes == 0 || bytes % 16 != 0 || !aligned16(src)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, out);
    return static_cast<int>(hipGetLastError());
}

// src, dst: `bytes` device bytes each (a multiple of 16, 16-byte aligned,
// not overlapping).
int sdpa_ceiling_copy(const void* src, void* dst, size_t bytes, int n_wg, void* stream) {
    if (!src || !dst || n_wg <= 0 || bytes == 0 || bytes % 16 != 0 || !aligned16(src) ||
        !aligned16(dst))
        return -1;
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
