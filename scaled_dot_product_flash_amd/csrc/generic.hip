// generic.hip -- the any-shape attention kernel: every dtype, head_dim 1..256,
// any strides.  One wave owns one query row and walks the keys 64 at a time
// (one key per lane), folding each chunk into a running max / running sum /
// rescaled accumulator (online normaliser: OneGPU "Attention", introduction;
// llm.istanbul "05_attention", "Online Softmax Algoritmasi").  It is the
// fallback for shapes the tuned kernels do not cover, not a fast path.
#include "attn_internal.h"
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kRowsPerBlock = 4;   // one wave per query row
constexpr int kMaxD = 256;

template <typename T>
__global__ __launch_bounds__(256) void generic_kernel(Params p) {
    __shared__ float q_sh[kRowsPerBlock][kMaxD];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + w;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    if (i >= p.Lq) return;                 // whole wave leaves; no block barrier below
    const int g = h / p.group;
    const int D = p.D;

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    int64_t hi = kv_len;
    const int64_t delta = causal_delta(p, kv_len);
    if (p.causal) {
        const int64_t bound = i + delta + 1;   // keys j <= i + delta
        hi = bound < 0 ? 0 : (bound < hi ? bound : hi);
    }
    const int64_t lo = first_key(p, b, i, delta);   // and j >= lo (window, document)

    const int64_t qrow = b * p.qs.sb + h * p.qs.sh + i * p.qs.sr;
    for (int d = lane; d < D; d += 64) q_sh[w][d] = Elem<T>::load(p.q, qrow + d);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    const int64_t kbase = b * p.ks.sb + static_cast<int64_t>(g) * p.ks.sh;
    const int64_t vbase = b * p.vs.sb + static_cast<int64_t>(g) * p.vs.sh;
    const float* mrow = p.mask ? p.mask + b * p.ms.sb + h * p.ms.sh + i * p.ms.sr : nullptr;

    // Scores in natural units, t = scale * q.k (softcapped) + mask, so a large
    // finite mask value stays finite; p = exp2((t - m) * log2 e).
    float m = kNegInf;   // running max
    float l = 0.f;       // running sum of exp(t - m)
    float acc[kMaxD / 64];
#pragma unroll
    for (int c = 0; c < kMaxD / 64; ++c) acc[c] = 0.f;

    for (int64_t j0 = lo; j0 < hi; j0 += 64) {
        const int64_t j = j0 + lane;
        float t = kNegInf;
        if (j < hi) {
            const int64_t kr = kbase + j * p.ks.sr;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(q_sh[w][d], Elem<T>::load(p.k, kr + d), dot);
            const float madd = mrow ? mrow[j] : 0.f;
            if (p.softcap > 0.f)   // softcap on the scaled score, then the mask
                t = p.softcap * tanhf(dot * p.scale / p.softcap) + madd;
            else
                t = fmaf(dot, p.scale, madd);
        }
        const float m_new = fmaxf(m, wave_max(t));
        const float base = (m_new == kNegInf) ? 0.f : m_new;   // all hidden so far: exp2(-inf) = 0
        const float pj = fast_exp2((t - base) * kLog2e);
        const float alpha = fast_exp2((m - base) * kLog2e);
        l = l * alpha + wave_sum(pj);
#pragma unroll
        for (int c = 0; c < kMaxD / 64; ++c) acc[c] *= alpha;
        const int n = static_cast<int>((hi - j0) < 64 ? (hi - j0) : 64);
        for (int jj = 0; jj < n; ++jj) {
            // Uniform lane index: a scalar read of lane jj's weight.
            const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj));
            const int64_t vr = vbase + (j0 + jj) * p.vs.sr;
#pragma unroll
            for (int c = 0; c < kMaxD / 64; ++c) {
                const int d = lane + 64 * c;
                if (d < D) acc[c] = fmaf(pw, Elem<T>::load(p.v, vr + d), acc[c]);
            }
        }
        m = m_new;
    }

    const int64_t orow = b * p.os.sb + h * p.os.sh + i * p.os.sr;
    const float fs = fold_sink(p, h, m, l);
    const bool empty = (l == 0.f);
    const float inv = fs / l;
#pragma unroll
    for (int c = 0; c < kMaxD / 64; ++c) {
        const int d = lane + 64 * c;
        if (d < D) {
            float r = acc[c] * inv;
            if (empty) r = p.masked_zero ? 0.f : __builtin_nanf("");
            Elem<T>::store(p.o, orow + d, r);
        }
    }
    if (p.lse && lane == 0) {
        const float lse = empty ? kNegInf : row_lse(m, l);
        p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = lse;
    }
}

}  // namespace

hipError_t launch_generic(const Params& p, DType dt, hipStream_t s) {
    const dim3 grid((p.Lq + kRowsPerBlock - 1) / kRowsPerBlock, p.Hq, p.B);
    const dim3 block(64 * kRowsPerBlock);
    switch (dt) {
    case DType::F32: hipLaunchKernelGGL(generic_kernel<float>, grid, block, 0, s, p); break;
    case DType::F16: hipLaunchKernelGGL(generic_kernel<_Float16>, grid, block, 0, s, p); break;
    case DType::BF16: hipLaunchKernelGGL(generic_kernel<bf16_t>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

}  // namespace sdpa
