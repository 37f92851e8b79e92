// decode.hip -- single-query attention against a key/value cache, split over
// the keys, plus the ordered merge of the per-range partials.
//
// Decode reads every live key/value row once and does little arithmetic per
// byte, so it is bound by HBM bandwidth.  One key range of one (batch,
// kv-head) is one workgroup: the G = Hq/Hkv query heads that share the kv head
// are served by the same read of the cache.  The keys are cut into ranges of a
// fixed length chosen from the shape alone, each range's partial (reference
// max, sum, unnormalised accumulator) goes to the workspace, and a second
// kernel merges the ranges of each (batch, head) in increasing range order
// (OneGPU "Attention", "Accuracy at long key lengths", last paragraph; ONNX
// GroupQueryAttention README, split-K decode variants).  The query row against
// the cache follows llm.istanbul "05_attention", "attention_decode Farki".
//
// Inside a range, 128-key tiles are staged through LDS with coalesced 16-byte
// loads (prefetched into registers during the previous tile's math); each of
// the 4 waves takes 32 keys of the tile and runs the same matrix-core scheme
// as the prefill kernel with the G heads as the query columns of
// S^T = K Q^T (unused columns are zero).  The 4 waves' states are merged in
// wave order through LDS before the partial is written.
#include "attn_internal.h"
#include "device_common.h"
#include "mfma_common.h"

#include <cstdlib>

namespace sdpa {

namespace {

using namespace mfma;

constexpr int kStep = 32;        // keys per wave step (two 16-key MFMA blocks)
constexpr int kWaves = 1;        // one wave per workgroup: no LDS held by finished waves
constexpr float kSlack = 8.f;    // lazy-rescale threshold, base-2 units

// Wave-private LDS rows.  K rows are read 16 lanes x 16 bytes down one column
// (stride 16 mod 256 bytes spreads them over the banks); V rows are read by
// the transpose load, 8 rows x 32 bytes per 32 lanes (stride 32 mod 256 bytes).
template <int D> struct DLay {
    static constexpr int KS = D + 8;
    static constexpr int VS = D + 16;
    static constexpr int kRowChunks = D / 8;                 // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kRowChunks;     // rows one wave load covers
    static constexpr int kLoads = kStep / kRowsPerLoad;      // loads per lane per tensor
    static constexpr int kWaveBytes = kStep * (KS + VS) * 2;
};

// Partial record of one (b, h, range): [m, l, -, -, acc[0..D)], floats.
__host__ __device__ constexpr int rec_stride(int D) { return D + 4; }

__device__ __forceinline__ int64_t live_keys(const Params& p, int b) {
    int64_t kv = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    if (p.causal) {                  // the one query row is i = 0
        const int64_t bb = p.delta + 1;
        kv = bb < 0 ? 0 : (bb < kv ? bb : kv);
    }
    return kv;
}

// Each wave owns one key range of one (b, kv head, group of up to 16 query
// heads) and walks it in 32-key steps: the next step's K/V rows are loaded
// into registers (coalesced, 16 bytes per lane) while the current step runs
// from the wave's own LDS rows.  No workgroup barrier anywhere: the waves of a
// workgroup only share the launch.
template <bool kBf16, int D>
__global__ __launch_bounds__(64) void decode_split_kernel(Params p, int n_hgrp) {
    using M = Mma<kBf16>;
    using LY = DLay<D>;
    constexpr int KS = LY::KS, VS = LY::VS;
    constexpr int NT = D / 32;       // 32-wide d-steps of the score product
    constexpr int ND = D / 16;       // 16-row d-tiles of the output
    __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * LY::kWaveBytes];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x * kWaves + w;                // key range
    const int g = blockIdx.y / n_hgrp;                    // kv head
    const int hbase = (blockIdx.y % n_hgrp) * 16;         // first query head of the group slice
    const int b = blockIdx.z;
    const int64_t kv_hi = live_keys(p, b);
    const int64_t j_begin = static_cast<int64_t>(r) * p.split_len;
    if (r >= p.n_split || j_begin >= kv_hi) return;      // the merge reads only live ranges
    const int64_t j_end = (j_begin + p.split_len < kv_hi) ? j_begin + p.split_len : kv_hi;
    const int n_steps = static_cast<int>((j_end - j_begin + kStep - 1) / kStep);

    uint16_t* const k_sh = reinterpret_cast<uint16_t*>(smem + w * LY::kWaveBytes);
    uint16_t* const v_sh = k_sh + kStep * KS;
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v) + b * p.vs.sb + g * p.vs.sh;

    const int col = lane & 15, q4 = lane >> 4;
    const bool live_col = hbase + col < p.group;
    const int h = g * p.group + (live_col ? hbase + col : 0);

    // Q^T operand (16x16x32 B layout): column col, d = 32t + 8*q4 + e.
    i16x8 qop[NT];
    {
        const uint16_t* src = static_cast<const uint16_t*>(p.q) + b * p.qs.sb + h * p.qs.sh + 8 * q4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const i16x8 v = *reinterpret_cast<const i16x8*>(src + 32 * t);
            qop[t] = live_col ? v : i16x8{};
        }
    }
    const float* mrow = (p.mask && live_col) ? p.mask + b * p.ms.sb + h * p.ms.sh : nullptr;

    // Coalesced staging: one load covers kRowsPerLoad whole rows.  Raw buffer
    // loads whose range ends at this wave's last key return zeros past it, so
    // the tail needs no branch and rows beyond the length are never read.
    const int ld_row = lane / LY::kRowChunks;
    const int ld_col = (lane % LY::kRowChunks) * 8;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, j_end * p.ks.sr * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, j_end * p.vs.sr * 2);
    i16x8 kst[LY::kLoads], vst[LY::kLoads];
    auto fetch = [&](int step) {
        const int j0 = static_cast<int>(j_begin) + step * kStep + ld_row;
#pragma unroll
        for (int n = 0; n < LY::kLoads; ++n) {
            const int key = j0 + n * LY::kRowsPerLoad;
            kst[n] = load16(krs, (key * static_cast<int>(p.ks.sr) + ld_col) * 2);
            vst[n] = load16(vrs, (key * static_cast<int>(p.vs.sr) + ld_col) * 2);
        }
    };

    float m_ref = kNegInf, l_sum = 0.f;
    f32x4 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x4{};

    fetch(0);
    for (int step = 0; step < n_steps; ++step) {
        // The previous step's LDS reads were issued before these writes, and one
        // wave's LDS operations complete in order, so a single buffer suffices.
#pragma unroll
        for (int n = 0; n < LY::kLoads; ++n) {
            const int row = n * LY::kRowsPerLoad + ld_row;
            *reinterpret_cast<i16x8*>(&k_sh[row * KS + ld_col]) = kst[n];
            *reinterpret_cast<i16x8*>(&v_sh[row * VS + ld_col]) = vst[n];
        }
        if (step + 1 < n_steps) fetch(step + 1);
        const int64_t j0 = j_begin + static_cast<int64_t>(step) * kStep;

        // S^T = K Q^T: two 16-key blocks; lane holds keys kb*16 + 4*q4 + rr of column col.
        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{};
            const uint16_t* krow = &k_sh[(kb * 16 + col) * KS + 8 * q4];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                s[kb] = M::mfma16(*reinterpret_cast<const i16x8*>(krow + 32 * t), qop[t], s[kb]);
        }
        const bool partial = j0 + kStep > j_end;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int64_t key0 = j0 + kb * 16 + 4 * q4;
            float madd[4] = {0.f, 0.f, 0.f, 0.f};
            if (mrow) {
#pragma unroll
                for (int e = 0; e < 4; ++e) madd[e] = (key0 + e < j_end) ? mrow[key0 + e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t = fmaf(s[kb][e], p.scale_log2, madd[e] * kLog2e);
                if (partial && key0 + e >= j_end) t = kNegInf;
                s[kb][e] = t;
            }
        }
        // Row maximum over the 4 lanes that share column col.
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool raise = mx > m_ref + kSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mx : m_ref;
            const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;   // 0 when m_ref = -inf
            l_sum *= alpha;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[d][e] *= alpha;
            m_ref = m_new;
        }
        const float base = (m_ref == kNegInf) ? 0.f : m_ref;
        // P^T operand (16x16x32 B layout): k = 8*q4 + e <-> key (e < 4 ? 4*q4 + e : 16 + 4*q4 + e - 4).
        uint32_t w4[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float ra, rb;
                w4[2 * kb + e] = M::pack(fast_exp2(s[kb][2 * e] - base),
                                         fast_exp2(s[kb][2 * e + 1] - base), ra, rb);
                l_sum += ra + rb;
            }
        }
        const i16x8 pop = __builtin_bit_cast(i16x8, (uint4){w4[0], w4[1], w4[2], w4[3]});
        // O^T += V^T P^T; V^T from the transpose read: rows 4*q4 + i/4 (+16), cols 16*dt + 4*(i%4).
        const int gi = lane & 15;
        const uint16_t* v0 = &v_sh[(4 * q4 + (gi >> 2)) * VS + 4 * (gi & 3)];
        const uint16_t* v1 = v0 + 16 * VS;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const i16x4 lo = tr_read(v0 + 16 * d);
            const i16x4 hi = tr_read(v1 + 16 * d);
            const i16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[d] = M::mfma16(a, pop, acc[d]);
        }
    }

    // Column total of the running sum: the 4 lanes of column col, fixed order.
    float lt = l_sum + __shfl_xor(l_sum, 16, 64);
    lt = lt + __shfl_xor(lt, 32, 64);
    if (live_col) {
        float* rec = static_cast<float*>(p.ws) +
                     ((static_cast<int64_t>(b) * p.Hq + h) * p.n_split + r) * rec_stride(D);
#pragma unroll
        for (int d = 0; d < ND; ++d)
            *reinterpret_cast<f32x4*>(rec + 4 + 16 * d + 4 * q4) = acc[d];
        if (q4 == 0) {
            rec[0] = m_ref;
            rec[1] = lt;
        }
    }
}

// One wave per (b, h): merge the live ranges in increasing order.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (bh >= static_cast<int64_t>(p.B) * p.Hq) return;
    const int b = static_cast<int>(bh / p.Hq), h = static_cast<int>(bh % p.Hq);
    const int64_t kv_hi = live_keys(p, b);
    const int n_live = static_cast<int>((kv_hi + p.split_len - 1) / p.split_len);
    const int rs = rec_stride(D);
    const float* recs = static_cast<const float*>(p.ws) + bh * p.n_split * rs;
    constexpr int NPL = (D + 63) / 64;
    float M = kNegInf, L = 0.f, A[NPL];
#pragma unroll
    for (int c = 0; c < NPL; ++c) A[c] = 0.f;
    // Ranges in batches of 64: lane r of a batch loads range r's (m, l).
    for (int r0 = 0; r0 < n_live; r0 += 64) {
        const int n = (n_live - r0) < 64 ? (n_live - r0) : 64;
        const float mr = lane < n ? recs[(r0 + lane) * rs] : kNegInf;
        const float lr = lane < n ? recs[(r0 + lane) * rs + 1] : 0.f;
        const float Mb = wave_max(mr);
        const float Mn = fmaxf(M, Mb);
        // Rescale what earlier batches accumulated (only when the max moved).
        if (Mn > M) {
            const float a = (M == kNegInf) ? 0.f : fast_exp2(M - Mn);
            L *= a;
#pragma unroll
            for (int c = 0; c < NPL; ++c) A[c] *= a;
            M = Mn;
        }
        const float f = (mr == kNegInf) ? 0.f : fast_exp2(mr - M);
        const float lf = lr * f;
        // In range order: uniform loop, the weight of range r read from lane r.
        for (int i = 0; i < n; i += 8) {
            float val[8][NPL], fw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int rr = (i + u < n) ? i + u : i;
                fw[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), rr));
#pragma unroll
                for (int c = 0; c < NPL; ++c) {
                    const int d = lane + 64 * c;
                    val[u][c] = (d < D) ? recs[(r0 + rr) * rs + 4 + d] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (i + u < n) {
                    L += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lf), i + u));
#pragma unroll
                    for (int c = 0; c < NPL; ++c) A[c] = fmaf(val[u][c], fw[u], A[c]);
                }
            }
        }
    }
    const bool empty = (L == 0.f);
    const float inv = 1.f / L;
    const int64_t orow = b * p.os.sb + h * p.os.sh;
#pragma unroll
    for (int c = 0; c < NPL; ++c) {
        const int d = lane + 64 * c;
        if (d < D) {
            const float o = empty ? (p.masked_zero ? 0.f : __builtin_nanf("")) : A[c] * inv;
            Elem<T>::store(p.o, orow + d, o);
        }
    }
    if (p.lse && lane == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh] = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
}

template <bool kBf16, int D>
hipError_t launch_one(const Params& p, hipStream_t s) {
    const int n_hgrp = (p.group + 15) / 16;
    const dim3 grid((p.n_split + kWaves - 1) / kWaves, p.Hkv * n_hgrp, p.B);
    hipLaunchKernelGGL((decode_split_kernel<kBf16, D>), grid, dim3(64 * kWaves), 0, s, p, n_hgrp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq;
    const dim3 cgrid(static_cast<uint32_t>((rows + 3) / 4));
    if (kBf16)
        hipLaunchKernelGGL((decode_combine_kernel<bf16_t, D>), cgrid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((decode_combine_kernel<_Float16, D>), cgrid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Key range length (keys per wave): about a tenth of the cache capacity, a
// multiple of the 32-key step, between 256 and 4096 keys, so a long cache
// is cut into ~10 ranges per (batch, kv head) and a short one into few.
// (Measured on fp16 B=64 Hkv=8 D=128 with an 8192-key cache: 768-896 keys
// per range beat 256-640 and 1024-2048.)  SDPA_FLASH_DECODE_SPLIT=<keys>
// overrides it (tuning only).
void decode_split_plan(int Lk, int* split_len, int* n_split) {
    int len = Lk / 10;
    len = len / 128 * 128;
    if (len < 256) len = 256;
    if (len > 4096) len = 4096;
    if (const char* e = std::getenv("SDPA_FLASH_DECODE_SPLIT")) {
        const int v = std::atoi(e);
        if (v >= kStep) len = v;
    }
    len = (len + kStep - 1) / kStep * kStep;
    *split_len = len;
    *n_split = Lk > 0 ? (Lk + len - 1) / len : 0;
}

size_t decode_workspace_bytes(int B, int Hq, int Lk, int D) {
    int len, n;
    decode_split_plan(Lk, &len, &n);
    return static_cast<size_t>(B) * Hq * n * rec_stride(D) * sizeof(float);
}

bool decode_split_supported(const Params& p, DType dt) {
    if (dt != DType::BF16 && dt != DType::F16) return false;
    if (p.D != 64 && p.D != 128) return false;
    if (p.Lq != 1 || p.Lk == 0) return false;
    if (static_cast<int64_t>(p.Hkv) * ((p.group + 15) / 16) > 65535 || p.B > 65535) return false;
    // Buffer offsets of one (b, kv head) slice are 32-bit.
    if (p.ks.sr >= (1 << 24) || p.vs.sr >= (1 << 24)) return false;
    if ((static_cast<int64_t>(p.Lk) * p.ks.sr + p.D) * 2 >= (int64_t(1) << 31) ||
        (static_cast<int64_t>(p.Lk) * p.vs.sr + p.D) * 2 >= (int64_t(1) << 31))
        return false;
    if ((static_cast<int64_t>(p.n_split) + 3) / 4 > 0x7fffffff) return false;
    auto al = [](const void* ptr, const Strides& st, int a) {
        return reinterpret_cast<uintptr_t>(ptr) % (2 * a) == 0 && st.sb % a == 0 &&
               st.sh % a == 0 && st.sr % a == 0;
    };
    return al(p.q, p.qs, 8) && al(p.k, p.ks, 8) && al(p.v, p.vs, 8);
}

hipError_t launch_decode_split(const Params& p, DType dt, hipStream_t s) {
    if (dt == DType::BF16) return p.D == 128 ? launch_one<true, 128>(p, s) : launch_one<true, 64>(p, s);
    return p.D == 128 ? launch_one<false, 128>(p, s) : launch_one<false, 64>(p, s);
}

}  // namespace sdpa
