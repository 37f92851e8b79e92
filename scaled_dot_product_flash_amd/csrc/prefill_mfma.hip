// prefill_mfma.hip -- fused attention for bf16 / fp16 inputs with fp32
// accumulation on the gfx950 matrix cores (head_dim 64 or 128).
//
// Work decomposition.  A workgroup of 4 waves owns one (batch, query head,
// block of 128 query rows); each wave owns 32 rows.  The keys are visited in
// increasing order, 64 per tile, staged through LDS (double buffered, one
// barrier per tile) with coalesced 16-byte global loads; rows past the key
// length are zero-filled and never read from memory.  (OneGPU "Attention",
// introduction and "Variants and ordering": a workgroup keeps a block of query
// rows and walks key/value tiles held in workgroup memory.)
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
// output column is the query, so lane l owns query l%32 and holds 16 of its
// keys per 32-key block; lane l^32 holds the other 16.  A row's maximum is an
// in-lane reduction plus one exchange with lane l^32 (OneGPU "Apple simdgroup
// kernel": scores transposed so one lane keeps one row).
//
// Online normaliser (OneGPU "Attention", introduction; llm.istanbul
// "05_attention", "Online Softmax Algoritmasi") with a lazily raised reference
// maximum: the reference m only moves when a tile's maximum exceeds it by more
// than 8 (base 2), so exp2(t - m) <= 2^8 and the accumulator is rescaled
// rarely (OneGPU "Apple simdgroup kernel", reference maximum).  Raising is a
// per-row decision taken identically in both lanes of the row, from data only.
//
// P is rounded to the element type before the P V product and the running sum
// adds the rounded values, so numerator and denominator see the same p
// (OneGPU "Matrix hardware").  O^T = V^T P^T runs on the same MFMA shape: the
// rounded scores are already in the B-operand layout, and the V^T operand is
// read from the row-major V tile with the LDS transpose read ds_read_b64_tr_b16.
//
// Special values (OneGPU "Special values"): hidden keys get -inf and weigh 0;
// a row whose reference max is still -inf uses 0 as the exponent base, so
// exp2(-inf) = 0 and never exp2(-inf - -inf); a row with no visible key ends
// with l == 0 and follows the masked-row policy; NaN / +inf scores make l NaN.
#include "attn_internal.h"
#include "device_common.h"

namespace sdpa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr float kSlack = 8.f;  // lazy-rescale threshold, base-2 units

template <bool kBf16> struct Mma;

template <> struct Mma<true> {
    using vec8 = bf16x8;
    static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
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
};

template <> struct Mma<false> {
    using vec8 = f16x8;
    static __device__ __forceinline__ f32x16 mfma(i16x8 a, i16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
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
};

// LDS row strides (elements).  K rows are read 16 lanes x 16 bytes at a time
// down one column: a stride of 16 mod 256 bytes spreads them over all banks.
// V rows are read by the transpose load, 4 rows x 64 bytes per 32 lanes: a
// stride of 64 mod 256 bytes keeps those rows apart.
template <int D> struct Tile {
    static constexpr int KS = D + 8;
    static constexpr int VS = D + 32;
    static constexpr int kChunks = kBN * D / 8;              // 16-byte chunks per tile
    static constexpr int kLoads = kChunks / (64 * kWaves);   // per thread
    static constexpr int kRowChunks = D / 8;
};

__device__ __forceinline__ i16x4 tr_read(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3)))*)(
            (__attribute__((address_space(3))) uint16_t*)(p)));
}

template <bool kBf16, int D>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(Params p, int n_qblk,
                                                              int xcd_units, int mask_vec4) {
    using M = Mma<kBf16>;
    using TL = Tile<D>;
    constexpr int KS = TL::KS, VS = TL::VS;
    constexpr int NT = D / 16;   // 16-wide d-steps of the score product
    constexpr int ND = D / 32;   // 32-row d-tiles of the output
    __shared__ __attribute__((aligned(16))) uint16_t k_sh[2][kBN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t v_sh[2][kBN * VS];

    // ---- which (b, h, query block) this workgroup owns -------------------
    // Heaviest causal blocks first.  When the (batch, kv-head) units split
    // evenly over the 8 XCDs (consecutive workgroups go to consecutive XCDs),
    // each XCD keeps whole units so the query heads sharing K/V share its L2.
    int b, h, qb;
    {
        const int L = blockIdx.x;
        if (xcd_units > 0) {
            const int xcd = L & 7, slot = L >> 3;
            const int per = xcd_units * p.group;
            qb = n_qblk - 1 - slot / per;
            const int rem = slot % per;
            const int unit = xcd * xcd_units + rem / p.group;
            b = unit / p.Hkv;
            h = (unit % p.Hkv) * p.group + rem % p.group;
        } else {
            const int bh = p.B * p.Hq;
            qb = n_qblk - 1 - L / bh;
            const int rem = L % bh;
            b = rem / p.Hq;
            h = rem % p.Hq;
        }
    }
    const int g = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hh = lane >> 5;          // which half of the wave
    const int col = lane & 31;         // query column owned by this lane

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const int64_t q0 = static_cast<int64_t>(qb) * kBM;
    const int64_t qw0 = q0 + 32 * w;
    // Keys the block needs: [0, blk_hi); keys this wave can see: [0, wave_hi).
    int64_t blk_hi = kv_len, wave_hi = kv_len;
    if (p.causal) {
        const int64_t last = (q0 + kBM < p.Lq ? q0 + kBM : p.Lq) - 1;
        const int64_t bb = last + p.delta + 1;
        blk_hi = bb < 0 ? 0 : (bb < blk_hi ? bb : blk_hi);
        const int64_t wl = (qw0 + 32 < p.Lq ? qw0 + 32 : p.Lq) - 1;
        const int64_t wb = wl + p.delta + 1;
        wave_hi = wb < 0 ? 0 : (wb < wave_hi ? wb : wave_hi);
    }
    if (qw0 >= p.Lq) wave_hi = 0;
    const int n_tiles = static_cast<int>((blk_hi + kBN - 1) / kBN);

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v) + b * p.vs.sb + g * p.vs.sh;

    // ---- Q^T operand, resident in registers -------------------------------
    const int64_t qrow = qw0 + col;
    i16x8 qop[NT];
    {
        const bool ok = qrow < p.Lq;
        const uint16_t* src = qg + b * p.qs.sb + h * p.qs.sh + (ok ? qrow : 0) * p.qs.sr + 8 * hh;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            i16x8 v = *reinterpret_cast<const i16x8*>(src + 16 * t);
            qop[t] = ok ? v : i16x8{};
        }
    }

    // ---- staging of one K/V tile: global -> registers -> LDS --------------
    i16x8 kst[TL::kLoads], vst[TL::kLoads];
    auto fetch = [&](int tile) {
        const int64_t j0 = static_cast<int64_t>(tile) * kBN;
#pragma unroll
        for (int n = 0; n < TL::kLoads; ++n) {
            const int c = tid + 256 * n;
            const int r = c / TL::kRowChunks;
            const int cc = (c % TL::kRowChunks) * 8;
            const int64_t key = j0 + r;
            if (key < kv_len) {
                kst[n] = *reinterpret_cast<const i16x8*>(kg + key * p.ks.sr + cc);
                vst[n] = *reinterpret_cast<const i16x8*>(vg + key * p.vs.sr + cc);
            } else {
                kst[n] = i16x8{};
                vst[n] = i16x8{};
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int n = 0; n < TL::kLoads; ++n) {
            const int c = tid + 256 * n;
            const int r = c / TL::kRowChunks;
            const int cc = (c % TL::kRowChunks) * 8;
            *reinterpret_cast<i16x8*>(&k_sh[buf][r * KS + cc]) = kst[n];
            *reinterpret_cast<i16x8*>(&v_sh[buf][r * VS + cc]) = vst[n];
        }
    };

    const float* mrow = nullptr;
    if (p.mask && qrow < p.Lq) mrow = p.mask + b * p.ms.sb + h * p.ms.sh + qrow * p.ms.sr;

    float m_ref = kNegInf;   // reference maximum of this lane's row (base 2)
    float l_sum = 0.f;       // this lane's share of the running sum
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x16{};

    if (n_tiles > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < n_tiles) fetch(tile + 1);
        const int64_t j0 = static_cast<int64_t>(tile) * kBN;

        if (j0 < wave_hi) {
            // -- S^T = K Q^T for two 32-key blocks --
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                const uint16_t* krow = &k_sh[buf][(kb * 32 + col) * KS + 8 * hh];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const i16x8 a = *reinterpret_cast<const i16x8*>(krow + 16 * t);
                    s[kb] = M::mfma(a, qop[t], s[kb]);
                }
            }
            // -- scores in base-2 units; hide keys past the length / causal bound --
            const bool partial = (j0 + kBN > kv_len) ||
                                 (p.causal && j0 + kBN - 1 > qw0 + p.delta);
            const int64_t qlim = qrow + p.delta;   // causal: key <= qlim
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kofs = kb * 32 + 8 * u + 4 * hh;   // first of 4 keys
                    float madd[4] = {0.f, 0.f, 0.f, 0.f};
                    if (mrow) {
                        const int64_t key = j0 + kofs;
                        if (mask_vec4 && key + 3 < kv_len) {
                            const float4 mv = *reinterpret_cast<const float4*>(mrow + key);
                            madd[0] = mv.x; madd[1] = mv.y; madd[2] = mv.z; madd[3] = mv.w;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                madd[e] = (key + e < kv_len) ? mrow[key + e] : 0.f;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * u + e;
                        float t = fmaf(s[kb][r], p.scale_log2, madd[e] * kLog2e);
                        if (partial) {
                            const int64_t key = j0 + kofs + e;
                            const bool hidden = key >= kv_len || (p.causal && key > qlim);
                            t = hidden ? kNegInf : t;
                        }
                        s[kb][r] = t;
                    }
                }
            }
            // -- row maximum: 32 values in-lane, then the partner lane --
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // -- lazy raise of the reference maximum --
            const bool raise = mx > m_ref + kSlack;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float m_new = raise ? mx : m_ref;
                // 0 when m_ref = -inf; rows that do not raise keep alpha = 1 exactly.
                const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;
                l_sum *= alpha;
#pragma unroll
                for (int d = 0; d < ND; ++d)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
                m_ref = m_new;
            }
            const float base = (m_ref == kNegInf) ? 0.f : m_ref;
            // -- p = exp2(t - base), rounded to the element type; l sums the rounded p --
            i16x8 pop[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    uint32_t w4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 8 * st + 2 * e;
                        float ra, rb;
                        w4[e] = M::pack(fast_exp2(s[kb][r] - base), fast_exp2(s[kb][r + 1] - base),
                                        ra, rb);
                        l_sum += ra + rb;
                    }
                    pop[kb][st] = __builtin_bit_cast(i16x8, (uint4){w4[0], w4[1], w4[2], w4[3]});
                }
            }
            // -- O^T += V^T P^T; V^T comes from the transpose read of row-major V --
            const int gi = lane & 15;
            const int dsub = 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int row = kb * 32 + 16 * st + 4 * hh + (gi >> 2);
                    const uint16_t* v0 = &v_sh[buf][row * VS + dsub];
                    const uint16_t* v1 = v0 + 8 * VS;
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const i16x4 lo = tr_read(v0 + 32 * d);
                        const i16x4 hi = tr_read(v1 + 32 * d);
                        const i16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc[d] = M::mfma(a, pop[kb][st], acc[d]);
                    }
                }
            }
        }
        if (tile + 1 < n_tiles) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l (or the masked-row policy), LSE = m + log l --
    const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
    if (qrow < p.Lq) {
        const bool empty = (l_tot == 0.f);
        const float inv = 1.f / l_tot;
        const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
        uint16_t* og = static_cast<uint16_t*>(p.o) + b * p.os.sb + h * p.os.sh + qrow * p.os.sr;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float o4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = empty ? fill : acc[d][4 * u + e] * inv;
                const uint2 pk = {M::pack_out(o4[0], o4[1]), M::pack_out(o4[2], o4[3])};
                *reinterpret_cast<uint2*>(og + 32 * d + 8 * u + 4 * hh) = pk;
            }
        }
        if (p.lse && hh == 0) {
            const float lse = empty ? kNegInf : (m_ref + fast_log2(l_tot)) * kLn2;
            p.lse[b * p.ls.sb + h * p.ls.sh + qrow * p.ls.sr] = lse;
        }
    }
}

template <bool kBf16, int D>
hipError_t launch_one(const Params& p, hipStream_t s) {
    const int n_qblk = (p.Lq + kBM - 1) / kBM;
    const int units = p.B * p.Hkv;
    const int xcd_units = (units % 8 == 0) ? units / 8 : 0;
    const int mask_vec4 = p.mask && (reinterpret_cast<uintptr_t>(p.mask) % 16 == 0) &&
                          p.ms.sb % 4 == 0 && p.ms.sh % 4 == 0 && p.ms.sr % 4 == 0;
    const int64_t blocks = static_cast<int64_t>(n_qblk) * p.B * p.Hq;
    hipLaunchKernelGGL((prefill_mfma_kernel<kBf16, D>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(256), 0, s, p, n_qblk, xcd_units, mask_vec4);
    return hipGetLastError();
}

}  // namespace

bool prefill_mfma_supported(const Params& p, DType dt) {
    if (dt != DType::BF16 && dt != DType::F16) return false;
    if (p.D != 64 && p.D != 128) return false;
    // 16-byte loads of Q/K/V rows and 8-byte stores of O need aligned rows.
    auto al = [](const void* ptr, const Strides& st, int a) {
        return reinterpret_cast<uintptr_t>(ptr) % (2 * a) == 0 && st.sb % a == 0 &&
               st.sh % a == 0 && st.sr % a == 0;
    };
    if (!al(p.q, p.qs, 8) || !al(p.o, p.os, 4)) return false;
    if (p.Lk > 0 && (!al(p.k, p.ks, 8) || !al(p.v, p.vs, 8))) return false;
    const int64_t blocks = static_cast<int64_t>((p.Lq + kBM - 1) / kBM) * p.B * p.Hq;
    return blocks < (int64_t(1) << 31);
}

hipError_t launch_prefill_mfma(const Params& p, DType dt, hipStream_t s) {
    if (dt == DType::BF16) return p.D == 128 ? launch_one<true, 128>(p, s) : launch_one<true, 64>(p, s);
    return p.D == 128 ? launch_one<false, 128>(p, s) : launch_one<false, 64>(p, s);
}

}  // namespace sdpa
