// decode.hip -- single-query attention against a key/value cache, split over
// the keys, plus the ordered merge of the partials.
//
// Decode reads every live key/value row once and does little arithmetic per
// byte, so it is bound by HBM bandwidth.  The G = Hq/Hkv query heads sharing a
// kv head are served by the same read of the cache (up to 16 heads per pass;
// larger groups are cut into slices of 16).  A *unit* is one (batch entry, kv
// head, head slice); its live keys (the batch entry's length, clamped, and the
// causal bound of the one query row) form ceil(len/32) steps of 32 keys.
//
// Load balance.  Per-batch lengths differ widely, so cutting each unit into
// fixed ranges leaves the GPU half idle at the end.  Instead W waves (1024
// or 2048 by head dim and cache type: four or eight per CU of an MI355X; as
// many as there are steps when there are fewer) each take an equal
// contiguous share of the concatenated steps of all units, in unit order;
// every wave computes the same per-batch prefix sums from the lengths, so the
// cut needs no host round trip.  A wave writes one partial record (reference max, sum,
// unnormalised accumulator) for each unit it touches, at slot (unit + wave):
// waves and units advance together, so no two (unit, wave) pairs share a slot,
// and U + W - 1 slots suffice.  The merge kernel recomputes which waves cover
// a unit and folds their records in wave order, i.e. in key order (OneGPU
// "Attention", "Accuracy at long key lengths", last paragraph: ranges store
// partials, a second pass merges them in range order; ONNX GroupQueryAttention
// README, split-K decode variants).  The query row against the cache follows
// llm.istanbul "05_attention", "attention_decode Farki".
//
// Unit mode, for calls too small to need that balance (a few steps per
// wave): one workgroup per unit, its waves taking equal contiguous shares of
// the unit's steps; the workgroup folds its waves' partials in LDS in wave
// order (key order) and writes the outputs, with no workspace records and no
// merge kernel.  The host picks the mode from the shape.
//
// A step: K/V rows are loaded with coalesced 16-byte raw-buffer loads bounded
// at the unit's live length (zeros past it; rows past the length are never
// read), marked non-temporal since each byte is read once, and prefetched
// into registers one step ahead, also across unit boundaries; the wave
// stores them in its own LDS rows (no barriers) and runs S^T = K Q^T and
// O^T += V^T P^T on 16x16x32 MFMAs with the query heads as the columns.
// Online normaliser with a lazily raised reference maximum; P is rounded to
// the element type and the sum adds the rounded values.  Scores are raw
// (q.k) without a mask and natural (scale * q.k + mask, the mask added as
// given) with one, so a large finite mask value stays finite.
//
// Score-rule variants (ONNX GroupQueryAttention README, "Attributes",
// "Inputs"): a local window moves the start of the live range up (the range
// is [lo, hi) and steps count from lo); the softcap maps raw scores before
// the mask; the sink joins the denominator in the merge.
//
// fp32 Q/K/V (head dims up to 128): the same steps on 16x16x4 fp32 matrix
// operations, P not rounded; rows staged as fp32 in LDS.
//
// Int8 cache (GroupQueryAttention README, "Inputs": k_scale / v_scale): rows
// are read as 16-byte loads of 16 int8 values -- half the bytes of fp16 --
// stored in LDS as they are, and widened to the element type as the MFMA
// operands are read (exact: |x| <= 128): K rows by 8-byte reads, V columns
// by the 8-bit transpose read, half the LDS bytes of widened rows.
// A per-tensor K scale multiplies the exponent constant (exact); a
// per-channel K scale is folded into the query row, rounded to the element
// type.  V scales apply per output element in the merge, where they factor
// out of the sum over keys.
#include "attn_internal.h"
#include "device_common.h"
#include "mfma_common.h"

namespace sdpa {

namespace {

using namespace mfma;

constexpr int kStep = 32;          // keys per wave step (two 16-key MFMA blocks)

// Persistent waves (256 CUs) for padded head dim DP and cache type, the
// fastest of 1024 / 1536 / 2048 measured on each: four per CU for 16-bit
// caches at 128 and 256 (at 256 the LDS rows are twice as long), eight for
// 64 and for int8 caches, whose steps carry fewer bytes.
__host__ __device__ constexpr int waves_total(int DP, bool i8) {
    return DP > 128 || (DP == 128 && !i8) ? 1024 : 2048;
}
constexpr int kWavesMax = 2048;
// Unit mode: waves per workgroup at most, for padded head dim DP and cache
// type (the register budget of a workgroup that size: at 64, four waves per
// SIMD; at 128 and for int8 rows at 256, two; 16-bit rows at 256, one; fp32
// rows: what fits the LDS, 8 at 64 and 4 at 128).
__host__ __device__ constexpr int unit_waves_max(int DP, bool i8, bool f32 = false) {
    return f32 ? (DP == 64 ? 8 : 4) : (DP == 64 ? 16 : (DP == 128 || i8 ? 8 : 4));
}
constexpr float kSlack = 8.f;      // lazy-rescale threshold, base-2 units

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

// Int8 rows: 16 values per 16-byte load, kept as int8 in LDS (rows of RS
// bytes, K and V alike; 16 bytes of padding keep the 8-byte K reads and the
// transposing V reads within two-way bank conflicts).
template <int D> struct I8Lay {
    static constexpr int kRowChunks = D / 16;
    static constexpr int kRowsPerLoad = 64 / kRowChunks;
    static constexpr int kLoads = kStep / kRowsPerLoad;
    static constexpr int RS = D + 16;
    static constexpr int kWaveBytes = kStep * 2 * RS;
};

// fp32 rows (fp32 Q/K/V, head dims up to 128): 4 floats per 16-byte load,
// rows of RS floats (16 bytes of padding) for K and V alike.  The K reads
// (16 bytes per lane, 16 rows) land 16 bytes mod 256 apart on the banks.
template <int D> struct F32Lay {
    static constexpr int kRowChunks = D / 4;
    static constexpr int kRowsPerLoad = 64 / kRowChunks;
    static constexpr int kLoads = kStep / kRowsPerLoad;
    static constexpr int RS = D + 4;
    static constexpr int kWaveBytes = kStep * 2 * RS * 4;
};

// 16 signed bytes -> 16 elements of the MFMA type, exactly.
template <bool kBf16>
__device__ __forceinline__ void widen_i8(uint4 raw, i16x8& lo, i16x8& hi) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t out[8];
    if (kBf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f0 = static_cast<float>(static_cast<int8_t>(w[i] & 0xffu));
            const float f1 = static_cast<float>(static_cast<int8_t>((w[i] >> 8) & 0xffu));
            const float f2 = static_cast<float>(static_cast<int8_t>((w[i] >> 16) & 0xffu));
            const float f3 = static_cast<float>(static_cast<int8_t>(w[i] >> 24));
            out[2 * i] = Mma<true>::pack_out(f0, f1);
            out[2 * i + 1] = Mma<true>::pack_out(f2, f3);
        }
    } else {
        // fp16 0x6400 | u is 1024 + u for a byte u; u = x + 128 (x ^ 0x80),
        // then one packed subtract of 1152 gives x.  One byte permute builds
        // two such halves from bytes of u and the constant 0x64.
        const f16x2 bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = w[i] ^ 0x80808080u;
            const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);   // bytes 0, 1
            const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);   // bytes 2, 3
            out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) - bias);
            out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, b) - bias);
        }
    }
    lo = __builtin_bit_cast(i16x8, (uint4){out[0], out[1], out[2], out[3]});
    hi = __builtin_bit_cast(i16x8, (uint4){out[4], out[5], out[6], out[7]});
}

// 8 signed bytes -> 8 elements of the MFMA type, exactly (as widen_i8).
template <bool kBf16>
__device__ __forceinline__ i16x8 widen8_i8(uint2 raw) {
    i16x8 lo, hi;
    widen_i8<kBf16>(make_uint4(raw.x, raw.y, 0u, 0u), lo, hi);
    return lo;
}

// Partial record of one (slot, head): [m, l, -, -, acc[0..D)], floats.
__host__ __device__ constexpr int rec_stride(int D) { return D + 4; }

// A value every lane holds alike, moved to scalar registers.  The entry
// index, lengths and step counts below are wave-uniform, but the compiler
// cannot tell for values loaded from memory or summed across lanes; without
// this, every K/V load built from them is wrapped in a per-lane loop over
// buffer descriptors.
__device__ __forceinline__ int32_t uniform32(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Live keys of batch entry b: [lo, lo + n).  The one query row is i = 0.
// kUniform: b is the same in every active lane (the loaded values go to
// scalar registers); otherwise each lane asks for its own entry.
struct LiveRange {
    int64_t lo, n;
};
template <bool kUniform>
__device__ __forceinline__ LiveRange live_range_t(const Params& p, int b) {
    int64_t kv = p.Lk;
    if (p.lens) {
        const int64_t L = kUniform ? uniform32(p.lens[b]) : p.lens[b];
        kv = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    int64_t hi = kv, lo = 0;
    if (p.causal) {
        const int64_t delta = causal_delta(p, kv);
        const int64_t bb = delta + 1;
        hi = bb < 0 ? 0 : (bb < kv ? bb : kv);
        lo = window_lo(p, 0, delta);
    }
    if (p.doc_start) {               // the row's document start (q_len == 1)
        const int64_t d = kUniform ? uniform32(p.doc_start[b]) : p.doc_start[b];
        lo = d > lo ? d : lo;
    }
    return {lo < hi ? lo : hi, lo < hi ? hi - lo : 0};
}

__device__ __forceinline__ LiveRange live_range(const Params& p, int b) {   // b wave-uniform
    return live_range_t<true>(p, b);
}

__device__ __forceinline__ int64_t steps_of(const Params& p, int b) {        // b wave-uniform
    return (live_range_t<true>(p, b).n + kStep - 1) / kStep;
}
__device__ __forceinline__ int64_t steps_of_lane(const Params& p, int b) {   // b per lane
    return (live_range_t<false>(p, b).n + kStep - 1) / kStep;
}

// Steps before batch entry b (all kv heads and slices of entries < b), summed
// in a fixed order by one wave (lanes take batch entries, then a butterfly).
__device__ int64_t steps_before(const Params& p, int b, int per_b_units) {
    const int lane = threadIdx.x & 63;
    int64_t total = 0;
    for (int b0 = 0; b0 < b; b0 += 64) {
        const int bb = b0 + lane;
        int64_t v = (bb < b) ? steps_of_lane(p, bb) : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
        total += v;
    }
    return uniform64(total * per_b_units);
}

// Waves that share S steps: every wave gets at least one.
__device__ __forceinline__ int64_t share_waves(int64_t S, int DP, bool i8) {
    return S < waves_total(DP, i8) ? S : waves_total(DP, i8);
}

// Wave that owns flattened step x when S steps are cut into W equal shares
// (share w = [floor(S*w/W), floor(S*(w+1)/W))).
__device__ __forceinline__ int owner_wave(int64_t x, int64_t S, int64_t W) {
    return static_cast<int>(((x + 1) * W - 1) / S);
}

// LDS bytes per wave of the unit mode: its staging rows, later its records
// (16 heads x rec_stride floats).
template <int D, bool kI8, bool kF32 = false>
__host__ __device__ constexpr int unit_wave_bytes() {
    constexpr int stage =
        kF32 ? F32Lay<D>::kWaveBytes : (kI8 ? I8Lay<D>::kWaveBytes : DLay<D>::kWaveBytes);
    constexpr int recs = 16 * rec_stride(D) * 4;
    return stage > recs ? stage : recs;
}

// The decode step loop of one wave.  Split mode (kUnit false): the wave is a
// workgroup of its own and takes an equal share of all units' steps, writing
// one record per unit it touches to the workspace.  Unit mode: a workgroup
// takes one whole unit, its waves equal contiguous shares of that unit's
// steps, and the workgroup folds its waves' records in LDS (wave order = key
// order) and writes the outputs itself, with no workspace and no merge
// kernel.  smem: this workgroup's LDS (one wave's rows in split mode, one
// unit_wave_bytes() slice per wave in unit mode).
// kF32: fp32 Q/K/V (kBf16 unused), on 16x16x4 fp32 matrix operations: the
// scores' d-sum runs lane group q4 over columns (D/4) q4 .. + D/4 - 1 (each
// lane's K and Q pieces contiguous), and output row i of d-tile dt is column
// (D/16) i + dt (each lane's V piece contiguous); P is not rounded.
template <bool kBf16, int D, bool kCap, bool kI8, bool kUnit, bool kF32 = false>
__device__ __forceinline__ void decode_body(const Params& p, int n_hgrp, int slot_heads,
                                            uint8_t* smem_base) {
    using M = Mma<kBf16>;
    using LY = DLay<D>;
    constexpr int KS = LY::KS, VS = LY::VS;
    constexpr int NT = D / 32;       // 32-wide d-steps of the score product
    constexpr int ND = D / 16;       // 16-row d-tiles of the output
    using L8 = I8Lay<D>;
    using FL = F32Lay<D>;
    static_assert(!kF32 || (!kI8 && D <= 128), "fp32 rows: no int8, head dims up to 128");

    const int lane = kUnit ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
    const int wave = kUnit ? uniform32(threadIdx.x >> 6) : blockIdx.x;
    uint8_t* const smem = smem_base + (kUnit ? wave * unit_wave_bytes<D, kI8, kF32>() : 0);
    uint16_t* const k_sh = reinterpret_cast<uint16_t*>(smem);
    uint16_t* const v_sh = k_sh + kStep * KS;
    uint8_t* const k8 = smem;                         // int8 cache: rows of L8::RS bytes
    uint8_t* const v8 = smem + kStep * L8::RS;
    float* const kf = reinterpret_cast<float*>(smem);     // fp32 rows of FL::RS floats
    float* const vf = kf + kStep * FL::RS;
    const int Dt = p.D;              // true head dim (<= D, the padded one)
    const int per_b = p.Hkv * n_hgrp;            // units per batch entry

    int b = 0;
    int64_t sb = 0;                              // steps of each unit of entry b
    int uu = 0;                                  // unit within the entry
    int64_t ls = 0;                              // step within the unit
    int64_t a = 0, e = 0;                        // this wave's steps, flattened
    if constexpr (kUnit) {
        const int nw = uniform32(blockDim.x >> 6);
        b = static_cast<int>(blockIdx.x / per_b);
        uu = static_cast<int>(blockIdx.x % per_b);
        sb = steps_of(p, b);
        ls = sb * wave / nw;
        e = sb * (wave + 1) / nw - ls;           // may be 0: the wave still joins the fold
    } else {
        const int64_t S = steps_before(p, p.B, per_b);
        const int64_t W = share_waves(S, D, kI8);
        if (wave >= W) return;
        a = S * wave / W;
        e = S * (wave + 1) / W;
        if (a >= e) return;

        // Locate the unit holding step a: 64 entries per round, one per lane;
        // an inclusive prefix sum over the lanes finds the first entry whose
        // steps end past a (a < S, so some round finds it).
        int64_t base_b = 0;                      // first step of entry b
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int bb = b0 + lane;
            const int64_t st = bb < p.B ? steps_of_lane(p, bb) : 0;
            int64_t incl = st * per_b;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            const uint64_t hit = __builtin_amdgcn_ballot_w64(base_b + incl > a);
            if (hit) {
                const int l = __builtin_ctzll(hit);
                b = b0 + l;
                sb = uniform64(__shfl(st, l, 64));
                base_b = uniform64(base_b + __shfl(incl, l, 64) - sb * per_b);
                break;
            }
            base_b = uniform64(base_b + __shfl(incl, 63, 64));
        }
        // The scan and steps_before count the same steps, so an entry is always
        // found; a wave that found none (sb == 0) has nothing to do.
        if (sb <= 0) return;
        uu = static_cast<int>((a - base_b) / sb);
        ls = (a - base_b) % sb;
    }

    const int col = lane & 15, q4 = lane >> 4;
    const int ld_row = kF32 ? lane / FL::kRowChunks : (kI8 ? lane / L8::kRowChunks : lane / LY::kRowChunks);
    const int ld_col = kF32 ? (lane % FL::kRowChunks) * 4
                            : (kI8 ? (lane % L8::kRowChunks) * 16 : (lane % LY::kRowChunks) * 8);
    // Raw scores are q.k with the K integers; a per-tensor K scale joins c.
    // With a mask the scores are natural: sc = scale (times that K scale)
    // maps raw to natural, and c = log2(e).
    const float kscale = (kI8 && p.k_quant == 1) ? p.k_scale[0] : 1.f;
    const bool k_chan = kI8 && p.k_quant == 2;
    const bool nat = p.mask != nullptr;
    const float sc = p.scale * kscale;
    const float c = nat ? kLog2e : p.scale_log2 * kscale;
    const float slack = kSlack / c;
    const float cap_k2 = kCap ? 2.f * kLog2e * p.scale * kscale / p.softcap : 0.f;
    const float cap_back = kCap ? p.softcap / (p.scale * kscale) : 0.f;

    // Per-unit state (wave-uniform: b, uu, live range; per-lane: the head).
    int h = 0;
    bool live_col = false;
    int64_t kv_lo = 0, kv_hi = 0;   // kv_hi: live keys counted from kv_lo
    i16x8 qop[NT];
    float qf[kF32 ? D / 4 : 1];      // fp32: Q columns (D/4) q4 .. + D/4 - 1 of head col
    const float* mrow = nullptr;
    float m_ref = kNegInf, l_sum = 0.f;
    f32x4 acc[ND];

    auto begin_unit = [&]() {
        const int g = uu / n_hgrp;
        const int hbase = (uu % n_hgrp) * 16;
        live_col = hbase + col < p.group;
        h = g * p.group + (live_col ? hbase + col : 0);
        const LiveRange lr = live_range(p, b);
        kv_lo = lr.lo;
        kv_hi = lr.n;
        if constexpr (kF32) {
            // Whole 16-byte chunks (the true head dim is a multiple of 4):
            // columns past it are zero, loaded unconditionally from the row's
            // first chunk and replaced.
            const float* srcf = static_cast<const float*>(p.q) + b * p.qs.sb + h * p.qs.sh;
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
                const int c0 = (D / 4) * q4 + 4 * m;
                const bool cin = live_col && c0 < Dt;
                const f32x4 raw = *reinterpret_cast<const f32x4*>(srcf + (c0 < Dt ? c0 : 0));
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) qf[4 * m + e2] = cin ? raw[e2] : 0.f;
            }
        }
        const uint16_t* src = static_cast<const uint16_t*>(p.q) + b * p.qs.sb + h * p.qs.sh + 8 * q4;
#pragma unroll
        for (int t = 0; t < (kF32 ? 0 : NT); ++t) {
            // Columns past the true head dim (a multiple of 8) are zero: the
            // load is unconditional (from the row's first chunk there) and
            // its value replaced, so no load waits behind a branch.
            const bool cin = 32 * t + 8 * q4 < Dt;
            const i16x8 raw = *reinterpret_cast<const i16x8*>(src + (cin ? 32 * t : -8 * q4));
            i16x8 v = cin ? raw : i16x8{};
            if (k_chan && cin) {   // q_d * k_scale[g, d], rounded to the element type
                const float* ks = p.k_scale + g * Dt + 32 * t + 8 * q4;
                const uint4 u = __builtin_bit_cast(uint4, v);
                const uint32_t in[4] = {u.x, u.y, u.z, u.w};
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // Elements 2e (low half) and 2e + 1 (high half) of the word.
                    const uint16_t b0 = static_cast<uint16_t>(in[e] & 0xffffu);
                    const uint16_t b1 = static_cast<uint16_t>(in[e] >> 16);
                    float x0, x1;
                    if (kBf16) {
                        x0 = __uint_as_float(static_cast<uint32_t>(b0) << 16);
                        x1 = __uint_as_float(static_cast<uint32_t>(b1) << 16);
                    } else {
                        x0 = static_cast<float>(__builtin_bit_cast(_Float16, b0));
                        x1 = static_cast<float>(__builtin_bit_cast(_Float16, b1));
                    }
                    w[e] = M::pack_out(x0 * ks[2 * e], x1 * ks[2 * e + 1]);
                }
                v = __builtin_bit_cast(i16x8, (uint4){w[0], w[1], w[2], w[3]});
            }
            qop[t] = live_col ? v : i16x8{};
        }
        mrow = (p.mask && live_col) ? p.mask + b * p.ms.sb + h * p.ms.sh + kv_lo : nullptr;
        m_ref = kNegInf;
        l_sum = 0.f;
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[d] = f32x4{};
    };
    // This lane's accumulators into record rec (acc[0..D) at rec + 4).
    auto store_acc = [&](float* rec) {
        if constexpr (kF32) {
            // acc[dt][r] holds column (D/16) (4 q4 + r) + dt.
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m = 0; m < D / 64; ++m)
                    *reinterpret_cast<f32x4*>(rec + 4 + (D / 16) * (4 * q4 + r) + 4 * m) =
                        f32x4{acc[4 * m][r], acc[4 * m + 1][r], acc[4 * m + 2][r], acc[4 * m + 3][r]};
        } else {
#pragma unroll
            for (int d = 0; d < ND; ++d)
                *reinterpret_cast<f32x4*>(rec + 4 + 16 * d + 4 * q4) = acc[d];
        }
    };
    auto end_unit = [&]() {
        // Column total of the running sum: the 4 lanes of column col, fixed order.
        float lt = l_sum + __shfl_xor(l_sum, 16, 64);
        lt = lt + __shfl_xor(lt, 32, 64);
        if (live_col) {
            const int64_t unit = static_cast<int64_t>(b) * per_b + uu;
            float* rec = static_cast<float*>(p.ws) + ((unit + wave) * slot_heads + col) * rec_stride(D);
            store_acc(rec);
            if (q4 == 0) {
                rec[0] = m_ref;
                rec[1] = lt;
            }
        }
    };

    // Prefetch of one step, given the (entry, unit, step-in-unit) of that step.
    constexpr int kEs = kF32 ? 4 : (kI8 ? 1 : 2);             // cache bytes per element
    constexpr int kLd = kF32 ? FL::kLoads : (kI8 ? L8::kLoads : LY::kLoads);
    constexpr int kRpl = kF32 ? FL::kRowsPerLoad : (kI8 ? L8::kRowsPerLoad : LY::kRowsPerLoad);
    i16x8 kst[kLd], vst[kLd];
    auto fetch = [&](int fb, int fuu, int64_t fls) {
        const int fg = fuu / n_hgrp;
        const LiveRange lr = live_range(p, fb);
        const uint8_t* kg = static_cast<const uint8_t*>(p.k) +
                            (fb * p.ks.sb + fg * p.ks.sh + lr.lo * p.ks.sr) * kEs;
        const uint8_t* vg = static_cast<const uint8_t*>(p.v) +
                            (fb * p.vs.sb + fg * p.vs.sh + lr.lo * p.vs.sr) * kEs;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, lr.n * p.ks.sr * kEs);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, lr.n * p.vs.sr * kEs);
        const int j0 = static_cast<int>(fls) * kStep + ld_row;
        // Padded columns load as zeros: their lanes' offsets start 2^31 bytes
        // past any row (one select per step, so every load stays one
        // unconditional instruction).
        const uint32_t col_off = ld_col < Dt ? static_cast<uint32_t>(ld_col * kEs) : 0x80000000u;
#pragma unroll
        for (int n = 0; n < kLd; ++n) {
            const int key = j0 + n * kRpl;
            kst[n] = load16_stream(krs, static_cast<int>(static_cast<uint32_t>(key * static_cast<int>(p.ks.sr) * kEs) + col_off));
            vst[n] = load16_stream(vrs, static_cast<int>(static_cast<uint32_t>(key * static_cast<int>(p.vs.sr) * kEs) + col_off));
        }
    };

    begin_unit();
    if (!kUnit || a < e) fetch(b, uu, ls);
    for (int64_t x = a; x < e; ++x) {
        // Cursor of step x + 1 (next unit, skipping entries with no live key).
        int nb = b, nuu = uu;
        int64_t nls = ls + 1;
        if (!kUnit && nls == sb) {
            nls = 0;
            if (++nuu == per_b) {
                nuu = 0;
                do {
                    ++nb;
                } while (nb < p.B && steps_of(p, nb) == 0);
            }
        }
        // The previous step's LDS reads precede these writes in this wave's
        // in-order LDS queue, so one buffer suffices.
#pragma unroll
        for (int n = 0; n < kLd; ++n) {
            const int row = n * kRpl + ld_row;
            if (kF32) {
                *reinterpret_cast<i16x8*>(&kf[row * FL::RS + ld_col]) = kst[n];
                *reinterpret_cast<i16x8*>(&vf[row * FL::RS + ld_col]) = vst[n];
            } else if (kI8) {
                *reinterpret_cast<i16x8*>(&k8[row * L8::RS + ld_col]) = kst[n];
                *reinterpret_cast<i16x8*>(&v8[row * L8::RS + ld_col]) = vst[n];
            } else {
                *reinterpret_cast<i16x8*>(&k_sh[row * KS + ld_col]) = kst[n];
                *reinterpret_cast<i16x8*>(&v_sh[row * VS + ld_col]) = vst[n];
            }
        }
        if (x + 1 < e) fetch(nb, nuu, nls);
        const int64_t j0 = ls * kStep;

        // S^T = K Q^T: two 16-key blocks; lane holds keys key_at(kb, r) of column col.
        // fp16/bf16 rows: block kb holds keys kb*16 + 4*q4 + r.  Int8 rows: the
        // A operand's row m of block kb is key 8*(m/4) + 4*kb + m%4, so that
        // lane q4 ends up with the eight consecutive keys 8*q4 + 4*kb + r,
        // which the transposing 8-bit V read delivers as one operand.
        auto key_at = [&](int kb, int r) { return kI8 ? 8 * q4 + 4 * kb + r : 16 * kb + 4 * q4 + r; };
        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{};
            if constexpr (kF32) {
                // Operation t: A[col][q4] = K[16 kb + col][(D/4) q4 + t],
                // B[q4][col] = Q[head col][(D/4) q4 + t].
                const float* krow = &kf[(kb * 16 + col) * FL::RS + (D / 4) * q4];
#pragma unroll
                for (int m = 0; m < D / 16; ++m) {
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 4 * m);
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e2], qf[4 * m + e2], s[kb], 0, 0, 0);
                }
            } else if constexpr (kI8) {
                const uint8_t* krow = &k8[(8 * (col >> 2) + 4 * kb + (col & 3)) * L8::RS + 8 * q4];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    s[kb] = M::mfma16(widen8_i8<kBf16>(*reinterpret_cast<const uint2*>(krow + 32 * t)),
                                      qop[t], s[kb]);
            } else {
                const uint16_t* krow = &k_sh[(kb * 16 + col) * KS + 8 * q4];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    s[kb] = M::mfma16(*reinterpret_cast<const i16x8*>(krow + 32 * t), qop[t], s[kb]);
            }
        }
        if (kCap) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kb][r] = softcap_raw(s[kb][r], cap_k2, cap_back);
        }
        if (mrow) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int64_t key0 = j0 + key_at(kb, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[kb][r] = (key0 + r < kv_hi) ? fmaf(s[kb][r], sc, mrow[key0 + r])
                                                  : s[kb][r] * sc;
            }
        }
        if (j0 + kStep > kv_hi) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (j0 + key_at(kb, r) >= kv_hi) s[kb][r] = kNegInf;
        }
        // Row maximum over the 4 lanes that share column col.
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool raise = mx > m_ref + slack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mx : m_ref;
            const float alpha = raise ? fast_exp2((m_ref - m_new) * c) : 1.f;   // 0 when m_ref = -inf
            l_sum *= alpha;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[d][r] *= alpha;
            m_ref = m_new;
        }
        // exp2(s*c - m*c), or exp2((s - m)*c) with a mask: a reference far
        // from zero (a large finite mask value) can neither overflow the
        // product nor round away the scores' differences.
        const float neg_mc = (m_ref == kNegInf || nat) ? 0.f : -m_ref * c;
        const float sub = (m_ref == kNegInf || !nat) ? 0.f : m_ref;
        // P^T operand (16x16x32 B layout): k = 8*q4 + e <-> key key_at(e / 4, e % 4)
        // (fp16/bf16 rows: e < 4 ? 4*q4 + e : 16 + 4*q4 + e - 4; int8 rows: 8*q4 + e).
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        float pf[2][4];                  // fp32 rows: p of key key_at(kb, r), not rounded
        if constexpr (kF32) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pf[kb][r] = fast_exp2(fmaf(s[kb][r] - sub, c, neg_mc));
                    l_sum += pf[kb][r];
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    w4[2 * kb + e2] = M::pack_out(fast_exp2(fmaf(s[kb][2 * e2] - sub, c, neg_mc)),
                                                  fast_exp2(fmaf(s[kb][2 * e2 + 1] - sub, c, neg_mc)));
                    l_sum = M::sum2(w4[2 * kb + e2], l_sum);
                }
            }
        }
        const i16x8 pop = __builtin_bit_cast(i16x8, (uint4){w4[0], w4[1], w4[2], w4[3]});
        // O^T += V^T P^T.  fp16/bf16 rows: V^T from the 16-bit transpose read,
        // rows 4*q4 + i/4 (+16), cols 16*dt + 4*(i%4).  Int8 rows: one 8-bit
        // transpose read per d-tile: lane 2k + h of each 16-lane group points
        // at row 8*q4 + k, bytes 16*dt + 8*h .. + 7, and lane 8*h + i receives
        // byte i of those eight rows, i.e. column 16*dt + (lane % 16) of keys
        // 8*q4 .. 8*q4 + 7, the P^T operand's keys.
        const int gi = lane & 15;
        if constexpr (kF32) {
            // Operation (kb, u): A[col][q4] = V[16 kb + 4 q4 + u][(D/16) col + dt],
            // B[q4][col] = p of key 16 kb + 4 q4 + u (this lane's score r = u).
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float* vrow = &vf[(16 * kb + 4 * q4 + u) * FL::RS + (D / 16) * col];
#pragma unroll
                    for (int m = 0; m < D / 64; ++m) {
                        const f32x4 vv = *reinterpret_cast<const f32x4*>(vrow + 4 * m);
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2)
                            acc[4 * m + e2] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                vv[e2], pf[kb][u], acc[4 * m + e2], 0, 0, 0);
                    }
                }
        } else if constexpr (kI8) {
            const uint8_t* vr = &v8[(8 * q4 + (gi >> 1)) * L8::RS + 8 * (gi & 1)];
#pragma unroll
            for (int d = 0; d < ND; ++d)
                acc[d] = M::mfma16(widen8_i8<kBf16>(tr_read8(vr + 16 * d)), pop, acc[d]);
        } else {
            const uint16_t* v0 = &v_sh[(4 * q4 + (gi >> 2)) * VS + 4 * (gi & 3)];
            const uint16_t* v1 = v0 + 16 * VS;
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const i16x4 lo = tr_read(v0 + 16 * d);
                const i16x4 hi = tr_read(v1 + 16 * d);
                const i16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[d] = M::mfma16(av, pop, acc[d]);
            }
        }

        if (!kUnit && (nb != b || nuu != uu || x + 1 == e)) {
            end_unit();
            if (x + 1 < e) {
                b = nb;
                uu = nuu;
                sb = steps_of(p, b);
                begin_unit();
            }
        }
        ls = nls;
    }
    if constexpr (kUnit) {
        // Column totals of the running sums, as end_unit.
        float lt = l_sum + __shfl_xor(l_sum, 16, 64);
        lt = lt + __shfl_xor(lt, 32, 64);
        __syncthreads();             // every wave is done with its staging rows
        constexpr int RS = rec_stride(D);
        float* const recs = reinterpret_cast<float*>(smem_base);   // [wave][16 heads][RS]
        float* const rec = recs + (wave * 16 + col) * RS;
        store_acc(rec);
        if (q4 == 0) {
            rec[0] = m_ref;
            rec[1] = lt;
        }
        __syncthreads();
        // Fold the waves' records in wave order (= key order), then the sink,
        // the empty-row policy and the LSE, as the merge kernel does; items
        // (head, d) with d fastest, so the stores are contiguous.
        using T = std::conditional_t<kF32, float, std::conditional_t<kBf16, bf16_t, _Float16>>;
        const int nw = uniform32(blockDim.x >> 6);
        const int g = uu / n_hgrp, hbase = (uu % n_hgrp) * 16;
        const int nh = p.group - hbase < 16 ? p.group - hbase : 16;
        const float ksc = (kI8 && p.k_quant == 1) ? p.k_scale[0] : 1.f;
        const float cr = p.mask ? kLog2e : p.scale_log2 * ksc;
        const float to_nat = p.mask ? 1.f : p.scale * ksc;
        for (int it = threadIdx.x; it < nh * Dt; it += blockDim.x) {
            const int hc = it / Dt, d = it - hc * Dt;
            float Mx = kNegInf;
            for (int w = 0; w < nw; ++w) Mx = fmaxf(Mx, recs[(w * 16 + hc) * RS]);
            float L = 0.f, A = 0.f;
            for (int w = 0; w < nw; ++w) {
                const float* r = recs + (w * 16 + hc) * RS;
                const float f = (r[0] == kNegInf) ? 0.f : fast_exp2((r[0] - Mx) * cr);
                L = fmaf(r[1], f, L);
                A = fmaf(r[4 + d], f, A);
            }
            const int h = g * p.group + hbase + hc;
            float m_nat = Mx * to_nat;
            const float fs = fold_sink(p, h, m_nat, L);
            const bool empty = (L == 0.f);
            const float inv = fs / L;
            const float vsc = !kI8 ? 1.f : (p.v_quant == 1 ? p.v_scale[0] : p.v_scale[g * Dt + d]);
            const float o = empty ? (p.masked_zero ? 0.f : __builtin_nanf("")) : A * vsc * inv;
            Elem<T>::store(p.o, b * p.os.sb + h * p.os.sh + d, o);
            if (p.lse && d == 0)
                p.lse[b * p.ls.sb + h * p.ls.sh] = empty ? kNegInf : row_lse(m_nat, L);
        }
    }
}

template <bool kBf16, int D, bool kCap, bool kI8, bool kF32 = false>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(Params p, int n_hgrp, int slot_heads) {
    __shared__ __attribute__((aligned(16))) uint8_t
        smem[kF32 ? F32Lay<D>::kWaveBytes : (kI8 ? I8Lay<D>::kWaveBytes : DLay<D>::kWaveBytes)];
    decode_body<kBf16, D, kCap, kI8, false, kF32>(p, n_hgrp, slot_heads, smem);
}

// One workgroup per unit; nw = blockDim.x / 64 waves, nw * unit_wave_bytes()
// bytes of dynamic LDS.
template <bool kBf16, int D, bool kCap, bool kI8, bool kF32 = false>
__global__ __launch_bounds__(64 * unit_waves_max(D, kI8, kF32)) void decode_unit_kernel(Params p, int n_hgrp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsmem[];
    decode_body<kBf16, D, kCap, kI8, true, kF32>(p, n_hgrp, 0, dsmem);
}

// One wave per (b, h): merge the records of the waves that covered its unit,
// in wave order (= key order).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(Params p, int n_hgrp, int slot_heads) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (bh >= static_cast<int64_t>(p.B) * p.Hq) return;
    const int b = static_cast<int>(bh / p.Hq), h = static_cast<int>(bh % p.Hq);
    const int per_b = p.Hkv * n_hgrp;
    const int g = h / p.group, hin = h % p.group;
    const int uu = g * n_hgrp + hin / 16, col = hin % 16;
    const int64_t S = steps_before(p, p.B, per_b);
    const int64_t sb = steps_of(p, b);
    const int64_t unit = static_cast<int64_t>(b) * per_b + uu;
    const int64_t first = steps_before(p, b, per_b) + uu * sb;   // first step of the unit
    constexpr int NPL = (D + 63) / 64;
    // Records are in the split kernel's score units: raw (a per-tensor int8
    // K scale joins c and to_nat), or natural with a mask.
    const float ksc = (p.kv_int8 && p.k_quant == 1) ? p.k_scale[0] : 1.f;
    const float c = p.mask ? kLog2e : p.scale_log2 * ksc;
    const float to_nat = p.mask ? 1.f : p.scale * ksc;
    float M = kNegInf, L = 0.f, A[NPL];
#pragma unroll
    for (int cc = 0; cc < NPL; ++cc) A[cc] = 0.f;
    if (sb > 0) {
        const int64_t W = share_waves(S, D, p.kv_int8 != 0);
        const int w_lo = owner_wave(first, S, W), w_hi = owner_wave(first + sb - 1, S, W);
        const int n = w_hi - w_lo + 1;
        const int rs = rec_stride(D);
        const float* base = static_cast<const float*>(p.ws);
        auto rec = [&](int w) { return base + ((unit + w) * slot_heads + col) * rs; };
        // A wave with an empty share wrote no record (none while W <= S).
        auto empty_share = [&](int w) { return S * w / W == S * (w + 1) / W; };
        // Record headers are fetched one per lane (64 at a time), so the
        // loads overlap instead of forming a chain; the first 64 headers and
        // the first eight records' rows are fetched together, since their
        // addresses do not depend on the headers' values.
        float mh = kNegInf, lh = 0.f;            // header of record w_lo + lane
        float v0[8][NPL];
        {
            const int w = w_lo + lane;
            if (lane < n && !empty_share(w)) {
                const float* r = rec(w);
                mh = r[0];
                lh = r[1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int cc = 0; cc < NPL; ++cc) {
                    const int d = lane + 64 * cc;
                    v0[u][cc] = (u < n && d < D) ? rec(w_lo + u)[4 + d] : 0.f;
                }
        }
        M = mh;
        for (int c0 = 64; c0 < n; c0 += 64) {
            const int w = w_lo + c0 + lane;
            if (c0 + lane < n && !empty_share(w)) M = fmaxf(M, rec(w)[0]);
        }
        M = wave_max(M);
        for (int c0 = 0; c0 < n; c0 += 64) {
            float f = 0.f, l = 0.f;
            if (c0 == 0) {
                f = (mh == kNegInf) ? 0.f : fast_exp2((mh - M) * c);
                l = lh;
            } else {
                const int w = w_lo + c0 + lane;
                if (c0 + lane < n && !empty_share(w)) {
                    const float* r = rec(w);
                    f = (r[0] == kNegInf) ? 0.f : fast_exp2((r[0] - M) * c);
                    l = r[1];
                }
            }
            const int cnt = n - c0 < 64 ? n - c0 : 64;
            // Accumulators: 8 records' rows loaded ahead, folded in wave order.
            for (int i0 = 0; i0 < cnt; i0 += 8) {
                float v[8][NPL];
                if (c0 == 0 && i0 == 0) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
#pragma unroll
                        for (int cc = 0; cc < NPL; ++cc) v[u][cc] = v0[u][cc];
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
#pragma unroll
                        for (int cc = 0; cc < NPL; ++cc) {
                            const int d = lane + 64 * cc;
                            v[u][cc] = (i0 + u < cnt && d < D) ? rec(w_lo + c0 + i0 + u)[4 + d]
                                                               : 0.f;
                        }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u;
                    if (i < cnt && !empty_share(w_lo + c0 + i)) {
                        const float fi = __shfl(f, i, 64), li = __shfl(l, i, 64);
                        L = fmaf(li, fi, L);
#pragma unroll
                        for (int cc = 0; cc < NPL; ++cc) A[cc] = fmaf(v[u][cc], fi, A[cc]);
                    }
                }
            }
        }
    }
    float m_nat = M * to_nat;                    // natural units (-inf stays -inf)
    const float fs = fold_sink(p, h, m_nat, L);
    const bool empty = (L == 0.f);
    const float inv = fs / L;
    const int64_t orow = b * p.os.sb + h * p.os.sh;
#pragma unroll
    for (int cc = 0; cc < NPL; ++cc) {
        const int d = lane + 64 * cc;
        if (d < p.D) {   // columns past the true head dim are padding
            // An int8 V scale factors out of the sum over keys.
            const float vsc = !p.kv_int8 ? 1.f : (p.v_quant == 1 ? p.v_scale[0] : p.v_scale[g * p.D + d]);
            const float o = empty ? (p.masked_zero ? 0.f : __builtin_nanf("")) : A[cc] * vsc * inv;
            Elem<T>::store(p.o, orow + d, o);
        }
    }
    if (p.lse && lane == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh] = empty ? kNegInf : row_lse(m_nat, L);
}

int slice_count(int group) { return (group + 15) / 16; }
int heads_per_slot(int group) { return group < 16 ? group : 16; }

// Steps of the longest possible unit: the cache capacity bounds the live
// keys, and so does a causal local window (the one row sees at most W keys).
int64_t max_unit_steps(const Params& p) {
    int64_t keys = p.Lk;
    if (p.causal && p.window > 0 && p.window < keys) keys = p.window;
    return (keys + kStep - 1) / kStep;
}

// Waves per workgroup of the unit mode: one per step of the longest
// possible unit, at most unit_waves_max.
int unit_waves(const Params& p, int DP, bool f32) {
    const int64_t smax = max_unit_steps(p);
    const int cap = unit_waves_max(DP, p.kv_int8 != 0, f32);
    return smax < cap ? static_cast<int>(smax < 1 ? 1 : smax) : cap;
}

template <bool kBf16, int D>
hipError_t launch_unit(const Params& p, hipStream_t s) {
    const int n_hgrp = slice_count(p.group);
    const int nw = unit_waves(p, D, false);
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(p.B) * p.Hkv * n_hgrp)), blk(64 * nw);
    const bool cap = p.softcap > 0.f;
    if (p.kv_int8) {
        const size_t lds = static_cast<size_t>(nw) * unit_wave_bytes<D, true>();
        if (cap)
            hipLaunchKernelGGL((decode_unit_kernel<kBf16, D, true, true>), g, blk, lds, s, p, n_hgrp);
        else
            hipLaunchKernelGGL((decode_unit_kernel<kBf16, D, false, true>), g, blk, lds, s, p, n_hgrp);
    } else {
        const size_t lds = static_cast<size_t>(nw) * unit_wave_bytes<D, false>();
        if (cap)
            hipLaunchKernelGGL((decode_unit_kernel<kBf16, D, true, false>), g, blk, lds, s, p, n_hgrp);
        else
            hipLaunchKernelGGL((decode_unit_kernel<kBf16, D, false, false>), g, blk, lds, s, p, n_hgrp);
    }
    return hipGetLastError();
}

template <bool kBf16, int D>
hipError_t launch_one(const Params& p, hipStream_t s, bool unit) {
    if (unit) return launch_unit<kBf16, D>(p, s);
    const int n_hgrp = slice_count(p.group), hs = heads_per_slot(p.group);
    const dim3 g(waves_total(D, p.kv_int8 != 0)), blk(64);
    const bool cap = p.softcap > 0.f;
    if (p.kv_int8 && cap)
        hipLaunchKernelGGL((decode_split_kernel<kBf16, D, true, true>), g, blk, 0, s, p, n_hgrp, hs);
    else if (p.kv_int8)
        hipLaunchKernelGGL((decode_split_kernel<kBf16, D, false, true>), g, blk, 0, s, p, n_hgrp, hs);
    else if (cap)
        hipLaunchKernelGGL((decode_split_kernel<kBf16, D, true, false>), g, blk, 0, s, p, n_hgrp, hs);
    else
        hipLaunchKernelGGL((decode_split_kernel<kBf16, D, false, false>), g, blk, 0, s, p, n_hgrp, hs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq;
    const dim3 cgrid(static_cast<uint32_t>((rows + 3) / 4));
    if (kBf16)
        hipLaunchKernelGGL((decode_combine_kernel<bf16_t, D>), cgrid, dim3(256), 0, s, p, n_hgrp, hs);
    else
        hipLaunchKernelGGL((decode_combine_kernel<_Float16, D>), cgrid, dim3(256), 0, s, p, n_hgrp, hs);
    return hipGetLastError();
}

// fp32 Q/K/V (head dims up to 128): the same two modes.
template <int D>
hipError_t launch_one_f32(const Params& p, hipStream_t s, bool unit) {
    const int n_hgrp = slice_count(p.group), hs = heads_per_slot(p.group);
    const bool cap = p.softcap > 0.f;
    if (unit) {
        const int nw = unit_waves(p, D, true);
        const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(p.B) * p.Hkv * n_hgrp)), blk(64 * nw);
        const size_t lds = static_cast<size_t>(nw) * unit_wave_bytes<D, false, true>();
        if (cap)
            hipLaunchKernelGGL((decode_unit_kernel<false, D, true, false, true>), g, blk, lds, s, p, n_hgrp);
        else
            hipLaunchKernelGGL((decode_unit_kernel<false, D, false, false, true>), g, blk, lds, s, p, n_hgrp);
        return hipGetLastError();
    }
    const dim3 g(waves_total(D, false)), blk(64);
    if (cap)
        hipLaunchKernelGGL((decode_split_kernel<false, D, true, false, true>), g, blk, 0, s, p, n_hgrp, hs);
    else
        hipLaunchKernelGGL((decode_split_kernel<false, D, false, false, true>), g, blk, 0, s, p, n_hgrp, hs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq;
    const dim3 cgrid(static_cast<uint32_t>((rows + 3) / 4));
    hipLaunchKernelGGL((decode_combine_kernel<float, D>), cgrid, dim3(256), 0, s, p, n_hgrp, hs);
    return hipGetLastError();
}

}  // namespace

// The kernel's head dim for a true head dim D: 64, 128 or 256, columns past
// D padded with zeros (loaded as zeros, never stored).
int decode_padded_dim(int D) { return D <= 64 ? 64 : (D <= 128 ? 128 : 256); }

// U + W - 1 record slots of min(G, 16) heads each (U = units, W = waves).
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D) {
    const int group = Hq / Hkv;
    const int64_t units = static_cast<int64_t>(B) * Hkv * slice_count(group);
    // Slots for the most waves any cache type uses at this shape.
    const int DP = decode_padded_dim(D);
    return static_cast<size_t>(units + kWavesMax) * heads_per_slot(group) * rec_stride(DP) *
           sizeof(float);
}

bool decode_split_supported(const Params& p, DType dt) {
    const bool f32 = dt == DType::F32;
    if (f32) {
        // fp32: head dims that are whole 16-byte chunks up to 128, run at 64
        // or 128.
        if (p.kv_int8 || p.D < 4 || p.D > 128 || p.D % 4 != 0) return false;
    } else {
        if (dt != DType::BF16 && dt != DType::F16) return false;
        // Head dims that are whole 16-byte chunks (whole 16-value chunks for
        // an int8 cache) up to 256, run at 64, 128 or 256.
        if (p.D < 8 || p.D > 256 || p.D % (p.kv_int8 ? 16 : 8) != 0) return false;
    }
    if (p.Lq != 1 || p.Lk == 0) return false;
    // Buffer offsets of one (b, kv head) slice are 32-bit, including the
    // up-to-one-step overrun past the live length.
    const int64_t es = f32 ? 4 : 2;                  // bytes per element (int8: at most)
    if (p.ks.sr >= (1 << 24) || p.vs.sr >= (1 << 24)) return false;
    if ((static_cast<int64_t>(p.Lk) + kStep) * p.ks.sr * es >= (int64_t(1) << 31) ||
        (static_cast<int64_t>(p.Lk) + kStep) * p.vs.sr * es >= (int64_t(1) << 31))
        return false;
    if (f32) {   // 16-byte loads of 4 floats
        auto al4 = [](const void* ptr, const Strides& st) {
            return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && st.sb % 4 == 0 &&
                   st.sh % 4 == 0 && st.sr % 4 == 0;
        };
        return al4(p.q, p.qs) && al4(p.k, p.ks) && al4(p.v, p.vs);
    }
    auto al = [](const void* ptr, const Strides& st, int a) {
        return reinterpret_cast<uintptr_t>(ptr) % (2 * a) == 0 && st.sb % a == 0 &&
               st.sh % a == 0 && st.sr % a == 0;
    };
    if (p.kv_int8) {   // 16-byte loads of 16 int8 values
        auto al8 = [](const void* ptr, const Strides& st) {
            return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && st.sb % 16 == 0 &&
                   st.sh % 16 == 0 && st.sr % 16 == 0;
        };
        return al(p.q, p.qs, 8) && al8(p.k, p.ks) && al8(p.v, p.vs);
    }
    return al(p.q, p.qs, 8) && al(p.k, p.ks, 8) && al(p.v, p.vs, 8);
}

// The unit mode saves the merge kernel and the records (about 10 us on small
// calls) but runs each unit on one workgroup, whose waves walk their steps
// one HBM round trip after another; the split mode spreads every unit over
// the whole GPU.  Measured crossovers (one MI355X, full-length caches): the
// unit mode wins up to 16 steps per wave at head dim 64 (64 entries of 8192
// keys, 8192 waves in two rounds: 103 us against 110 split), up to 8 at 128
// (16 when at most 256 waves run in all), 4 at 256 with 16-bit rows and 16
// with int8 rows, while its workgroups fit in about two rounds on the GPU
// (e.g. 64 entries of 2048 keys, or of a 2047-key window over 8192: 79 us
// against 88 split; 64 entries of 8192 keys at 128: 190 against 173).  fp32
// rows: up to 8 steps per wave at 64 (16 entries of 2048 keys: 29 against 32
// split), 4 at 128 (4 entries of 1024 keys: 36 against 26 split).
bool decode_unit_preferred(const Params& p, DType dt) {
    const int DP = decode_padded_dim(p.D);
    const bool i8 = p.kv_int8 != 0, f32 = dt == DType::F32;
    const int64_t smax = max_unit_steps(p);
    const int nw = unit_waves(p, DP, f32);
    const int64_t waves = static_cast<int64_t>(p.B) * p.Hkv * slice_count(p.group) * nw;
    const int64_t per_wave = (smax + nw - 1) / nw;
    if (DP == 64 && !i8 && !f32) return per_wave <= 16 && waves <= 8192;
    // fp32 rows: four waves per workgroup at 128, eight at 64.
    if (f32) return per_wave <= (DP == 128 ? 4 : 8) && waves <= 4096;
    const int64_t limit = i8 ? 16 : (DP == 256 ? 4 : (waves <= 256 ? 16 : 8));
    return per_wave <= limit && waves <= 4096;
}

hipError_t launch_decode_split(const Params& p, DType dt, hipStream_t s, bool unit) {
    const int DP = decode_padded_dim(p.D);
    if (dt == DType::F32)
        return DP == 64 ? launch_one_f32<64>(p, s, unit) : launch_one_f32<128>(p, s, unit);
    if (dt == DType::BF16)
        return DP == 64 ? launch_one<true, 64>(p, s, unit)
                        : (DP == 128 ? launch_one<true, 128>(p, s, unit)
                                     : launch_one<true, 256>(p, s, unit));
    return DP == 64 ? launch_one<false, 64>(p, s, unit)
                    : (DP == 128 ? launch_one<false, 128>(p, s, unit)
                                 : launch_one<false, 256>(p, s, unit));
}

}  // namespace sdpa
