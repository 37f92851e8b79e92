// prefill_f32.hip -- fused attention for float32 inputs on the vector FMA
// units, head dims 1..256 (padded to 32, 64, 96, 128 or 256; padded columns
// load as zeros and are not stored).
//
// A group of G neighbouring lanes (G = 4, or 8 at the 256 padding) owns a
// query row, each lane DP / G of its columns: a score is G partial dot
// products added by exchanges inside the group, so every lane of the group
// holds the same score and takes the same softmax decisions (OneGPU
// "Attention", "Variants and ordering": the `pairs` variant splits the head
// dimension over neighbouring threads and joins the parts with a shuffle).
// For paddings up to 64 each group owns two rows (16 apart), so every K/V
// value read from LDS feeds two FMAs: one read per FMA would leave the loop
// bound by LDS bandwidth.  Keys are folded in increasing order, 16 per tile (8
// at the 256 padding), from the wave's own LDS rows (coalesced loads, next
// tile prefetched into registers), with the online normaliser and a lazily
// raised reference max as in the matrix-core kernel; in float32 the
// probabilities are not rounded.
//
// Blockwise summation (OneGPU "Attention", "Accuracy at long key lengths"):
// each tile's products and probabilities are summed into zero-started
// partials, which are then added to the running accumulator and sum once, so
// a long row adds one value per tile to the running totals instead of one per
// key.
//
// Score-rule variants (ONNX GroupQueryAttention README, "Attributes",
// "Inputs") and document masks (llm.istanbul "05_attention", "Phase 0" and
// "K-block iteration") in the kVar kernel: each row's first visible key (local
// window, document start) bounds it from below and the tiles below the
// block's smallest bound are skipped; the softcap maps the raw score before
// the mask; the sink joins the denominator at the end.
//
// When the query blocks are too few to fill the GPU, the keys are cut into
// contiguous ranges (a multiple of 32 keys, at least 128, at most 16 ranges);
// each (rows, range) wave writes its partial (m, l, acc) and a second kernel
// merges the ranges of each row in range order (OneGPU "Attention", "Accuracy
// at long key lengths", last paragraph).  The cut depends only on the shape.
#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kRangeQuantum = 32;   // key ranges are multiples of this
constexpr float kSlack = 8.f;       // lazy-rescale threshold, base-2 units

// Layout per padded head dim DP: G lanes per row, R rows per lane group,
// T keys per tile.
template <int DP> struct F32Lay {
    static constexpr int G = DP == 256 ? 8 : 4;
    static constexpr int R = DP <= 64 ? 2 : 1;
    static constexpr int DQ = DP / G;                 // columns per lane
    static constexpr int kGroups = 64 / G;            // lane groups per wave
    static constexpr int RW = kGroups * R;            // rows per wave
    static constexpr int T = DP == 256 ? 8 : 16;      // keys per tile
    static constexpr int kRowF4 = DP / 4;             // float4 per padded row
    static constexpr int kLoads = T * kRowF4 / 64;    // float4 per lane per tensor
    static_assert(T * kRowF4 % 64 == 0, "tile loads must cover the wave");
    static_assert(DQ % 4 == 0, "a lane's columns are whole float4");
};

// Sum over the G lanes of a group: every step adds the same two numbers on
// each partner, so all lanes end with identical bits.
template <int G> __device__ __forceinline__ float group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // ^1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // ^2
    if constexpr (G == 8) x += __shfl_xor(x, 4, 64);
    return x;
}

template <int DP, bool kMask, bool kSplit, bool kVar>
__global__ __launch_bounds__(64) void prefill_f32_kernel(Params p, int n_rblk, int vec) {
    using LY = F32Lay<DP>;
    constexpr int G = LY::G, R = LY::R, DQ = LY::DQ, RW = LY::RW, kTile = LY::T;
    __shared__ __attribute__((aligned(16))) float k_sh[kTile * DP];
    __shared__ __attribute__((aligned(16))) float v_sh[kTile * DP];

    // blockIdx.x: row block (heaviest causal blocks first); y: head; z: batch * ranges.
    const int rb = n_rblk - 1 - static_cast<int>(blockIdx.x);
    const int h = blockIdx.y;
    const int b = static_cast<int>(blockIdx.z) / p.n_split;
    const int rng = static_cast<int>(blockIdx.z) % p.n_split;
    const int g = h / p.group;
    const int lane = threadIdx.x;
    const int grp = lane / G, gl = lane % G;
    const int D = p.D;

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const int64_t delta = causal_delta(p, kv_len);

    // This lane's rows: rb * RW + kGroups r + grp, r < R; keys [row_lo, row_hi)
    // are visible to row r (before the mask).
    int64_t row[R], row_hi[R], row_lo[R];
    bool row_ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = static_cast<int64_t>(rb) * RW + LY::kGroups * r + grp;
        row_ok[r] = row[r] < p.Lq;
        int64_t hi = kv_len;
        if (p.causal) {
            const int64_t bb = row[r] + delta + 1;   // keys j <= i + delta
            hi = bb < hi ? bb : hi;
        }
        row_hi[r] = row_ok[r] ? hi : 0;
        row_lo[r] = (kVar && row_ok[r]) ? first_key(p, b, row[r], delta) : 0;
    }
    // Keys the block can see: [blk_lo, blk_hi); this range of them.
    int64_t blk_hi = 0, blk_lo = INT64_MAX;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (!row_ok[r]) continue;
        blk_hi = row_hi[r] > blk_hi ? row_hi[r] : blk_hi;
        blk_lo = row_lo[r] < blk_lo ? row_lo[r] : blk_lo;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {   // wave-wide max / min
        const int64_t oh = __shfl_xor(blk_hi, off, 64), ol = __shfl_xor(blk_lo, off, 64);
        blk_hi = oh > blk_hi ? oh : blk_hi;
        blk_lo = ol < blk_lo ? ol : blk_lo;
    }
    int64_t j_begin = kSplit ? static_cast<int64_t>(rng) * p.split_len : 0;
    int64_t j_end = blk_hi;
    if (kSplit && j_begin + p.split_len < j_end) j_end = j_begin + p.split_len;
    if (kVar && blk_lo != INT64_MAX && blk_lo > j_begin)   // whole tiles below every row's bound
        j_begin += (blk_lo - j_begin) / kTile * kTile;
    const int n_tiles = j_end > j_begin ? static_cast<int>((j_end - j_begin + kTile - 1) / kTile) : 0;

    const float* qg = static_cast<const float*>(p.q);
    const float* kg = static_cast<const float*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const float* vg = static_cast<const float*>(p.v) + b * p.vs.sb + g * p.vs.sh;

    // Columns gl * DQ .. gl * DQ + DQ - 1 of the padded row; columns >= D are 0.
    float q[R][DQ];
    const float* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float* src = qg + b * p.qs.sb + h * p.qs.sh + (row_ok[r] ? row[r] : 0) * p.qs.sr;
#pragma unroll
        for (int d = 0; d < DQ; ++d) {
            const int cix = gl * DQ + d;
            q[r][d] = (row_ok[r] && cix < D) ? src[cix] : 0.f;
        }
        mrow[r] = (kMask && row_ok[r]) ? p.mask + b * p.ms.sb + h * p.ms.sh + row[r] * p.ms.sr
                                       : nullptr;
    }

    // Tile loads: float4 f = n * 64 + lane of the tile is row f / kRowF4,
    // columns 4 (f % kRowF4) .. + 3; keys past the range and columns past D
    // load as zeros.
    float4 kst[LY::kLoads], vst[LY::kLoads];
    auto ld4 = [&](const float* base, int64_t sr, int64_t key, int c4, bool in) {
        if (!in) return make_float4(0.f, 0.f, 0.f, 0.f);
        const float* src = base + key * sr + c4;
        if (vec && c4 + 3 < D) return *reinterpret_cast<const float4*>(src);
        return make_float4(c4 < D ? src[0] : 0.f, c4 + 1 < D ? src[1] : 0.f,
                           c4 + 2 < D ? src[2] : 0.f, c4 + 3 < D ? src[3] : 0.f);
    };
    auto fetch = [&](int tile) {
#pragma unroll
        for (int n = 0; n < LY::kLoads; ++n) {
            const int f = n * 64 + lane;
            const int64_t key = j_begin + static_cast<int64_t>(tile) * kTile + f / LY::kRowF4;
            const int c4 = 4 * (f % LY::kRowF4);
            const bool in = key < j_end;
            kst[n] = ld4(kg, p.ks.sr, key, c4, in);
            vst[n] = ld4(vg, p.vs.sr, key, c4, in);
        }
    };

    // Score units: raw q.k without a mask; natural (scale * q.k + mask, the
    // mask added as given, so a large finite value stays finite) with one.
    const float c = kMask ? kLog2e : p.scale_log2;   // score units -> base 2
    const float to_nat = kMask ? 1.f : p.scale;       // score units -> natural
    const float slack = kSlack / c;
    const bool cap = kVar && p.softcap > 0.f;
    const float cap_k2 = cap ? 2.f * kLog2e * p.scale / p.softcap : 0.f;
    const float cap_back = cap ? p.softcap / p.scale : 0.f;
    float m_ref[R], l_sum[R], acc[R][DQ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m_ref[r] = kNegInf;
        l_sum[r] = 0.f;
#pragma unroll
        for (int d = 0; d < DQ; ++d) acc[r][d] = 0.f;
    }

    if (n_tiles > 0) fetch(0);
    for (int tile = 0; tile < n_tiles; ++tile) {
        // The previous tile's LDS reads precede these writes in this wave's
        // in-order LDS queue, so one buffer suffices.
#pragma unroll
        for (int n = 0; n < LY::kLoads; ++n) {
            const int f = n * 64 + lane;
            const int rr = f / LY::kRowF4, c4 = 4 * (f % LY::kRowF4);
            *reinterpret_cast<float4*>(&k_sh[rr * DP + c4]) = kst[n];
            *reinterpret_cast<float4*>(&v_sh[rr * DP + c4]) = vst[n];
        }
        if (tile + 1 < n_tiles) fetch(tile + 1);
        const int64_t j0 = j_begin + static_cast<int64_t>(tile) * kTile;

        float s[R][kTile];
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float* kr = &k_sh[j * DP + gl * DQ];
            float part[R];
#pragma unroll
            for (int r = 0; r < R; ++r) part[r] = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d += 4) {
                const float4 kv = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    part[r] = fmaf(q[r][d], kv.x, part[r]);
                    part[r] = fmaf(q[r][d + 1], kv.y, part[r]);
                    part[r] = fmaf(q[r][d + 2], kv.z, part[r]);
                    part[r] = fmaf(q[r][d + 3], kv.w, part[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) s[r][j] = group_sum<G>(part[r]);
        }
        float tacc[R][DQ];   // this tile's products (blockwise summation)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (cap) {
#pragma unroll
                for (int j = 0; j < kTile; ++j) s[r][j] = softcap_raw(s[r][j], cap_k2, cap_back);
            }
            if (kMask && mrow[r]) {
#pragma unroll
                for (int j = 0; j < kTile; ++j)
                    s[r][j] = (j0 + j < j_end) ? fmaf(s[r][j], p.scale, mrow[r][j0 + j])
                                               : s[r][j] * p.scale;
            }
            const bool partial = (j0 + kTile > j_end) || (j0 + kTile > row_hi[r]) ||
                                 (kVar && j0 < row_lo[r]) || !row_ok[r];
            if (partial) {
#pragma unroll
                for (int j = 0; j < kTile; ++j) {
                    const int64_t key = j0 + j;
                    if (key >= j_end || key >= row_hi[r] || (kVar && key < row_lo[r]))
                        s[r][j] = kNegInf;
                }
            }
            float mx = kNegInf;
#pragma unroll
            for (int j = 0; j < kTile; j += 2) mx = fmaxf(mx, fmaxf(s[r][j], s[r][j + 1]));
            const bool raise = mx > m_ref[r] + slack;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float m_new = raise ? mx : m_ref[r];
                const float alpha = raise ? fast_exp2((m_ref[r] - m_new) * c) : 1.f;   // 0 when m_ref = -inf
                l_sum[r] *= alpha;
#pragma unroll
                for (int d = 0; d < DQ; ++d) acc[r][d] *= alpha;
                m_ref[r] = m_new;
            }
            // (s - m) * c rather than fma(s, c, -m*c): the subtraction is
            // exact for the row maximum, so its weight is exactly 1 (p is not
            // rounded to a narrower type on this path).
            const float base = (m_ref[r] == kNegInf) ? 0.f : m_ref[r];
            float tl = 0.f;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                s[r][j] = fast_exp2((s[r][j] - base) * c);
                tl += s[r][j];
            }
            l_sum[r] += tl;
#pragma unroll
            for (int d = 0; d < DQ; ++d) tacc[r][d] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float* vr = &v_sh[j * DP + gl * DQ];
#pragma unroll
            for (int d = 0; d < DQ; d += 4) {
                const float4 vv = *reinterpret_cast<const float4*>(vr + d);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    tacc[r][d] = fmaf(s[r][j], vv.x, tacc[r][d]);
                    tacc[r][d + 1] = fmaf(s[r][j], vv.y, tacc[r][d + 1]);
                    tacc[r][d + 2] = fmaf(s[r][j], vv.z, tacc[r][d + 2]);
                    tacc[r][d + 3] = fmaf(s[r][j], vv.w, tacc[r][d + 3]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int d = 0; d < DQ; ++d) acc[r][d] += tacc[r][d];
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (!row_ok[r]) continue;
        const int64_t i = row[r];
        if (kSplit) {
            float* rec = static_cast<float*>(p.ws) +
                         (((static_cast<int64_t>(b) * p.Hq + h) * p.Lq + i) * p.n_split + rng) * (DP + 4);
#pragma unroll
            for (int d = 0; d < DQ; d += 4)
                *reinterpret_cast<float4*>(rec + 4 + gl * DQ + d) =
                    make_float4(acc[r][d], acc[r][d + 1], acc[r][d + 2], acc[r][d + 3]);
            if (gl == 0) {
                rec[0] = m_ref[r];
                rec[1] = l_sum[r];
            }
            continue;
        }
        float m_nat = m_ref[r] * to_nat;          // natural units (-inf stays -inf)
        float l_tot = l_sum[r];
        const float fs = fold_sink(p, h, m_nat, l_tot);
        const bool empty = (l_tot == 0.f);
        const float inv = fs / l_tot;
        const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
        float* og = static_cast<float*>(p.o) + b * p.os.sb + h * p.os.sh + i * p.os.sr;
#pragma unroll
        for (int d = 0; d < DQ; ++d) {
            const int cix = gl * DQ + d;
            if (cix < D) og[cix] = empty ? fill : acc[r][d] * inv;
        }
        if (p.lse && gl == 0)
            p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = empty ? kNegInf : row_lse(m_nat, l_tot);
    }
}

// Rows per wave of the kernel that runs head dim D.
int f32_padded(int D) {
    return D <= 32 ? 32 : (D <= 64 ? 64 : (D <= 96 ? 96 : (D <= 128 ? 128 : 256)));
}
int f32_rows_per_wave(int D) {
    switch (f32_padded(D)) {
    case 32: return F32Lay<32>::RW;
    case 64: return F32Lay<64>::RW;
    case 96: return F32Lay<96>::RW;
    case 128: return F32Lay<128>::RW;
    default: return F32Lay<256>::RW;
    }
}

// One thread per (b, h, row, dim): merge the ranges the row's block wrote, in
// order, then the sink, the masked-row policy and the LSE as the main
// kernel's epilogue does.  Records are in the main kernel's score units: c
// converts a difference of them to base 2, to_nat a value to natural units.
template <int DP>
__global__ __launch_bounds__(256) void prefill_f32_merge_kernel(Params p, float c, float to_nat) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(p.B) * p.Hq * p.Lq * p.D;
    if (t >= total) return;
    const int d = static_cast<int>(t % p.D);
    const int64_t row = t / p.D;                     // (b, h, i) flattened
    const int64_t i = row % p.Lq;
    const int h = static_cast<int>((row / p.Lq) % p.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(p.Lq) * p.Hq));
    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    // The ranges below the block's causal bound are the ones its wave wrote
    // (a range past it returned before writing).
    constexpr int rw = F32Lay<DP>::RW;
    int64_t blk_hi = kv_len;
    if (p.causal) {
        const int64_t last = ((i / rw + 1) * rw < p.Lq ? (i / rw + 1) * rw : p.Lq) - 1;
        const int64_t bb = last + causal_delta(p, kv_len) + 1;
        blk_hi = bb < 0 ? 0 : (bb < blk_hi ? bb : blk_hi);
    }
    const int n_live = static_cast<int>((blk_hi + p.split_len - 1) / p.split_len);
    const float* recs = static_cast<const float*>(p.ws) + row * p.n_split * (DP + 4);
    // Eight ranges' (m, l, acc[d]) are fetched together per round; the
    // reference maximum is the largest seen so far, so up to eight ranges
    // fold in one round exactly as a separate maximum pass would.
    float M = kNegInf, L = 0.f, A = 0.f;
    for (int r0 = 0; r0 < n_live; r0 += 8) {
        float m8[8], l8[8], a8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = r0 + u < n_live;
            const float* rec = recs + (in ? r0 + u : 0) * (DP + 4);
            m8[u] = in ? rec[0] : kNegInf;
            l8[u] = in ? rec[1] : 0.f;
            a8[u] = in ? rec[4 + d] : 0.f;
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, m8[u]);
        if (Mn != M) {   // raise the reference (from -inf: nothing folded yet)
            const float al = (M == kNegInf) ? 0.f : fast_exp2((M - Mn) * c);
            L *= al;
            A *= al;
            M = Mn;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (r0 + u >= n_live) break;
            const float f = (m8[u] == kNegInf) ? 0.f : fast_exp2((m8[u] - M) * c);
            L = fmaf(l8[u], f, L);
            A = fmaf(a8[u], f, A);
        }
    }
    float m_nat = M * to_nat;
    const float fs = fold_sink(p, h, m_nat, L);
    const bool empty = (L == 0.f);
    const float o = empty ? (p.masked_zero ? 0.f : __builtin_nanf("")) : A * (fs / L);
    static_cast<float*>(p.o)[b * p.os.sb + h * p.os.sh + i * p.os.sr + d] = o;
    if (p.lse && d == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = empty ? kNegInf : row_lse(m_nat, L);
}

bool f32_var(const Params& p) {
    return p.softcap > 0.f || (p.causal && p.window > 0) || p.doc_start || p.sink;
}

template <int DP>
hipError_t launch_d(const Params& p, hipStream_t s) {
    const int n_rblk = (p.Lq + F32Lay<DP>::RW - 1) / F32Lay<DP>::RW;
    const dim3 grid(n_rblk, p.Hq, p.B * p.n_split);
    const bool split = p.n_split > 1;
    // 16-byte K/V loads when every row starts 16-byte aligned and holds whole float4s.
    auto al = [](const void* ptr, const Strides& st) {
        return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && st.sb % 4 == 0 && st.sh % 4 == 0 &&
               st.sr % 4 == 0;
    };
    const int vec = (p.D % 4 == 0) && (p.Lk == 0 || (al(p.k, p.ks) && al(p.v, p.vs)));
    auto go = [&](auto mask_c, auto split_c, auto var_c) {
        constexpr bool kM = decltype(mask_c)::value, kS = decltype(split_c)::value;
        constexpr bool kV = decltype(var_c)::value;
        hipLaunchKernelGGL((prefill_f32_kernel<DP, kM, kS, kV>), grid, dim3(64), 0, s, p, n_rblk, vec);
    };
    using T = std::true_type;
    using F = std::false_type;
    auto by_var = [&](auto mask_c, auto split_c) {
        if (f32_var(p)) go(mask_c, split_c, T{});
        else go(mask_c, split_c, F{});
    };
    auto by_split = [&](auto mask_c) {
        if (split) by_var(mask_c, T{});
        else by_var(mask_c, F{});
    };
    if (p.mask) by_split(T{});
    else by_split(F{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    const int64_t total = static_cast<int64_t>(p.B) * p.Hq * p.Lq * p.D;
    const float c = p.mask ? kLog2e : p.scale_log2, to_nat = p.mask ? 1.f : p.scale;
    hipLaunchKernelGGL((prefill_f32_merge_kernel<DP>), dim3(static_cast<uint32_t>((total + 255) / 256)),
                       dim3(256), 0, s, p, c, to_nat);
    return hipGetLastError();
}

}  // namespace

// Key ranges for the fp32 kernel: only when the row blocks give fewer than
// ~2048 waves; ranges are multiples of 32 keys, at least 128, at most 16.
void prefill_f32_plan(int B, int Hq, int Lq, int Lk, int D, int* split_len, int* n_split) {
    const int rw = f32_rows_per_wave(D);
    const int64_t units = static_cast<int64_t>((Lq + rw - 1) / rw) * Hq * B;
    int n = 1;
    if (units < 2048 && Lk >= 256) {
        const int64_t want = (2048 + units - 1) / units;
        const int64_t most = Lk / 128;
        n = static_cast<int>(want < most ? want : most);
        if (n > 16) n = 16;
        if (n < 1) n = 1;
    }
    int len = (Lk + n - 1) / n;
    len = (len + kRangeQuantum - 1) / kRangeQuantum * kRangeQuantum;
    if (len < kRangeQuantum) len = kRangeQuantum;
    *split_len = len;
    *n_split = Lk > 0 ? (Lk + len - 1) / len : 1;
    if (*n_split < 1) *n_split = 1;
}

size_t prefill_f32_workspace_bytes(int B, int Hq, int Lq, int Lk, int D) {
    int len, n;
    prefill_f32_plan(B, Hq, Lq, Lk, D, &len, &n);
    if (n <= 1) return 0;
    return static_cast<size_t>(B) * Hq * Lq * n * (f32_padded(D) + 4) * sizeof(float);
}

bool prefill_f32_supported(const Params& p, DType dt) {
    if (dt != DType::F32) return false;
    if (p.D < 1 || p.D > 256) return false;
    // Q, O and the mask are read and written per element; K and V per
    // float4 when aligned, else per element (the launch picks).
    return p.Hq <= 65535 && static_cast<int64_t>(p.B) * p.n_split <= 65535;
}

hipError_t launch_prefill_f32(const Params& p, DType, hipStream_t s) {
    switch (f32_padded(p.D)) {
    case 32: return launch_d<32>(p, s);
    case 64: return launch_d<64>(p, s);
    case 96: return launch_d<96>(p, s);
    case 128: return launch_d<128>(p, s);
    default: return launch_d<256>(p, s);
    }
}

}  // namespace sdpa
