// prefill_f32.hip -- fused attention for float32 inputs on the vector FMA
// units (head_dim 32, 64 or 128).
//
// Four neighbouring lanes own a query row, each a quarter of the head
// dimension: a score is four partial dot products added by two quad
// exchanges (DPP), so every lane of the quad holds the same score and takes
// the same softmax decisions (OneGPU "Attention", "Variants and ordering":
// the `pairs` variant splits the head dimension over neighbouring threads and
// joins the halves with a shuffle).  For head dims up to 64 each quad owns
// two rows (16 apart), so every K/V value read from LDS feeds two FMAs: one
// read per FMA would leave the loop bound by LDS bandwidth, not by the FMA
// units.  A wave therefore owns 32 rows (16 at head dim 128) of one (batch,
// head).  Keys are folded in increasing order, 16 per tile (32 at head dim
// 128), from the wave's own LDS rows (coalesced 16-byte loads, next tile
// prefetched into registers), with the online normaliser and a lazily raised
// reference max as in the matrix-core kernel; in float32 the probabilities
// are not rounded.  (Two rows per quad with 32-key tiles, or four rows, need
// more than 256 registers and leave one wave per SIMD: both measured slower.)
//
// When the query blocks are too few to fill the GPU, the keys are cut into
// contiguous ranges (a multiple of 32 keys, at least 128, at most 16 ranges);
// each (rows, range) wave writes its partial (m, l, acc) and a second kernel
// merges the ranges of each row in range order (OneGPU "Attention", "Accuracy
// at long key lengths", last paragraph).  The cut depends only on the shape.
#include "attn_internal.h"
#include "device_common.h"

namespace sdpa {

namespace {

constexpr int kRangeQuantum = 32;   // key ranges are multiples of this

// Rows per lane quad, and rows per wave.
__host__ __device__ constexpr int rows_per_quad(int D) { return D <= 64 ? 2 : 1; }
__host__ __device__ constexpr int rows_per_wave(int D) { return 16 * rows_per_quad(D); }
// Keys per tile: 16 when a quad owns two rows, so the scores fit beside the
// prefetched tile in 256 registers (two waves per SIMD).
__host__ __device__ constexpr int tile_of(int D) { return rows_per_quad(D) == 2 ? 16 : 32; }
constexpr float kSlack = 8.f;    // lazy-rescale threshold, base-2 units

// Quad sum: both exchange steps add the same two numbers on each partner, so
// all four lanes end with identical bits.
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    return x;
}

template <int D> struct F32Lay {
    static constexpr int kTile = tile_of(D);
    static constexpr int DQ = D / 4;                  // dims per lane
    static constexpr int kRowF4 = D / 4;              // float4 per row
    static constexpr int kLoads = kTile * kRowF4 / 64;   // float4 loads per lane per tensor
    static constexpr int kRowsPerLoad = 64 / kRowF4;
};

template <int D, bool kMask, bool kSplit>
__global__ __launch_bounds__(64) void prefill_f32_kernel(Params p, int n_rblk) {
    using LY = F32Lay<D>;
    constexpr int DQ = LY::DQ;
    constexpr int R = rows_per_quad(D);
    constexpr int RW = rows_per_wave(D);
    constexpr int kTile = LY::kTile;
    __shared__ __attribute__((aligned(16))) float k_sh[kTile * D];
    __shared__ __attribute__((aligned(16))) float v_sh[kTile * D];

    // blockIdx.x: row block (heaviest causal blocks first); y: head; z: batch * ranges.
    const int rb = n_rblk - 1 - static_cast<int>(blockIdx.x);
    const int h = blockIdx.y;
    const int b = static_cast<int>(blockIdx.z) / p.n_split;
    const int rng = static_cast<int>(blockIdx.z) % p.n_split;
    const int g = h / p.group;
    const int lane = threadIdx.x;
    const int quad = lane >> 2, qd = lane & 3;

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const int64_t delta = causal_delta(p, kv_len);
    // Keys the block can see, and this range of them.
    int64_t blk_hi = kv_len;
    if (p.causal) {
        const int64_t last = (static_cast<int64_t>(rb + 1) * RW < p.Lq
                                  ? static_cast<int64_t>(rb + 1) * RW : p.Lq) - 1;
        const int64_t bb = last + delta + 1;
        blk_hi = bb < 0 ? 0 : (bb < blk_hi ? bb : blk_hi);
    }
    const int64_t j_begin = kSplit ? static_cast<int64_t>(rng) * p.split_len : 0;
    int64_t j_end = blk_hi;
    if (kSplit && j_begin + p.split_len < j_end) j_end = j_begin + p.split_len;
    if (kSplit && j_begin >= blk_hi) return;   // no row of the block sees this range
    const int n_tiles = j_end > j_begin ? static_cast<int>((j_end - j_begin + kTile - 1) / kTile) : 0;

    // This lane's rows: rb * RW + 16 r + quad, r < R.
    int64_t row[R], row_hi[R];
    bool row_ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = static_cast<int64_t>(rb) * RW + 16 * r + quad;
        row_ok[r] = row[r] < p.Lq;
        row_hi[r] = p.causal ? row[r] + delta + 1 : kv_len;   // key < row_hi visible
    }

    const float* qg = static_cast<const float*>(p.q);
    const float* kg = static_cast<const float*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const float* vg = static_cast<const float*>(p.v) + b * p.vs.sb + g * p.vs.sh;

    float q[R][DQ];
    const float* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float* src = qg + b * p.qs.sb + h * p.qs.sh + (row_ok[r] ? row[r] : 0) * p.qs.sr + qd * DQ;
#pragma unroll
        for (int d = 0; d < DQ; d += 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + d);
            q[r][d] = row_ok[r] ? v.x : 0.f;
            q[r][d + 1] = row_ok[r] ? v.y : 0.f;
            q[r][d + 2] = row_ok[r] ? v.z : 0.f;
            q[r][d + 3] = row_ok[r] ? v.w : 0.f;
        }
        mrow[r] = (kMask && row_ok[r]) ? p.mask + b * p.ms.sb + h * p.ms.sh + row[r] * p.ms.sr
                                       : nullptr;
    }

    const int ld_row = lane / LY::kRowF4;
    const int ld_col = (lane % LY::kRowF4) * 4;
    float4 kst[LY::kLoads], vst[LY::kLoads];
    auto fetch = [&](int tile) {
#pragma unroll
        for (int n = 0; n < LY::kLoads; ++n) {
            const int64_t key = j_begin + static_cast<int64_t>(tile) * kTile + n * LY::kRowsPerLoad + ld_row;
            if (key < j_end) {
                kst[n] = *reinterpret_cast<const float4*>(kg + key * p.ks.sr + ld_col);
                vst[n] = *reinterpret_cast<const float4*>(vg + key * p.vs.sr + ld_col);
            } else {
                kst[n] = make_float4(0.f, 0.f, 0.f, 0.f);
                vst[n] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };

    // Score units: raw q.k without a mask; natural (scale * q.k + mask, the
    // mask added as given, so a large finite value stays finite) with one.
    const float c = kMask ? kLog2e : p.scale_log2;   // score units -> base 2
    const float to_nat = kMask ? 1.f : p.scale;       // score units -> natural
    const float slack = kSlack / c;
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
            const int rr = n * LY::kRowsPerLoad + ld_row;
            *reinterpret_cast<float4*>(&k_sh[rr * D + ld_col]) = kst[n];
            *reinterpret_cast<float4*>(&v_sh[rr * D + ld_col]) = vst[n];
        }
        if (tile + 1 < n_tiles) fetch(tile + 1);
        const int64_t j0 = j_begin + static_cast<int64_t>(tile) * kTile;

        float s[R][kTile];
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float* kr = &k_sh[j * D + qd * DQ];
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
            for (int r = 0; r < R; ++r) s[r][j] = quad_sum(part[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (kMask && mrow[r]) {
#pragma unroll
                for (int j = 0; j < kTile; ++j)
                    s[r][j] = (j0 + j < j_end) ? fmaf(s[r][j], p.scale, mrow[r][j0 + j])
                                               : s[r][j] * p.scale;
            }
            const bool partial = (j0 + kTile > j_end) || (j0 + kTile > row_hi[r]) || !row_ok[r];
            if (partial) {
#pragma unroll
                for (int j = 0; j < kTile; ++j) {
                    const int64_t key = j0 + j;
                    if (key >= j_end || key >= row_hi[r] || key >= kv_len || !row_ok[r])
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
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                s[r][j] = fast_exp2((s[r][j] - base) * c);
                l_sum[r] += s[r][j];
            }
        }
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float* vr = &v_sh[j * D + qd * DQ];
#pragma unroll
            for (int d = 0; d < DQ; d += 4) {
                const float4 vv = *reinterpret_cast<const float4*>(vr + d);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    acc[r][d] = fmaf(s[r][j], vv.x, acc[r][d]);
                    acc[r][d + 1] = fmaf(s[r][j], vv.y, acc[r][d + 1]);
                    acc[r][d + 2] = fmaf(s[r][j], vv.z, acc[r][d + 2]);
                    acc[r][d + 3] = fmaf(s[r][j], vv.w, acc[r][d + 3]);
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (!row_ok[r]) continue;
        const int64_t i = row[r];
        if (kSplit) {
            float* rec = static_cast<float*>(p.ws) +
                         (((static_cast<int64_t>(b) * p.Hq + h) * p.Lq + i) * p.n_split + rng) * (D + 4);
#pragma unroll
            for (int d = 0; d < DQ; d += 4)
                *reinterpret_cast<float4*>(rec + 4 + qd * DQ + d) =
                    make_float4(acc[r][d], acc[r][d + 1], acc[r][d + 2], acc[r][d + 3]);
            if (qd == 0) {
                rec[0] = m_ref[r];
                rec[1] = l_sum[r];
            }
            continue;
        }
        const bool empty = (l_sum[r] == 0.f);
        const float inv = 1.f / l_sum[r];
        const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
        float* og = static_cast<float*>(p.o) + b * p.os.sb + h * p.os.sh + i * p.os.sr + qd * DQ;
#pragma unroll
        for (int d = 0; d < DQ; d += 4)
            *reinterpret_cast<float4*>(og + d) =
                empty ? make_float4(fill, fill, fill, fill)
                      : make_float4(acc[r][d] * inv, acc[r][d + 1] * inv, acc[r][d + 2] * inv,
                                    acc[r][d + 3] * inv);
        if (p.lse && qd == 0)
            p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] =
                empty ? kNegInf : row_lse(m_ref[r] * to_nat, l_sum[r]);
    }
}

// One thread per (b, h, row, dim): merge the row's live ranges in order.
// Records are in the main kernel's score units: c converts a difference of
// them to base 2, to_nat a value to natural units.
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_merge_kernel(Params p, float c, float to_nat) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(p.B) * p.Hq * p.Lq * D;
    if (t >= total) return;
    const int d = static_cast<int>(t % D);
    const int64_t row = t / D;                       // (b, h, i) flattened
    const int64_t i = row % p.Lq;
    const int h = static_cast<int>((row / p.Lq) % p.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(p.Lq) * p.Hq));
    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    int64_t hi = kv_len;
    if (p.causal) {
        const int64_t bb = i + causal_delta(p, kv_len) + 1;
        hi = bb < 0 ? 0 : (bb < hi ? bb : hi);
    }
    const int n_live = static_cast<int>((hi + p.split_len - 1) / p.split_len);
    const float* recs = static_cast<const float*>(p.ws) + row * p.n_split * (D + 4);
    // Eight ranges' (m, l, acc[d]) are fetched together per round; the
    // reference maximum is the largest seen so far, so up to eight ranges
    // fold in one round exactly as a separate maximum pass would.
    float M = kNegInf, L = 0.f, A = 0.f;
    for (int r0 = 0; r0 < n_live; r0 += 8) {
        float m8[8], l8[8], a8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = r0 + u < n_live;
            const float* rec = recs + (in ? r0 + u : 0) * (D + 4);
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
    const bool empty = (L == 0.f);
    const float o = empty ? (p.masked_zero ? 0.f : __builtin_nanf("")) : A / L;
    static_cast<float*>(p.o)[b * p.os.sb + h * p.os.sh + i * p.os.sr + d] = o;
    if (p.lse && d == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = empty ? kNegInf : row_lse(M * to_nat, L);
}

template <int D>
hipError_t launch_d(const Params& p, hipStream_t s) {
    const int n_rblk = (p.Lq + rows_per_wave(D) - 1) / rows_per_wave(D);
    const dim3 grid(n_rblk, p.Hq, p.B * p.n_split);
    const bool split = p.n_split > 1;
    if (p.mask) {
        if (split) hipLaunchKernelGGL((prefill_f32_kernel<D, true, true>), grid, dim3(64), 0, s, p, n_rblk);
        else hipLaunchKernelGGL((prefill_f32_kernel<D, true, false>), grid, dim3(64), 0, s, p, n_rblk);
    } else {
        if (split) hipLaunchKernelGGL((prefill_f32_kernel<D, false, true>), grid, dim3(64), 0, s, p, n_rblk);
        else hipLaunchKernelGGL((prefill_f32_kernel<D, false, false>), grid, dim3(64), 0, s, p, n_rblk);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    const int64_t total = static_cast<int64_t>(p.B) * p.Hq * p.Lq * D;
    const float c = p.mask ? kLog2e : p.scale_log2, to_nat = p.mask ? 1.f : p.scale;
    hipLaunchKernelGGL((prefill_f32_merge_kernel<D>), dim3(static_cast<uint32_t>((total + 255) / 256)),
                       dim3(256), 0, s, p, c, to_nat);
    return hipGetLastError();
}

}  // namespace

// Key ranges for the fp32 kernel: only when the row blocks give fewer than
// ~2048 waves; ranges are multiples of 32 keys, at least 128, at most 16.
void prefill_f32_plan(int B, int Hq, int Lq, int Lk, int D, int* split_len, int* n_split) {
    const int rw = rows_per_wave(D);
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
    return static_cast<size_t>(B) * Hq * Lq * n * (D + 4) * sizeof(float);
}

bool prefill_f32_supported(const Params& p, DType dt) {
    if (dt != DType::F32) return false;
    if (p.D != 32 && p.D != 64 && p.D != 128) return false;
    // Local window, softcap and sink run on the any-shape kernel for fp32.
    if (p.window > 0 || p.softcap > 0.f || p.sink || p.doc_start) return false;
    auto al = [](const void* ptr, const Strides& st) {
        return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && st.sb % 4 == 0 && st.sh % 4 == 0 &&
               st.sr % 4 == 0;
    };
    if (!al(p.q, p.qs) || !al(p.o, p.os)) return false;
    if (p.Lk > 0 && (!al(p.k, p.ks) || !al(p.v, p.vs))) return false;
    return p.Hq <= 65535 && static_cast<int64_t>(p.B) * p.n_split <= 65535;
}

hipError_t launch_prefill_f32(const Params& p, DType, hipStream_t s) {
    if (p.D == 32) return launch_d<32>(p, s);
    if (p.D == 64) return launch_d<64>(p, s);
    return launch_d<128>(p, s);
}

}  // namespace sdpa
