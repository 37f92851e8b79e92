// prefill_f32.hip -- fused attention for float32 inputs on the gfx950 matrix
// cores (v_mfma_f32_32x32x2_f32: float32 operands and accumulation), head
// dims 1..256 (padded to 32, 64, 96, 128 or 256; padded columns load as zeros
// and are not stored).
//
// A workgroup of four waves owns 128 query rows of one kv head's group
// (4 heads x 32 positions, 2 x 64 or 1 x 128, the most heads that divide the
// group), each wave 32 rows.  Keys come in tiles of 32, loaded by all four
// waves straight from HBM into LDS (4-byte buffer loads into LDS: any head
// dim and row stride, zeros past the key length and the head dim), double
// buffered.  Per tile and wave:
//   S^T = K Q^T    -- DP/2 matrix ops; lane l holds query row l%32 and Q's
//                     columns h DP/2 .. h DP/2 + DP/2 - 1 (h = l/32) in
//                     registers, K's matching columns come from LDS;
//   softmax        -- the lane owns its row's 16 keys 8(r/4) + 4h + r%4 of
//                     the tile (the other 16 are in lane l^32): lazily raised
//                     reference max, p = 2^((s - m) c), not rounded (fp32);
//   O^T += V^T P^T -- P^T is the score accumulator itself (register r is the
//                     operand of step r), V^T read per lane from LDS.
// Blockwise summation (OneGPU "Attention", "Accuracy at long key lengths"):
// each tile's products go to a zero-started accumulator and its
// probabilities to a zero-started sum, which are added to the running ones
// once per tile.
//
// Score-rule variants (ONNX GroupQueryAttention README, "Attributes",
// "Inputs") and document masks (llm.istanbul "05_attention", "Phase 0" and
// "K-block iteration") in the kVar kernel: each row's first visible key
// (local window, document start) bounds it from below and the tiles below
// the workgroup's smallest bound are skipped; the softcap maps the raw score
// before the mask; the sink joins the denominator at the end.  A wave skips
// the matrix work of a tile none of its rows can see.
//
// When the workgroups are too few to fill the GPU, the keys are cut into
// contiguous ranges (whole tiles); each (rows, range) wave writes its partial
// (m, l, acc) and a second kernel merges the ranges of each row in range
// order (OneGPU "Attention", "Accuracy at long key lengths", last paragraph).
// The cut depends only on the shape.
#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"
#include "mfma_common.h"

namespace sdpa {

namespace {

using mfma::f32x16;
using mfma::f32x4;
using mfma::halves_max;
using mfma::halves_sum;
using mfma::make_rsrc;
using mfma::max_nan;

constexpr int kTileN = 32;          // keys per tile
constexpr int kRangeQuantum = 64;   // key ranges are multiples of this (two tiles)
constexpr int kWavesF = 4;          // waves per workgroup
constexpr float kSlack = 8.f;       // lazy-rescale threshold, base-2 units
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past any tensor

// Padded head dim DP: LDS rows of DP + 4 floats (the 16-byte shift per row
// keeps the 16-byte column reads of 16 rows on distinct banks).
template <int DP> struct F32Cfg {
    static constexpr int kRowF = DP + 4;                    // floats per LDS row
    static constexpr int kTileF = kTileN * kRowF;           // floats of a tile
    static constexpr int kLoads = kTileF / 64;              // 4-byte DMA rows per tile
    static constexpr int kLoads16 = (kTileF + 255) / 256;   // 16-byte DMA rows per tile
    static constexpr int kBufF = kLoads16 * 256;            // floats per tile buffer
    static constexpr int kHalf = DP / 2;                    // Q columns per lane
    static constexpr int kBlk = DP / 32;                    // 32-column output blocks
    static constexpr int kMinWg = DP <= 128 ? 2 : 1;        // workgroups per CU (registers)
    // Up to 64 columns, three workgroups per CU where the registers allow
    // it without spills (not the key-range split kernels): 3-4% faster.
    static constexpr int kMinWg3 = DP <= 64 ? 3 : kMinWg;
    static_assert(kTileF % 64 == 0, "a tile buffer is whole DMA rows");
    static_assert(kHalf % 4 == 0, "Q halves are whole 16-byte LDS reads");
};

// One 4-byte-per-lane buffer load into LDS at lds_byte + 4 * lane (M0 holds
// the LDS address; one wait state after writing it), and the 16-byte form at
// lds_byte + 16 * lane.  Instructions of their own, so the compiler does not
// hold later LDS reads of the other buffer for them; the kernel waits for
// these loads itself before the barrier that publishes a tile.
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rs, uint32_t lds_byte,
                                          uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "{m0}"(lds_byte));
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_byte,
                                           uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "{m0}"(lds_byte));
}

__device__ __forceinline__ void dma_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Key offset (within a 32-key tile) of accumulator register r in lane half h:
// the 32x32 accumulator puts rows 8(r/4) + 4h + r%4 in register r.
__device__ __forceinline__ constexpr int key_of(int r, int h) {
    return 8 * (r / 4) + 4 * h + (r % 4);
}

template <int DP, bool kMask, bool kSplit, bool kVar>
__global__ __launch_bounds__(256, kSplit ? F32Cfg<DP>::kMinWg : F32Cfg<DP>::kMinWg3) void prefill_f32_kernel(Params p,
                                                                                int n_qblk,
                                                                                int gw,
                                                                                int vec) {
    using CF = F32Cfg<DP>;
    __shared__ __attribute__((aligned(16))) float k_sh[2][CF::kBufF];
    __shared__ __attribute__((aligned(16))) float v_sh[2][CF::kBufF];
    __shared__ int64_t wg_bounds[2 * kWavesF];

    // blockIdx.x: query block (heaviest causal blocks first); y: (kv head,
    // head slice); z: batch * ranges.
    const int qb = n_qblk - 1 - static_cast<int>(blockIdx.x);
    const int n_slice = p.group / gw;
    const int g = static_cast<int>(blockIdx.y) / n_slice;
    const int slice = static_cast<int>(blockIdx.y) % n_slice;
    const int b = static_cast<int>(blockIdx.z) / p.n_split;
    const int rng = static_cast<int>(blockIdx.z) % p.n_split;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int hh = lane >> 5, col = lane & 31;
    const int wph = kWavesF / gw;                 // waves per head
    const int h = g * p.group + slice * gw + w / wph;
    const int64_t row = static_cast<int64_t>(qb) * (32 * wph) + 32 * (w % wph) + col;
    const bool row_ok = row < p.Lq;
    const int D = p.D;

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const int64_t delta = causal_delta(p, kv_len);
    // Keys [row_lo, row_hi) are visible to this lane's row (before the mask).
    int64_t row_hi = kv_len, row_lo = 0;
    if (p.causal) {
        const int64_t bb = row + delta + 1;
        row_hi = bb < row_hi ? bb : row_hi;
    }
    if (row_hi < 0 || !row_ok) row_hi = 0;
    if (kVar && row_ok) row_lo = first_key(p, b, row, delta);

    // The wave's bounds (max of hi, min of lo over its valid rows), then the
    // workgroup's.
    int64_t w_hi = row_hi, w_lo = row_ok ? row_lo : INT64_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t oh = __shfl_xor(w_hi, off, 64), ol = __shfl_xor(w_lo, off, 64);
        w_hi = oh > w_hi ? oh : w_hi;
        w_lo = ol < w_lo ? ol : w_lo;
    }
    if (lane == 0) {
        wg_bounds[2 * w] = w_hi;
        wg_bounds[2 * w + 1] = w_lo;
    }
    __syncthreads();
    int64_t blk_hi = 0, blk_lo = INT64_MAX;
#pragma unroll
    for (int i = 0; i < kWavesF; ++i) {
        blk_hi = wg_bounds[2 * i] > blk_hi ? wg_bounds[2 * i] : blk_hi;
        blk_lo = wg_bounds[2 * i + 1] < blk_lo ? wg_bounds[2 * i + 1] : blk_lo;
    }
    const int64_t r_begin = kSplit ? static_cast<int64_t>(rng) * p.split_len : 0;
    // A range at or past the workgroup's bound: no wave has a record to write.
    if (kSplit && r_begin >= blk_hi) return;
    int64_t j_begin = r_begin;
    int64_t j_end = blk_hi;
    if (kSplit && j_begin + p.split_len < j_end) j_end = j_begin + p.split_len;
    if (kVar && blk_lo != INT64_MAX && blk_lo > j_begin)   // whole tiles below every row's bound
        j_begin += (blk_lo - j_begin) / kTileN * kTileN;
    const int n_tiles =
        j_end > j_begin ? static_cast<int>((j_end - j_begin + kTileN - 1) / kTileN) : 0;

    const float* kg = static_cast<const float*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const float* vg = static_cast<const float*>(p.v) + b * p.vs.sb + g * p.vs.sh;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, kv_len * p.ks.sr * 4);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, kv_len * p.vs.sr * 4);

    // Tile loads: float f of a tile buffer is key f / kRowF, column
    // f % kRowF; columns >= D and keys past the length load as zeros.  With
    // rows of whole, 16-byte aligned float4s (vec), lane l of DMA row i
    // loads floats 4 (i * 64 + l) .. + 3 (the last row runs into the buffer's
    // padding); else 4-byte loads, float i * 64 + l.  DMA rows i = w, w + 4,
    // ... are this wave's.
    auto dma = [&](int tile, int buf) {
        const int64_t key0 = j_begin + static_cast<int64_t>(tile) * kTileN;
        if (vec & 1) {
            for (int i = w; i < CF::kLoads16; i += kWavesF) {
                const int f = 4 * (i * 64 + lane);
                const int r = f / CF::kRowF, cc = f % CF::kRowF;
                const int64_t key = key0 + r;
                const bool in = r < kTileN && cc < D && key < kv_len;
                const uint32_t ko = in ? static_cast<uint32_t>((key * p.ks.sr + cc) * 4) : kOutOfRange;
                const uint32_t vo = in ? static_cast<uint32_t>((key * p.vs.sr + cc) * 4) : kOutOfRange;
                load_lds16(krs,
                           static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                               (__attribute__((address_space(3))) float*)(&k_sh[buf][i * 256]))),
                           ko);
                load_lds16(vrs,
                           static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                               (__attribute__((address_space(3))) float*)(&v_sh[buf][i * 256]))),
                           vo);
            }
            return;
        }
        for (int i = w; i < CF::kLoads; i += kWavesF) {
            const int f = i * 64 + lane;
            const int r = f / CF::kRowF, cc = f % CF::kRowF;
            const int64_t key = key0 + r;
            const bool in = cc < D && key < kv_len;
            const uint32_t ko = in ? static_cast<uint32_t>((key * p.ks.sr + cc) * 4) : kOutOfRange;
            const uint32_t vo = in ? static_cast<uint32_t>((key * p.vs.sr + cc) * 4) : kOutOfRange;
            load_lds4(krs,
                      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                          (__attribute__((address_space(3))) float*)(&k_sh[buf][i * 64]))),
                      ko);
            load_lds4(vrs,
                      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                          (__attribute__((address_space(3))) float*)(&v_sh[buf][i * 64]))),
                      vo);
        }
    };
    if (n_tiles > 0) dma(0, 0);

    // Q columns hh * DP/2 + t of this lane's row, zeros past D.  With rows
    // of whole, 16-byte aligned float4s (vec bit 1): 16-byte loads, each
    // instruction touching a quarter as many cache lines as 4-byte loads.
    float q[CF::kHalf];
    {
        const float* src = static_cast<const float*>(p.q) + b * p.qs.sb + h * p.qs.sh +
                           (row_ok ? row : 0) * p.qs.sr;
        // Every load unconditional (column clamped into the row, the value
        // zeroed after), so none waits behind a branch.
        if (vec & 2) {
#pragma unroll
            for (int t = 0; t < CF::kHalf; t += 4) {
                const int d = hh * CF::kHalf + t;
                const float4 v = *reinterpret_cast<const float4*>(src + (d < D ? d : 0));
                const bool in = row_ok && d < D;
                q[t] = in ? v.x : 0.f;
                q[t + 1] = in ? v.y : 0.f;
                q[t + 2] = in ? v.z : 0.f;
                q[t + 3] = in ? v.w : 0.f;
            }
        } else {
#pragma unroll
            for (int t = 0; t < CF::kHalf; ++t) {
                const int d = hh * CF::kHalf + t;
                const float v = src[d < D ? d : 0];
                q[t] = (row_ok && d < D) ? v : 0.f;
            }
        }
    }
    const float* mrow = (kMask && row_ok) ? p.mask + b * p.ms.sb + h * p.ms.sh + row * p.ms.sr
                                          : nullptr;

    // Score units: raw q.k without a mask; natural (scale * q.k + mask, the
    // mask added as given, so a large finite value stays finite) with one.
    const float c = kMask ? kLog2e : p.scale_log2;   // score units -> base 2
    const float to_nat = kMask ? 1.f : p.scale;       // score units -> natural
    const float slack = kSlack / c;
    const bool cap = kVar && p.softcap > 0.f;
    const float cap_k2 = cap ? 2.f * kLog2e * p.scale / p.softcap : 0.f;
    const float cap_back = cap ? p.softcap / p.scale : 0.f;
    float m_ref = kNegInf, l_sum = 0.f;
    f32x16 acc[CF::kBlk];
#pragma unroll
    for (int j = 0; j < CF::kBlk; ++j) acc[j] = f32x16{};

    // The Q loads are complete before the loop: left pending, the compiler's
    // wait for them at their first use inside the loop would wait, on every
    // tile, for the next tile's loads too.
#pragma unroll
    for (int t = 0; t < CF::kHalf; ++t) asm volatile("" ::"v"(q[t]));
    dma_wait_all();
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int buf = tile & 1;
        // With a mask, the next tile's loads go out after this tile's mask
        // values are in: the wait for those (the compiler's, which counts
        // only its own loads) would otherwise wait for the tile loads too.
        if (!kMask && tile + 1 < n_tiles) dma(tile + 1, buf ^ 1);
        const int64_t j0 = j_begin + static_cast<int64_t>(tile) * kTileN;
        // Matrix work only if one of the wave's rows sees a key of the tile.
        if (j0 < w_hi && (!kVar || j0 + kTileN > w_lo)) {
            float mv[16];
            if (kMask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = j0 + key_of(r, hh);
                    mv[r] = (mrow && key < row_hi) ? mrow[key] : 0.f;
                }
            }
            // -- S^T = K Q^T: one accumulation chain (dependent fp32 matrix
            // ops issue back to back at full rate on gfx950).
            f32x16 s = f32x16{};
            const float* krow = &k_sh[buf][col * CF::kRowF + hh * CF::kHalf];
#pragma unroll
            for (int u = 0; u < CF::kHalf / 4; ++u) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 4 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], q[4 * u + e], s, 0, 0, 0);
            }

            // -- score rule: softcap on the raw score, the mask, visibility.
            if (cap) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = softcap_raw(s[r], cap_k2, cap_back);
            }
            if (kMask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], p.scale, mv[r]);
            }
            const bool partial = (j0 + kTileN > row_hi) || (kVar && j0 < row_lo);
            if (__builtin_amdgcn_ballot_w64(partial)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = j0 + key_of(r, hh);
                    if (key >= row_hi || (kVar && key < row_lo)) s[r] = kNegInf;
                }
            }
            // -- online normaliser (lazy reference), this tile's p and sum.
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = max_nan(mx, max_nan(s[r], s[r + 1]));
            mx = halves_max(mx);
            const bool raise = mx > m_ref + slack;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float m_new = raise ? mx : m_ref;
                const float alpha = raise ? fast_exp2((m_ref - m_new) * c) : 1.f;   // 0 from -inf
                l_sum *= alpha;
#pragma unroll
                for (int j = 0; j < CF::kBlk; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] *= alpha;
                m_ref = m_new;
            }
            // (s - m) * c: exact 0 for the row maximum, so its weight is 1.
            const float base = (m_ref == kNegInf) ? 0.f : m_ref;
            float tl = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = fast_exp2((s[r] - base) * c);
                tl += s[r];
            }
            l_sum += tl;
            if (kMask && tile + 1 < n_tiles) dma(tile + 1, buf ^ 1);
            // -- O^T += V^T P^T per 32-column block, each tile's into a
            // zero-started partial.
#pragma unroll
            for (int j = 0; j < CF::kBlk; ++j) {
                f32x16 t = f32x16{};
                const float* vcol = &v_sh[buf][32 * j + col];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    t = __builtin_amdgcn_mfma_f32_32x32x2f32(vcol[key_of(r, hh) * CF::kRowF], s[r],
                                                             t, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][r] += t[r];
            }
        } else if (kMask && tile + 1 < n_tiles) {
            dma(tile + 1, buf ^ 1);   // a wave with no work in this tile
        }
        // The next tile's loads have landed in every wave before any wave
        // reads them, and this tile's buffer is free for the loads after next.
        dma_wait_all();
        __syncthreads();
    }

    if (!row_ok) return;
    // Lane l holds columns 32 j + 8 (r/4) + 4 hh + r%4 of its row.
    const float l_tot = halves_sum(l_sum);
    if (kSplit) {
        if (r_begin >= w_hi) return;     // past the wave's bound: the merge reads no record
        float* rec = static_cast<float*>(p.ws) +
                     (((static_cast<int64_t>(b) * p.Hq + h) * p.Lq + row) * p.n_split + rng) *
                         (DP + 4);
#pragma unroll
        for (int j = 0; j < CF::kBlk; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<float4*>(rec + 4 + 32 * j + 8 * u + 4 * hh) =
                    make_float4(acc[j][4 * u], acc[j][4 * u + 1], acc[j][4 * u + 2],
                                acc[j][4 * u + 3]);
        if (hh == 0) {
            rec[0] = m_ref;
            rec[1] = l_tot;
        }
        return;
    }
    float m_nat = m_ref * to_nat;          // natural units (-inf stays -inf)
    float l_f = l_tot;
    const float fs = fold_sink(p, h, m_nat, l_f);
    const bool empty = (l_f == 0.f);
    const float inv = fs / l_f;
    const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
    float* og = static_cast<float*>(p.o) + b * p.os.sb + h * p.os.sh + row * p.os.sr;
    if (vec & 2) {   // registers 4u .. 4u + 3 hold four consecutive columns
#pragma unroll
        for (int j = 0; j < CF::kBlk; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int d = 32 * j + key_of(4 * u, hh);
                if (d < D)
                    *reinterpret_cast<float4*>(og + d) =
                        empty ? make_float4(fill, fill, fill, fill)
                              : make_float4(acc[j][4 * u] * inv, acc[j][4 * u + 1] * inv,
                                            acc[j][4 * u + 2] * inv, acc[j][4 * u + 3] * inv);
            }
    } else {
#pragma unroll
        for (int j = 0; j < CF::kBlk; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = 32 * j + key_of(r, hh);
                if (d < D) og[d] = empty ? fill : acc[j][r] * inv;
            }
    }
    if (p.lse && hh == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh + row * p.ls.sr] = empty ? kNegInf : row_lse(m_nat, l_f);
}

// The head dim a problem runs at.
int f32_padded(int D) {
    return D <= 32 ? 32 : (D <= 64 ? 64 : (D <= 96 ? 96 : (D <= 128 ? 128 : 256)));
}

// Heads per workgroup: the most of 4, 2, 1 that divides the group.
int f32_heads_per_wg(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

int f32_n_qblk(int Lq, int gw) {
    const int P = 32 * (kWavesF / gw);
    return (Lq + P - 1) / P;
}

// One wave per (b, h, row), lanes over the head dim: merge the ranges the
// row's wave wrote, in order, then the sink, the masked-row policy and the
// LSE as the main kernel's epilogue does.  Records are in the main kernel's
// score units: c converts a difference of them to base 2, to_nat a value to
// natural units.
template <int DP>
__global__ __launch_bounds__(256) void prefill_f32_merge_kernel(Params p, float c, float to_nat) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (b, h, i)
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * p.Lq;
    if (row >= rows) return;
    const int64_t i = row % p.Lq;
    const int h = static_cast<int>((row / p.Lq) % p.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(p.Lq) * p.Hq));
    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    // The ranges below the causal bound of the row's wave (its 32 positions)
    // are the ones that wave wrote.
    int64_t blk_hi = kv_len;
    if (p.causal) {
        const int64_t last = ((i / 32 + 1) * 32 < p.Lq ? (i / 32 + 1) * 32 : p.Lq) - 1;
        const int64_t bb = last + causal_delta(p, kv_len) + 1;
        blk_hi = bb < 0 ? 0 : (bb < blk_hi ? bb : blk_hi);
    }
    const int n_live = static_cast<int>((blk_hi + p.split_len - 1) / p.split_len);
    const float* recs = static_cast<const float*>(p.ws) + row * p.n_split * (DP + 4);
    constexpr int NPL = (DP + 63) / 64;              // head-dim values per lane
    // Eight ranges' (m, l, acc) are fetched per round; the reference maximum
    // is the largest seen so far, so up to eight ranges fold in one round
    // exactly as a separate maximum pass would.
    float M = kNegInf, L = 0.f, A[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) A[k] = 0.f;
    for (int r0 = 0; r0 < n_live; r0 += 8) {
        float m8[8], l8[8], a8[8][NPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = r0 + u < n_live;
            const float* rec = recs + (in ? r0 + u : 0) * (DP + 4);
            m8[u] = in ? rec[0] : kNegInf;
            l8[u] = in ? rec[1] : 0.f;
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                const int d = lane + 64 * k;
                a8[u][k] = (in && d < p.D) ? rec[4 + d] : 0.f;
            }
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, m8[u]);
        if (Mn != M) {   // raise the reference (from -inf: nothing folded yet)
            const float al = (M == kNegInf) ? 0.f : fast_exp2((M - Mn) * c);
            L *= al;
#pragma unroll
            for (int k = 0; k < NPL; ++k) A[k] *= al;
            M = Mn;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (r0 + u >= n_live) break;
            const float f = (m8[u] == kNegInf) ? 0.f : fast_exp2((m8[u] - M) * c);
            L = fmaf(l8[u], f, L);
#pragma unroll
            for (int k = 0; k < NPL; ++k) A[k] = fmaf(a8[u][k], f, A[k]);
        }
    }
    float m_nat = M * to_nat;
    const float fs = fold_sink(p, h, m_nat, L);
    const bool empty = (L == 0.f);
    const float inv = fs / L;
    const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
    float* og = static_cast<float*>(p.o) + b * p.os.sb + h * p.os.sh + i * p.os.sr;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
        const int d = lane + 64 * k;
        if (d < p.D) og[d] = empty ? fill : A[k] * inv;
    }
    if (p.lse && lane == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = empty ? kNegInf : row_lse(m_nat, L);
}

bool f32_var(const Params& p) {
    return p.softcap > 0.f || (p.causal && p.window > 0) || p.doc_start || p.sink;
}

template <int DP>
hipError_t launch_d(const Params& p, hipStream_t s) {
    // 16-byte tile loads when every K and V row starts 16-byte aligned and
    // holds whole float4s.
    auto al = [](const void* ptr, const Strides& st) {
        return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && st.sb % 4 == 0 && st.sh % 4 == 0 &&
               st.sr % 4 == 0;
    };
    // Bit 0: K/V rows; bit 1: Q and O rows (16-byte loads and stores).
    const int vec = (p.D % 4 == 0 && (p.Lk == 0 || (al(p.k, p.ks) && al(p.v, p.vs))) ? 1 : 0) |
                    (p.D % 4 == 0 && al(p.q, p.qs) && al(p.o, p.os) ? 2 : 0);
    const int gw = f32_heads_per_wg(p.group);
    const int n_qblk = f32_n_qblk(p.Lq, gw);
    const dim3 grid(n_qblk, p.Hkv * (p.group / gw), p.B * p.n_split);
    const bool split = p.n_split > 1;
    auto go = [&](auto mask_c, auto split_c, auto var_c) {
        constexpr bool kM = decltype(mask_c)::value, kS = decltype(split_c)::value;
        constexpr bool kV = decltype(var_c)::value;
        hipLaunchKernelGGL((prefill_f32_kernel<DP, kM, kS, kV>), grid, dim3(64 * kWavesF), 0, s,
                           p, n_qblk, gw, vec);
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
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * p.Lq;
    const float c = p.mask ? kLog2e : p.scale_log2, to_nat = p.mask ? 1.f : p.scale;
    hipLaunchKernelGGL((prefill_f32_merge_kernel<DP>),
                       dim3(static_cast<uint32_t>((rows + 3) / 4)), dim3(256), 0, s, p, c,
                       to_nat);
    return hipGetLastError();
}

}  // namespace

// Key ranges for the fp32 kernel: only when the workgroups are fewer than
// two per CU and the keys span at least four tiles; ranges are multiples of
// 64 keys, at least 3 and at most 32 of them.
void prefill_f32_plan(int B, int Hq, int Hkv, int Lq, int Lk, int D, int* split_len,
                      int* n_split) {
    (void)D;
    const int group = (Hkv > 0 && Hq % Hkv == 0) ? Hq / Hkv : 1;
    const int gw = f32_heads_per_wg(group);
    const int64_t wgs = static_cast<int64_t>(f32_n_qblk(Lq, gw)) * (Hq / gw) * B;
    int n = 1;
    const int64_t target = 512;
    if (wgs > 0 && wgs < target && Lk >= 4 * kTileN) {
        const int64_t want = (target + wgs - 1) / wgs;
        const int64_t most = Lk / kRangeQuantum;
        n = static_cast<int>(want < most ? want : most);
        if (n > 32) n = 32;
        // Two ranges do not pay for their records and merge (measured: MiniLM
        // B8 S128 10.4 us whole against 15.9 us in two ranges, BERT-base B8
        // S512 84.6 against 90.7); from three on the added workgroups do.
        if (n < 3) n = 1;
    }
    int len = (Lk + n - 1) / n;
    len = (len + kRangeQuantum - 1) / kRangeQuantum * kRangeQuantum;
    if (len < kRangeQuantum) len = kRangeQuantum;
    *split_len = len;
    *n_split = Lk > 0 ? (Lk + len - 1) / len : 1;
    if (*n_split < 1) *n_split = 1;
}

size_t prefill_f32_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D) {
    int len, n;
    prefill_f32_plan(B, Hq, Hkv, Lq, Lk, D, &len, &n);
    if (n <= 1) return 0;
    return static_cast<size_t>(B) * Hq * Lq * n * (f32_padded(D) + 4) * sizeof(float);
}

bool prefill_f32_supported(const Params& p, DType dt) {
    if (dt != DType::F32) return false;
    if (p.D < 1 || p.D > 256) return false;
    const int gw = f32_heads_per_wg(p.group);
    // Buffer resources and their offsets are 32-bit: one (batch, kv head)
    // slice of K and of V must span less than 2 GiB.
    const int64_t lim = INT32_MAX;
    if (static_cast<int64_t>(p.Lk) * p.ks.sr * 4 >= lim) return false;
    if (static_cast<int64_t>(p.Lk) * p.vs.sr * 4 >= lim) return false;
    return static_cast<int64_t>(p.Hkv) * (p.group / gw) <= 65535 &&
           static_cast<int64_t>(p.B) * p.n_split <= 65535;
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
