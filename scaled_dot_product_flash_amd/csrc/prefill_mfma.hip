// prefill_mfma.hip -- fused attention for bf16 / fp16 inputs with fp32
// accumulation on the gfx950 matrix cores, head dims 1..256 (padded to 64,
// 128 or 256; a head dim that is not a multiple of 8 first has its K/V rows
// staged into the workspace as copies padded to one).
//
// Work decomposition.  A workgroup of W waves (8 for head dim 128, else 4;
// see Cfg) owns one (batch, kv head) and 32 W query rows that read it: gw
// query heads of the group (gw = 8, 4, 2 or 1, the largest that divides
// Hq/Hkv and is at most W) times 32 W / gw consecutive positions.  Each wave
// owns 32 rows of one head.  One K/V tile load thus serves every query head of
// the group that shares it (llm.istanbul "05_attention", "GQA").  The keys are
// visited in increasing order, 64 per tile, staged through LDS (one barrier
// per tile) by coalesced 16-byte raw-buffer loads that write LDS directly,
// with no register round trip; the buffer's range ends at the batch entry's
// key length, so rows past it arrive as zeros and are never fetched.
// (OneGPU "Attention", introduction and "Variants and ordering": a workgroup
// keeps a block of query rows and walks key/value tiles held in workgroup
// memory.)  When the query blocks would leave half of the GPU idle, each
// block's keys are cut into ranges whose partial records a second kernel
// merges in range order (OneGPU "Attention", "Accuracy at long key lengths").
// Workgroups run heaviest causal block first, or, without causality but with
// key lengths, longest batch entry first.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
// output column is the query, so lane l owns query l%32 and holds 16 of its
// keys per 32-key block; lane l^32 holds the other 16.  A row's maximum is an
// in-lane reduction plus one lane swap with lane l^32 (OneGPU "Apple simdgroup
// kernel": scores transposed so one lane keeps one row).
//
// Online normaliser (OneGPU "Attention", introduction; llm.istanbul
// "05_attention", "Online Softmax Algoritmasi").  Without a mask the scores
// stay raw (s = q.k): with c = scale*log2(e), p = exp2(s*c - m*c) is one FMA
// and one exp2 per score.  With a mask they are natural, s = scale*q.k +
// mask (one FMA, the mask added as given), and c = log2(e): folding the mask
// into raw units instead (mask / scale) would turn a large finite mask value
// into -inf.  The reference maximum m is raised lazily, only when a tile's
// maximum exceeds it by more than 8/c (so p <= 2^8), and the accumulators are
// rescaled only then (OneGPU "Apple simdgroup kernel", reference maximum).
// Raising is a per-row decision taken identically in both lanes of the row.
//
// P is rounded to the element type before the P V product, and the running
// sum is the sum of the ROUNDED values, so numerator and denominator see the
// same p (OneGPU "Matrix hardware"): one v_dot2 of each packed pair with
// (1, 1) adds both rounded values exactly.
// O^T = V^T P^T: the rounded scores are already in the B-operand layout, and
// the V^T operand is read from the row-major V tile with ds_read_b64_tr_b16.
//
// Element-wise work that only some tiles need (the causal diagonal, the tile
// holding the key length, the lower edge of a local window, the additive
// mask) is done only on those tiles; the mask, the window / softcap /
// document rules (with padded head dims), the short-row shape, the key-range
// split and the length order are compile-time variants of the kernel, so a
// kernel carries only the code it runs.  Score-rule variants follow the ONNX
// GroupQueryAttention README ("Attributes", "Inputs"): a local window starts
// the key loop at the block's first visible tile; the softcap maps each raw
// score before the mask is added; the sink joins the denominator at the end.
//
// Special values (OneGPU "Special values"): hidden keys get -inf and weigh 0;
// a row whose reference max is still -inf uses 0 as the exponent base, so
// exp2(-inf) = 0 and never exp2(-inf - -inf); a row with no visible key ends
// with l == 0 and follows the masked-row policy; NaN / +inf scores make l NaN.
#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"
#include "mfma_common.h"

namespace sdpa {

namespace {

using namespace mfma;

constexpr int kBN = 64;        // keys per tile
constexpr float kSlack = 8.f;  // lazy-rescale threshold, base-2 units

// Floats per partial record of the key-range split: m, l, two pads, then the
// accumulator padded to whole float4.
__host__ __device__ constexpr int record_stride(int D) { return (D + 3) / 4 * 4 + 4; }

// Workgroup shape per padded head dim DP, waves of 32 query rows.  DP = 128:
// 8 waves, two per SIMD (about 205 registers each).  DP = 256: a wave's Q
// operand, accumulators and scores need about 300 registers, so 4 waves (one
// per SIMD, 512 registers each).  DP = 64: under 170 registers a wave, so
// workgroups of 4 waves, three per CU -- three waves per SIMD hide more of the
// exponentials, which weigh twice as much against the matrix work at this
// head dim.  kShort (DP = 128 under a local window or document starts, where
// each workgroup walks few key tiles): 4 waves, two workgroups per CU, so one
// workgroup's prologue and epilogue overlap the other's tiles.  A head dim
// D < DP that is a multiple of 8 runs padded: columns d >= D load as zeros
// and are not stored.
template <int DP, bool kShort = false> struct Cfg {
    static constexpr int kWaves = (DP == 128 && !kShort) ? 8 : 4;
    static constexpr int kMinBlocks =
        DP == 64 ? 3 : (DP == 128 && kShort ? 2 : 1);   // resident workgroups per CU
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRows = 32 * kWaves;   // query rows (all heads) per workgroup
};

// LDS tile layout.  K/V tiles go from HBM straight into LDS (buffer loads
// with the LDS destination): one wave load writes 64 lanes x 16 bytes = 1 KiB
// contiguously, lane l at byte 16 l of its block.  A 64-row tile is cut into
// NB = D/8 such blocks, and block I holds the rows r with r % NB == I, so
// consecutive rows land in different blocks.  K rows are read 16 lanes x 16
// bytes down one column: blocks padded to 1040 bytes put consecutive rows 16
// bytes mod 256 apart, over all banks.  V rows are read by the transpose
// load, 4 rows x 64 bytes per 32 lanes: blocks padded to 1088 bytes put them
// 64 bytes mod 256 apart.
template <int D> struct Tile {
    static constexpr int NB = D / 8;                          // blocks = chunks per row
    static constexpr int KB = 1040, VB = 1088;                // block strides (bytes)
    static constexpr int RB = 2 * D;                          // row bytes
};

// Staging plan per padded head dim.  K tiles rotate over NK LDS buffers and
// V tiles over NV (tile t uses buffer (t - first tile) mod NK, resp. NV); K
// is loaded DK tiles ahead and V DV tiles ahead.  A buffer is refilled only
// after the barrier that ends the last iteration reading it: that needs
// DV <= NV - 1 and DK <= NK - 1, except that D = 256, with room for two K
// buffers only, loads K two ahead into the buffer the prologue's score reads
// used and puts a barrier after those reads.
//
// kAsm: the loads are issued as instructions the compiler does not see into
// (see load_lds16), so it does not hold every later LDS read for them and the
// loads overlap the next tile's work; the kernel then waits for exactly the
// loads the next tile needs.  kTop: the loads are issued at the top of the
// iteration (else after its mask reads).  D = 128 and 256 run with kAsm and
// deep prefetch; D = 64 (three workgroups per CU, little LDS each) measured
// best with compiler-visible loads at the top of the iteration.
template <int D, bool kShort = false> struct Stage;
template <> struct Stage<64> {
    static constexpr int NK = 3, NV = 2, DK = 2, DV = 1;
    static constexpr bool kPrologueBarrier = false, kAsm = false, kTop = true;
};
template <> struct Stage<128> {
    static constexpr int NK = 4, NV = 4, DK = 3, DV = 3;
    static constexpr bool kPrologueBarrier = false, kAsm = true, kTop = false;
};
template <> struct Stage<256> {
    static constexpr int NK = 2, NV = 2, DK = 2, DV = 1;
    static constexpr bool kPrologueBarrier = true, kAsm = true, kTop = false;
};
// Two workgroups per CU leave each 80 KiB: two buffers per tensor.
template <> struct Stage<128, true> {
    static constexpr int NK = 2, NV = 2, DK = 2, DV = 1;
    static constexpr bool kPrologueBarrier = true, kAsm = true, kTop = false;
};

// One 16-byte-per-lane buffer load into LDS at lds_byte + 16 * lane (the
// LDS address goes through M0; one wait state after writing M0).  Written as
// an instruction of its own so that the compiler, which cannot tell which LDS
// bytes such a load writes, does not hold later LDS reads of other buffers
// for it.  The kernel waits for these loads itself (vmcnt, in issue order)
// before the barrier that publishes a tile.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_byte,
                                           uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "{m0}"(lds_byte));
}

// Maximum of the 32 scores a lane holds for its row (NaN-propagating), as a
// tree of three-way maxima four levels deep.
__device__ __forceinline__ float row_max32(const f32x16 (&s)[2]) {
    float a[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const int j = 3 * i;   // values j, j+1, j+2 of the 32 (kb = j / 16)
        a[i] = max_nan(max_nan(s[j / 16][j % 16], s[(j + 1) / 16][(j + 1) % 16]),
                       s[(j + 2) / 16][(j + 2) % 16]);
    }
    a[10] = max_nan(s[1][14], s[1][15]);
    const float b0 = max_nan(max_nan(a[0], a[1]), a[2]), b1 = max_nan(max_nan(a[3], a[4]), a[5]);
    const float b2 = max_nan(max_nan(a[6], a[7]), a[8]), b3 = max_nan(a[9], a[10]);
    return max_nan(max_nan(b0, b1), max_nan(b2, b3));
}

// kSplit: the workgroup covers one key range and writes partial records.
// kOrder: workgroups take their units longest batch entry first (non-causal
// problems with per-entry key lengths).  Both are compile-time variants, so
// kernels without them carry none of their code (which would change the
// register allocation and schedule of the tile loop).
template <bool kBf16, int D, bool kMask, bool kVar, bool kShort, bool kSplit, bool kOrder>
__global__ __launch_bounds__((Cfg<D, kShort>::kThreads), (Cfg<D, kShort>::kMinBlocks)) void
prefill_mfma_kernel(
    Params p, int n_qblk, int gw, int xcd_units, int mask_vec4) {
    using M = Mma<kBf16>;
    using TL = Tile<D>;
    using CF = Cfg<D, kShort>;
    constexpr int kRows = CF::kRows, kWaves = CF::kWaves, kThreads = CF::kThreads;
    // True head dim (<= D).  Padded dims run the variant kernel; in the plain
    // one it is the compile-time D and the column guards below fold away.
    const int Dt = kVar ? p.D : D;
    // K/V columns per row: a head dim that is not a multiple of 8 reads
    // copies padded to one (zeros past Dt), staged into the workspace first;
    // its Q rows are then read and O rows written without 16-byte accesses
    // (see the row staging below).
    const int Dkv = kVar ? (p.D + 7) & ~7 : D;
    const bool elem = kVar && (p.D & 7) != 0;
    constexpr int NT = D / 16;   // 16-wide d-steps of the score product
    constexpr int ND = D / 32;   // 32-row d-tiles of the output
    constexpr int NB = TL::NB, KB = TL::KB, VB = TL::VB, RB = TL::RB;
    using SP = Stage<D, kShort>;
    static_assert(SP::DV <= SP::NV - 1, "a V buffer would be refilled while read");
    static_assert(SP::DK <= SP::NK - 1 || (SP::DK == SP::NK && SP::kPrologueBarrier),
                  "a K buffer would be refilled while read");
    __shared__ __attribute__((aligned(16))) uint8_t k_sh[SP::NK][NB * KB];
    __shared__ __attribute__((aligned(16))) uint8_t v_sh[SP::NV][NB * VB];

    // ---- which (b, kv head, key range, head slice, query block) this
    // workgroup owns.  Heaviest causal blocks first; without causality but
    // with per-entry key lengths, longest entries first (below).  Units are
    // (batch, kv head, key range) triples; without a key-range split there is
    // one range.
    // When the units split evenly over the 8 XCDs (consecutive workgroups go
    // to consecutive XCDs), each XCD keeps whole units, so the workgroups
    // reading the same K/V tiles share its L2.
    const int n_slice = p.group / gw;           // head slices per kv head
    const int ns = kSplit ? p.n_split : 1;
    int b, g, slice, qb, rng;
    if constexpr (kOrder) {
        // Non-causal rows with per-entry key lengths: every query block of an
        // entry costs about its length, so the units go longest entry first
        // (dealt round-robin over the XCDs), the query blocks inside a unit.
        const int L = blockIdx.x;
        const int per_unit = n_qblk * n_slice;
        int k, rem;
        if (xcd_units > 0) {
            const int xcd = L & 7, slot = L >> 3;
            k = (slot / per_unit) * 8 + xcd;
            rem = slot % per_unit;
        } else {
            k = L / per_unit;
            rem = L % per_unit;
        }
        qb = n_qblk - 1 - rem / n_slice;
        slice = rem % n_slice;
        // Rank of each entry by clamped length, longest first, ties by index.
        const int ln = threadIdx.x & 63;
        auto clamped = [&](int j) {
            const int64_t v = p.lens[j];
            return v < 0 ? int64_t(0) : (v > p.Lk ? int64_t(p.Lk) : v);
        };
        const int64_t li = ln < p.B ? clamped(ln) : -1;
        int rank = 0;
        for (int j = 0; j < p.B; ++j) {
            const int64_t lj = clamped(j);
            rank += (lj > li) || (lj == li && j < ln);
        }
        const int br = k / (p.Hkv * ns);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(ln < p.B && rank == br);
        b = static_cast<int>(__builtin_ctzll(hit));
        g = (k / ns) % p.Hkv;
        rng = k % ns;
    } else {
        const int L = blockIdx.x;
        int unit;
        if (xcd_units > 0) {
            const int xcd = L & 7, slot = L >> 3;
            const int per = xcd_units * n_slice;
            qb = n_qblk - 1 - slot / per;
            const int rem = slot % per;
            unit = xcd * xcd_units + rem / n_slice;
            slice = rem % n_slice;
        } else {
            const int per = p.B * p.Hkv * ns * n_slice;
            qb = n_qblk - 1 - L / per;
            const int rem = L % per;
            unit = rem / n_slice;
            slice = rem % n_slice;
        }
        rng = unit % ns;
        b = unit / ns / p.Hkv;
        g = unit / ns % p.Hkv;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hh = lane >> 5;          // which half of the wave
    const int col = lane & 31;         // query column owned by this lane
    const int rows_per_head = kRows / gw;
    const int waves_per_head = rows_per_head / 32;
    const int h = g * p.group + slice * gw + w / waves_per_head;

    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const int64_t delta = causal_delta(p, kv_len);
    const int64_t q0 = static_cast<int64_t>(qb) * rows_per_head;
    const int64_t qw0 = q0 + 32 * (w % waves_per_head);
    // Keys the block needs: [0, blk_hi); keys this wave can see: [0, wave_hi).
    int64_t blk_hi = kv_len, wave_hi = kv_len;
    if (p.causal) {
        const int64_t last = (q0 + rows_per_head < p.Lq ? q0 + rows_per_head : p.Lq) - 1;
        const int64_t bb = last + delta + 1;
        blk_hi = bb < 0 ? 0 : (bb < blk_hi ? bb : blk_hi);
        const int64_t wl = (qw0 + 32 < p.Lq ? qw0 + 32 : p.Lq) - 1;
        const int64_t wb = wl + delta + 1;
        wave_hi = wb < 0 ? 0 : (wb < wave_hi ? wb : wave_hi);
    }
    if (qw0 >= p.Lq) wave_hi = 0;
    int n_tiles = static_cast<int>((blk_hi + kBN - 1) / kBN);
    // Under a local window the block's first row sees the lowest keys, and a
    // tile below the wave's last row's window edge needs the element test.
    // Lower key bounds (local window, document starts; variant kernel only):
    // row_lo for this lane's row, wave_lo the largest in the wave (tiles below
    // it need the element test) and the block's smallest, which sets the first
    // tile -- blocks of keys before every row's bound are skipped (llm.istanbul
    // "05_attention", "K-block iteration").
    const int64_t qrow = qw0 + col;
    int64_t row_lo = 0, wave_lo = 0;
    int t_first = 0;
    if (kVar) {
        __shared__ int blk_min[kWaves];
        const bool ok = qrow < p.Lq;
        row_lo = ok ? first_key(p, b, qrow, delta) : 0;
        int mn = ok ? static_cast<int>(row_lo < kv_len ? row_lo : kv_len) : INT32_MAX;
        int mx = static_cast<int>(row_lo < kv_len ? row_lo : kv_len);
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) {
            mn = min(mn, __shfl_xor(mn, off, 64));
            mx = max(mx, __shfl_xor(mx, off, 64));
        }
        wave_lo = mx;
        if (lane == 0) blk_min[w] = mn;
        __syncthreads();
        int bm = INT32_MAX;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) bm = min(bm, blk_min[i]);
        t_first = bm == INT32_MAX ? n_tiles : bm / kBN;
    }

    if (kSplit) {   // this workgroup's key range: tiles [r_lo, r_hi)
        const int r_lo = rng * (p.split_len / kBN), r_hi = r_lo + p.split_len / kBN;
        t_first = t_first > r_lo ? t_first : r_lo;
        n_tiles = n_tiles < r_hi ? n_tiles : r_hi;
    }

    const uint16_t* qg = static_cast<const uint16_t*>(p.q);
    const uint16_t* kg = static_cast<const uint16_t*>(p.k) + b * p.ks.sb + g * p.ks.sh;
    const uint16_t* vg = static_cast<const uint16_t*>(p.v) + b * p.vs.sb + g * p.vs.sh;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, kv_len * p.ks.sr * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, kv_len * p.vs.sr * 2);

    // ---- Q^T operand, resident in registers -------------------------------
    // Rows whose length is not a multiple of 8 elements (no 16-byte access
    // applies).  D >= 128: Q comes in and O goes out through LDS, each wave
    // owning 32 rows of D elements at the front of the K buffers, free before
    // the first tile loads and after the last tile's barrier; global accesses
    // then go one row at a time with lanes over consecutive columns
    // (c = lane + 64 k), instead of each lane walking its own row, where
    // per-lane 2-byte accesses down 32 rows cost a memory transaction per
    // lane per instruction.  D = 64 (three workgroups per CU at the register
    // cap, where the staging code's registers would spill inside the tile
    // loop): per-lane element accesses, all Q loads issued before any is used.
    constexpr bool kRowStage = D >= 128;
    static_assert(!kRowStage || kRows * D * 2 <= SP::NK * NB * KB, "the row-staging area does not fit");
    uint16_t* const xrow = reinterpret_cast<uint16_t*>(&k_sh[0][0]) + w * 32 * D;
    constexpr int kColIt = D / 64;   // column steps of 64 per row

    // ---- Q^T operand, resident in registers -------------------------------
    i16x8 qop[NT];
    {
        const bool ok = qrow < p.Lq;
        if (elem && !kRowStage) {
            const uint16_t* row = qg + b * p.qs.sb + h * p.qs.sh + (ok ? qrow : 0) * p.qs.sr;
            short e16[NT][8];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 16 * t + 8 * hh + e;   // clamped into the row, zeroed below
                    e16[t][e] = static_cast<short>(row[c < Dt ? c : Dt - 1]);
                }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                i16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (ok && 16 * t + 8 * hh + e < Dt) ? e16[t][e] : short(0);
                qop[t] = v;
            }
        } else if (elem) {
            // Every load issued before any is stored, none conditional: the
            // row and column are clamped into the tensor and the values
            // outside it are zeroed when the operand is read back.
            // Sixteen rows per round (registers for 32 rows would spill).
            const uint16_t* qb = qg + b * p.qs.sb + h * p.qs.sh;
#pragma unroll
            for (int r0 = 0; r0 < 32; r0 += 16) {
                short qv[16][kColIt];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t qr = qw0 + r0 + r;
                    const uint16_t* src = qb + (qr < p.Lq ? qr : p.Lq - 1) * p.qs.sr;
#pragma unroll
                    for (int k = 0; k < kColIt; ++k) {
                        const int c = lane + 64 * k;
                        qv[r][k] = static_cast<short>(src[c < Dt ? c : Dt - 1]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int k = 0; k < kColIt; ++k)
                        xrow[(r0 + r) * D + lane + 64 * k] = static_cast<uint16_t>(qv[r][k]);
            }
            // The wave reads back what it wrote (LDS keeps one wave's
            // accesses in order).
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const i16x8 raw = *reinterpret_cast<const i16x8*>(xrow + col * D + 16 * t + 8 * hh);
                i16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (ok && 16 * t + 8 * hh + e < Dt) ? raw[e] : short(0);
                qop[t] = v;
            }
            __syncthreads();   // before any wave's tile loads overwrite the area
        } else {
            const uint16_t* row = qg + b * p.qs.sb + h * p.qs.sh + (ok ? qrow : 0) * p.qs.sr;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bool in = ok && 16 * t + 8 * hh < Dt;   // padded columns are zero
                qop[t] = in ? *reinterpret_cast<const i16x8*>(row + 8 * hh + 16 * t) : i16x8{};
            }
        }
    }

    // ---- staging: HBM -> LDS.  While tile t's softmax and P V run, tile
    // t+1's scores are computed from LDS, and the loads of K(t+DK) and V(t+DV)
    // land in free buffers; before the barrier that ends the tile each wave
    // waits for its own loads that the next tile needs.  Each wave loads NB / kWaves blocks per tensor per tile straight into LDS
    // (lane l fills bytes 16 l .. 16 l + 15 of its block): in block I, lane l
    // holds row I + NB * (l / (D/8)), 16-byte chunk l % (D/8).  Rows past the
    // key length and padded columns (d >= true head dim) read out of the
    // buffer's range, which writes zeros.
    constexpr int kLoadsW = NB / kWaves;
    const int ld_q = lane / (D / 8), ld_c = lane % (D / 8);
    constexpr uint32_t kOutOfRange = 0x7ffffff0u;
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, int64_t sr, uint8_t* buf, int stride, int tile) {
#pragma unroll
        for (int n = 0; n < kLoadsW; ++n) {
            const int I = n * kWaves + w;
            const int key = tile * kBN + I + NB * ld_q;
            const uint32_t off =
                8 * ld_c < Dkv ? static_cast<uint32_t>((key * static_cast<int>(sr) + 8 * ld_c) * 2)
                              : kOutOfRange;
            if constexpr (SP::kAsm)
                load_lds16(rs,
                           static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                               (__attribute__((address_space(3))) uint8_t*)(buf + I * stride))),
                           off);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)(buf + I * stride), 16, off, 0, 0,
                    0);
        }
    };
    auto kbuf = [&](int tile) { return (tile - t_first) % SP::NK; };
    auto vbuf = [&](int tile) { return (tile - t_first) % SP::NV; };
    auto fetch_k = [&](int tile) { dma(krs, p.ks.sr, k_sh[kbuf(tile)], KB, tile); };
    auto fetch_v = [&](int tile) { dma(vrs, p.vs.sr, v_sh[vbuf(tile)], VB, tile); };
    // Waits until at most n of this wave's loads are in flight (vmcnt n;
    // expcnt and lgkmcnt left free).  Loads complete in issue order.
    auto dma_wait_keep = [&](int n) {
        if (n == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
        else if (n == kLoadsW) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsW);
        else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLoadsW));
    };
    // The two 32-key blocks' MFMA chains alternate, so consecutive MFMAs are
    // independent.
    auto scores = [&](int buf, f32x16 (&s)[2]) {
        // Row col + 32 kb: block col % NB, row-in-block col / NB + kb * 32 / NB
        // (kb * 32 / NB rows = 512 bytes), chunk 2 t + hh.
        const uint8_t* krow = &k_sh[buf][(col % NB) * KB + (col / NB) * RB + 16 * hh];
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const i16x8 a = *reinterpret_cast<const i16x8*>(krow + kb * 512 + 32 * t);
                s[kb] = M::mfma(a, qop[t], s[kb]);
            }
        }
    };

    const float* mrow = nullptr;
    if (kMask && qrow < p.Lq) mrow = p.mask + b * p.ms.sb + h * p.ms.sh + qrow * p.ms.sr;
    // Score units: natural with a mask, raw without (see the file comment).
    const float c = kMask ? kLog2e : p.scale_log2;   // score units -> base 2 (> 0)
    const float to_nat = kMask ? 1.f : p.scale;       // score units -> natural
    const float slack = kSlack / c;                   // lazy threshold in score units
    const float sc = p.scale;                         // raw -> natural

    float m_ref = kNegInf;   // reference maximum of this lane's row, raw-score units
    float l_sum = 0.f;       // this lane's share of the sum of rounded p
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x16{};

    // Prologue: K of the first DK tiles and V of the first DV.
    for (int i = 0; i < SP::DK; ++i)
        if (t_first + i < n_tiles) fetch_k(t_first + i);
    for (int i = 0; i < SP::DV; ++i)
        if (t_first + i < n_tiles) fetch_v(t_first + i);
    dma_wait_keep(0);
    __syncthreads();

    f32x16 s_a[2], s_b[2];
    if (t_first < n_tiles) scores(kbuf(t_first), s_a);
    if (SP::kPrologueBarrier) __syncthreads();
    const bool cap = kVar && p.softcap > 0.f;
    const float cap_k2 = cap ? 2.f * kLog2e * p.scale / p.softcap : 0.f;
    const float cap_back = cap ? p.softcap / p.scale : 0.f;

    // One tile; s_cur holds its scores, s_next receives the next tile's.  The
    // loop below runs it twice per trip with the two score sets swapping
    // roles, so no scores are copied between tiles.
    // D = 256 issues the V loads just before P V rather than with the K
    // loads (measured 2.5% faster there; no difference at D = 128).
    constexpr bool kVLate = D == 256;
    auto step = [&](int tile, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
        const bool more_k = tile + SP::DK < n_tiles;
        const bool more_v = tile + SP::DV < n_tiles;
        if (SP::kTop) {
            if (more_k) fetch_k(tile + SP::DK);
            if (more_v) fetch_v(tile + SP::DV);
        }
        const int64_t j0 = static_cast<int64_t>(tile) * kBN;
        const bool sees = j0 < wave_hi;

        // -- softcap on the raw scores, before the mask --
        if (cap) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s_cur[kb][r] = softcap_raw(s_cur[kb][r], cap_k2, cap_back);
        }
        // -- additive mask, folded into raw-score units --
        if (kMask && mrow && sees && mask_vec4 && j0 + kBN <= kv_len) {
            // The whole tile lies inside the length: eight 16-byte loads.
            float4 m4[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    m4[kb][u] = *reinterpret_cast<const float4*>(mrow + j0 + kb * 32 + 8 * u + 4 * hh);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    s_cur[kb][4 * u] = fmaf(s_cur[kb][4 * u], sc, m4[kb][u].x);
                    s_cur[kb][4 * u + 1] = fmaf(s_cur[kb][4 * u + 1], sc, m4[kb][u].y);
                    s_cur[kb][4 * u + 2] = fmaf(s_cur[kb][4 * u + 2], sc, m4[kb][u].z);
                    s_cur[kb][4 * u + 3] = fmaf(s_cur[kb][4 * u + 3], sc, m4[kb][u].w);
                }
        } else if (kMask && mrow && sees) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t key = j0 + kb * 32 + 8 * u + 4 * hh;
                    float mv[4];
                    if (mask_vec4 && key + 3 < kv_len) {
                        const float4 m4 = *reinterpret_cast<const float4*>(mrow + key);
                        mv[0] = m4.x; mv[1] = m4.y; mv[2] = m4.z; mv[3] = m4.w;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) mv[e] = (key + e < kv_len) ? mrow[key + e] : 0.f;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s_cur[kb][4 * u + e] = fmaf(s_cur[kb][4 * u + e], sc, mv[e]);
                }
            }
        }
        // Loads for later tiles (K before V), after this tile's mask reads so
        // that waiting on those does not wait on these.
        if (!SP::kTop) {
            if (more_k) fetch_k(tile + SP::DK);
            if (more_v && !kVLate) fetch_v(tile + SP::DV);
        }
        // -- hide keys past the length / causal bound / below the window
        // (edge tiles only) --
        const bool partial = (j0 + kBN > kv_len) || (p.causal && j0 + kBN - 1 > qw0 + delta) ||
                             (kVar && j0 < wave_lo);
        if (partial) {
            // Score (kb, r) holds key j0 + 4 hh + o, o = 32 kb + 8 (r / 4) + r % 4
            // (a constant below 64): it is visible iff lo <= o < hi, with the
            // lane's key bounds taken relative to j0 + 4 hh and clamped to
            // [0, 64], which changes no comparison and fits 32 bits.
            const int64_t base = j0 + 4 * hh;
            int64_t top = kv_len;
            if (p.causal && qrow + delta + 1 < top) top = qrow + delta + 1;
            const int64_t th = top - base;
            const int hi = static_cast<int>(th < 0 ? 0 : (th > 64 ? 64 : th));
            int lo = 0;
            if (kVar) {
                const int64_t tl = row_lo - base;
                lo = static_cast<int>(tl < 0 ? 0 : (tl > 64 ? 64 : tl));
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o = kb * 32 + 8 * (r >> 2) + (r & 3);
                    if (o >= hi || (kVar && o < lo)) s_cur[kb][r] = kNegInf;
                }
        }

        // -- row maximum: 32 values in-lane (a tree of three-way maxima, four
        // levels deep), then the partner lane --
        float mx = halves_max(row_max32(s_cur));
        // -- lazy raise of the reference maximum --
        const bool raise = mx > m_ref + slack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mx : m_ref;
            // 0 when m_ref = -inf; rows that do not raise keep alpha = 1 exactly.
            const float alpha = raise ? fast_exp2((m_ref - m_new) * c) : 1.f;
            l_sum *= alpha;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
            m_ref = m_new;
        }
        float neg_mc = (m_ref == kNegInf) ? 0.f : -m_ref * c;
        if constexpr (kMask) {
            // A reference far from zero (a large finite mask on every key seen
            // so far): subtract it from the scores first, exactly for scores
            // near it, so the exponent argument neither overflows nor loses
            // the scores' differences in the rounding of m*c.
            const bool far = fabsf(neg_mc) >= 4096.f;
            if (__builtin_amdgcn_ballot_w64(far) && far) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s_cur[kb][r] -= m_ref;
                neg_mc = 0.f;
            }
        }
        // -- next tile's scores on the matrix core while this tile's softmax
        // runs (same basic block, so the two interleave).  After the last tile
        // the buffer holds stale keys and the result is discarded.
        scores(kbuf(tile + 1), s_next);
        // -- p = exp2(s*c - m*c), rounded to the element type; the tile's sum
        // of the rounded p in four independent chains (short dependences) --
        i16x8 pop[2][2];
        float l_part[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                uint32_t w4[4];
                float lp = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 8 * st + 2 * e;
                    w4[e] = M::pack_out(fast_exp2(fmaf(s_cur[kb][r], c, neg_mc)),
                                        fast_exp2(fmaf(s_cur[kb][r + 1], c, neg_mc)));
                    lp = M::sum2(w4[e], lp);
                }
                l_part[kb][st] = lp;
                pop[kb][st] = __builtin_bit_cast(i16x8, (uint4){w4[0], w4[1], w4[2], w4[3]});
            }
        }
        l_sum += (l_part[0][0] + l_part[0][1]) + (l_part[1][0] + l_part[1][1]);
        if (!SP::kTop && kVLate && more_v) fetch_v(tile + SP::DV);
        // -- O^T += V^T P^T (V^T by transpose read) --
        // A wave whose rows cannot see this tile has all p = 0 here (every score
        // was hidden), so the products add exact zeros.
        const int gi = lane & 15;
        const int dsub = 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
        const int vb = vbuf(tile);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                // Rows R0 + u (u = 4 hh + gi / 4 < 8) and R0 + u + 8, R0 = 32 kb + 16 st:
                // block (R0 % NB) + u, row-in-block R0 / NB (u + 8 wraps to the
                // next row of the same block when NB = 8).
                const int u = 4 * hh + (gi >> 2);
                const int r0 = kb * 32 + 16 * st;
                const uint8_t* v0 = &v_sh[vb][((r0 % NB) + u) * VB + (r0 / NB) * RB + 2 * dsub];
                const uint8_t* v1 = v0 + (NB > 8 ? 8 * VB : RB);
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const i16x4 lo = tr_read(reinterpret_cast<const uint16_t*>(v0 + 64 * d));
                    const i16x4 hi = tr_read(reinterpret_cast<const uint16_t*>(v1 + 64 * d));
                    const i16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[d] = M::mfma(a, pop[kb][st], acc[d]);
                }
            }
        }
        // The next iteration reads K(t+2) and V(t+1); loads issued after those
        // (this iteration's V when DV >= 2, and its K too when DK >= 3) may
        // stay in flight.
        int keep = 0;
        if (SP::DV >= 2 && more_v) keep += kLoadsW;
        if (SP::DK >= 3 && SP::DV >= 2 && more_k) keep += kLoadsW;
        dma_wait_keep(keep);
        __syncthreads();
    };
    for (int tile = t_first; tile < n_tiles; tile += 2) {
        step(tile, s_a, s_b);
        if (tile + 1 < n_tiles) step(tile + 1, s_b, s_a);
    }

    // ---- epilogue: O = acc / l (or the masked-row policy), LSE = m + log l --
    float l_tot = halves_sum(l_sum);
    if constexpr (kSplit) {
        // Partial record of this key range, (m, l, acc) in raw-score units
        // with acc unnormalised; the merge folds a row's ranges in order and
        // applies the sink, the masked-row policy and the LSE.
        if (qrow < p.Lq) {
            // Range-major records: [range][b][h][row][m, l, -, -, acc[D]].
            const int RS = record_stride(p.D);
            float* rec = static_cast<float*>(p.ws) +
                         (((static_cast<int64_t>(rng) * p.B + b) * p.Hq + h) * p.Lq + qrow) * RS;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (32 * d + 8 * u + 4 * hh < Dt)
                        *reinterpret_cast<f32x4*>(rec + 4 + 32 * d + 8 * u + 4 * hh) =
                            f32x4{acc[d][4 * u], acc[d][4 * u + 1], acc[d][4 * u + 2],
                                  acc[d][4 * u + 3]};
            if (hh == 0) {
                rec[0] = m_ref;   // score units (the merge gets the same c and to_nat)
                rec[1] = l_tot;
            }
        }
        return;
    }
    float m_nat = m_ref * to_nat;               // natural units (-inf stays -inf)
    const float fs = fold_sink(p, h, m_nat, l_tot);
    if (kRowStage && elem) {
        // Through the wave's LDS rows (see the Q load): the last tile's
        // barrier has ended every read of the K buffers.
        const bool empty = (l_tot == 0.f);
        const float inv = fs / l_tot;
        const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float o4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = empty ? fill : acc[d][4 * u + e] * inv;
                *reinterpret_cast<uint2*>(xrow + col * D + 32 * d + 8 * u + 4 * hh) =
                    uint2{M::pack_out(o4[0], o4[1]), M::pack_out(o4[2], o4[3])};
            }
        // Eight rows at a time: their LDS reads first, then the
        // (conditional) stores.
        uint16_t* ob = static_cast<uint16_t*>(p.o) + b * p.os.sb + h * p.os.sh;
        // A loop kept rolled: unrolled, the compiler hoists the 32 rows'
        // addresses above the tile loop, where they would spill.
#pragma unroll 1
        for (int r0 = 0; r0 < 32; r0 += 8) {
            uint16_t ov[8][kColIt];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int k = 0; k < kColIt; ++k) ov[r][k] = xrow[(r0 + r) * D + lane + 64 * k];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int64_t qr = qw0 + r0 + r;
#pragma unroll
                for (int k = 0; k < kColIt; ++k) {
                    const int c = lane + 64 * k;
                    if (qr < p.Lq && c < Dt) ob[qr * p.os.sr + c] = ov[r][k];
                }
            }
        }
        if (p.lse && hh == 0 && qrow < p.Lq) {
            const float lse = empty ? kNegInf : row_lse(m_nat, l_tot);
            p.lse[b * p.ls.sb + h * p.ls.sh + qrow * p.ls.sr] = lse;
        }
        return;
    }
    if (qrow < p.Lq) {
        const bool empty = (l_tot == 0.f);
        const float inv = fs / l_tot;
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
                const int c0 = 32 * d + 8 * u + 4 * hh;
                if (elem) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c0 + e < Dt)
                            og[c0 + e] = static_cast<uint16_t>(((e < 2 ? pk.x : pk.y) >> (16 * (e & 1))) & 0xffffu);
                } else if (c0 < Dt) {
                    *reinterpret_cast<uint2*>(og + c0) = pk;
                }
            }
        }
        if (p.lse && hh == 0) {
            const float lse = empty ? kNegInf : row_lse(m_nat, l_tot);
            p.lse[b * p.ls.sb + h * p.ls.sh + qrow * p.ls.sr] = lse;
        }
    }
}

// One wave per (b, h, row), lanes over the head dim: fold the row's
// key-range records in range order (OneGPU "Attention", "Accuracy at long
// key lengths", last paragraph), then the sink, the masked-row policy and the
// LSE as the kernel's own epilogue does.  Records are in the main kernel's
// score units: c converts a difference of them to base 2, to_nat a value to
// natural units.
template <typename T>
__global__ __launch_bounds__(256) void prefill_mfma_merge_kernel(Params p, float c, float to_nat) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (b, h, i)
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * p.Lq;
    if (row >= rows) return;
    const int64_t i = row % p.Lq;
    const int h = static_cast<int>((row / p.Lq) % p.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(p.Lq) * p.Hq));
    const int RS = record_stride(p.D);
    const int64_t range_stride = rows * RS;          // records of one range
    const float* recs = static_cast<const float*>(p.ws) + row * RS;
    constexpr int NPL = 4;                           // head-dim values per lane (D <= 256)
    // Eight ranges' (m, l, acc) are fetched per round, and the reference
    // maximum is the largest seen so far, so up to eight ranges fold in one
    // round exactly as after a separate maximum pass.
    float M = kNegInf, L = 0.f, A[NPL] = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < p.n_split; r0 += 8) {
        float m8[8], l8[8], a8[8][NPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = r0 + u < p.n_split;
            const float* rec = recs + (in ? r0 + u : 0) * range_stride;
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
            if (r0 + u >= p.n_split) break;
            const float f = (m8[u] == kNegInf) ? 0.f : fast_exp2((m8[u] - M) * c);
            L = fmaf(l8[u], f, L);
#pragma unroll
            for (int k = 0; k < NPL; ++k) A[k] = fmaf(a8[u][k], f, A[k]);
        }
    }
    float m_nat = M * to_nat;                    // natural units (-inf stays -inf)
    const float fs = fold_sink(p, h, m_nat, L);
    const bool empty = (L == 0.f);
    const float inv = fs / L;
    const float fill = p.masked_zero ? 0.f : __builtin_nanf("");
    const int64_t orow = b * p.os.sb + h * p.os.sh + i * p.os.sr;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
        const int d = lane + 64 * k;
        if (d < p.D) Elem<T>::store(p.o, orow + d, empty ? fill : A[k] * inv);
    }
    if (p.lse && lane == 0)
        p.lse[b * p.ls.sb + h * p.ls.sh + i * p.ls.sr] = empty ? kNegInf : row_lse(m_nat, L);
}

// Head dims that are not a multiple of 8 (rows not made of whole 16-byte
// chunks): one thread per 8-element chunk copies K and V rows into the
// workspace with the head dim padded to a multiple of 8 (zeros), so the main
// kernel's 16-byte loads apply.  Rows at or past a batch entry's key length
// are written as zeros, not read.
template <int W>
__global__ __launch_bounds__(256) void prefill_stage_kv_kernel(Params p, uint16_t* kd, uint16_t* vd,
                                                               int dp8) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int cpr = dp8 / 8;                                   // chunks per row
    const int64_t total = static_cast<int64_t>(p.B) * p.Hkv * p.Lk * cpr;
    if (t >= total) return;
    const int cch = static_cast<int>(t % cpr);
    const int64_t rowi = t / cpr;                              // (b, g, j) flattened
    const int64_t j = rowi % p.Lk;
    const int g = static_cast<int>((rowi / p.Lk) % p.Hkv);
    const int b = static_cast<int>(rowi / (static_cast<int64_t>(p.Lk) * p.Hkv));
    int64_t kv_len = p.Lk;
    if (p.lens) {
        const int64_t L = p.lens[b];
        kv_len = L < 0 ? 0 : (L > p.Lk ? p.Lk : L);
    }
    const uint16_t* ks = static_cast<const uint16_t*>(p.k) + b * p.ks.sb + g * p.ks.sh + j * p.ks.sr;
    const uint16_t* vs = static_cast<const uint16_t*>(p.v) + b * p.vs.sb + g * p.vs.sh + j * p.vs.sr;
    // W elements per load (W divides D and the rows are aligned to 2 W
    // bytes), so a group is wholly inside the row or wholly past it.
    uint16_t kx[8], vx[8];
#pragma unroll
    for (int e0 = 0; e0 < 8; e0 += W) {
        const int col = 8 * cch + e0;
        const bool in = j < kv_len && col < p.D;
        if constexpr (W == 4) {
            const uint2 kw = in ? *reinterpret_cast<const uint2*>(ks + col) : uint2{0, 0};
            const uint2 vw = in ? *reinterpret_cast<const uint2*>(vs + col) : uint2{0, 0};
            kx[e0] = kw.x & 0xffffu; kx[e0 + 1] = kw.x >> 16; kx[e0 + 2] = kw.y & 0xffffu; kx[e0 + 3] = kw.y >> 16;
            vx[e0] = vw.x & 0xffffu; vx[e0 + 1] = vw.x >> 16; vx[e0 + 2] = vw.y & 0xffffu; vx[e0 + 3] = vw.y >> 16;
        } else if constexpr (W == 2) {
            const uint32_t kw = in ? *reinterpret_cast<const uint32_t*>(ks + col) : 0u;
            const uint32_t vw = in ? *reinterpret_cast<const uint32_t*>(vs + col) : 0u;
            kx[e0] = kw & 0xffffu; kx[e0 + 1] = kw >> 16;
            vx[e0] = vw & 0xffffu; vx[e0 + 1] = vw >> 16;
        } else {
            kx[e0] = in ? ks[col] : uint16_t(0);
            vx[e0] = in ? vs[col] : uint16_t(0);
        }
    }
    const int64_t o = rowi * dp8 + 8 * cch;
    *reinterpret_cast<uint4*>(kd + o) = make_uint4(kx[0] | (uint32_t(kx[1]) << 16), kx[2] | (uint32_t(kx[3]) << 16),
                                                   kx[4] | (uint32_t(kx[5]) << 16), kx[6] | (uint32_t(kx[7]) << 16));
    *reinterpret_cast<uint4*>(vd + o) = make_uint4(vx[0] | (uint32_t(vx[1]) << 16), vx[2] | (uint32_t(vx[3]) << 16),
                                                   vx[4] | (uint32_t(vx[5]) << 16), vx[6] | (uint32_t(vx[7]) << 16));
}

// Padded head dim of the kernel that runs head dim D.
int padded_dim(int D) { return D <= 64 ? 64 : (D <= 128 ? 128 : 256); }

// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides the group
// and leaves each head at least one 32-row wave.
int heads_per_block(int group, int waves) {
    for (int gw = 8; gw > 1; gw >>= 1)
        if (group % gw == 0 && gw <= waves) return gw;
    return 1;
}

// Workgroups whose key range is cut short by a local window or document
// starts (head dim 128 runs them on the kShort shape).
bool short_rows(bool window, bool docs) { return window || docs; }

int waves_for(int DP, bool shrt) {
    if (DP == 128) return shrt ? Cfg<128, true>::kWaves : Cfg<128>::kWaves;
    return DP == 64 ? Cfg<64>::kWaves : Cfg<256>::kWaves;
}
int blocks_per_cu(int DP, bool shrt) {
    if (DP == 128) return shrt ? Cfg<128, true>::kMinBlocks : Cfg<128>::kMinBlocks;
    return DP == 64 ? Cfg<64>::kMinBlocks : Cfg<256>::kMinBlocks;
}
bool short_rows(const Params& p) { return short_rows(p.causal && p.window > 0, p.doc_start); }

int64_t block_count(const Params& p) {
    const int waves = waves_for(padded_dim(p.D), short_rows(p)), rows = 32 * waves;
    const int gw = heads_per_block(p.group, waves);
    const int64_t n_qblk = (p.Lq + rows / gw - 1) / (rows / gw);
    return n_qblk * p.B * p.Hkv * (p.group / gw);
}

template <bool kBf16, int D, bool kShort>
hipError_t launch_shape(const Params& p, hipStream_t s) {
    using CF = Cfg<D, kShort>;
    const int gw = heads_per_block(p.group, CF::kWaves);
    const int n_qblk = (p.Lq + CF::kRows / gw - 1) / (CF::kRows / gw);
    const int units = p.B * p.Hkv * p.n_split;
    const int xcd_units = (units % 8 == 0) ? units / 8 : 0;
    const int mask_vec4 = p.mask && (reinterpret_cast<uintptr_t>(p.mask) % 16 == 0) &&
                          p.ms.sb % 4 == 0 && p.ms.sh % 4 == 0 && p.ms.sr % 4 == 0;
    const dim3 grid(static_cast<uint32_t>(block_count(p) * p.n_split)), blk(CF::kThreads);
    const bool var = p.softcap > 0.f || (p.causal && p.window > 0) || p.doc_start || p.D != D;
    auto go = [&](auto mask_c, auto var_c, auto split_c, auto order_c) {
        constexpr bool kM = decltype(mask_c)::value, kV = decltype(var_c)::value;
        constexpr bool kS = decltype(split_c)::value, kO = decltype(order_c)::value;
        hipLaunchKernelGGL((prefill_mfma_kernel<kBf16, D, kM, kV, kShort, kS, kO>), grid, blk, 0, s,
                           p, n_qblk, gw, xcd_units, mask_vec4);
    };
    using T = std::true_type;
    using F = std::false_type;
    auto by_split = [&](auto mask_c, auto var_c, auto order_c) {
        if (p.n_split > 1) go(mask_c, var_c, T{}, order_c);
        else go(mask_c, var_c, F{}, order_c);
    };
    // Longest entries first: non-causal with per-entry lengths (up to 64
    // entries), on the kernels without score-rule variants.
    const bool order = !p.causal && p.lens != nullptr && p.B <= 64;
    if (kShort) {   // a window or document starts: always the variant kernel
        if (p.mask) by_split(T{}, T{}, F{});
        else by_split(F{}, T{}, F{});
    } else if (p.mask && var) {
        by_split(T{}, T{}, F{});
    } else if (p.mask) {
        if (order) by_split(T{}, F{}, T{});
        else by_split(T{}, F{}, F{});
    } else if (var) {
        by_split(F{}, T{}, F{});
    } else {
        if (order) by_split(F{}, F{}, T{});
        else by_split(F{}, F{}, F{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    const int64_t rows = static_cast<int64_t>(p.B) * p.Hq * p.Lq;
    const dim3 mgrid(static_cast<uint32_t>((rows + 3) / 4));   // a wave per row
    // The records' score units (natural with a mask, raw without).
    const float c = p.mask ? kLog2e : p.scale_log2, to_nat = p.mask ? 1.f : p.scale;
    if (kBf16)
        hipLaunchKernelGGL((prefill_mfma_merge_kernel<bf16_t>), mgrid, dim3(256), 0, s, p, c, to_nat);
    else
        hipLaunchKernelGGL((prefill_mfma_merge_kernel<_Float16>), mgrid, dim3(256), 0, s, p, c,
                           to_nat);
    return hipGetLastError();
}

template <bool kBf16, int D>
hipError_t launch_one(const Params& p, hipStream_t s) {
    if constexpr (D == 128)
        if (short_rows(p)) return launch_shape<kBf16, D, true>(p, s);
    return launch_shape<kBf16, D, false>(p, s);
}

}  // namespace

// Key ranges for small grids (shape only): when the query blocks would leave
// at least half of the GPU's resident workgroup slots empty (256 CUs of an
// MI355X; three slots per CU at head dim 64), each block's keys may be cut
// into ranges of a whole number of tiles, at most 32 ranges, aiming at two
// workgroups per slot.  Each range writes its rows' (m, l, acc) records in
// fp32 (about twice the output's bytes per range, read back by the merge
// kernel), so a range must carry enough tiles to pay for them; the fewer the
// blocks, the more an idle CU costs and the shorter a range may be:
//   blocks <= 32: ranges of at least 4 tiles;
//   blocks <= 128: at least 8 tiles, keys of at least 32 tiles;
//   blocks <= 256: at least 16 tiles, keys of at least 128 tiles;
//   more blocks: no split.
// (Measured on one MI355X over 16 shapes, head dims 64 and 128; e.g. BERT-
// base B8 S512 (384 blocks of 8 tiles) 44 us split into two ranges against
// 16 us whole, B1 H8 L1024 D128 (32 blocks of 16 tiles) 29 us in four
// ranges against 33 us whole.)
void prefill_mfma_plan(int B, int Hq, int Hkv, int Lq, int Lk, int D, bool window, bool docs,
                       int* split_len, int* n_split) {
    *split_len = 0;
    *n_split = 1;
    if (B <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq <= 0 || Lk <= 0 || D < 1 || D > 256) return;
    const bool shrt = short_rows(window, docs);
    const int DP = padded_dim(D), waves = waves_for(DP, shrt), rows = 32 * waves;
    const int group = Hq / Hkv, gw = heads_per_block(group, waves);
    const int64_t blocks = static_cast<int64_t>((Lq + rows / gw - 1) / (rows / gw)) * B * Hkv *
                           (group / gw);
    const int64_t slots = 256 * blocks_per_cu(DP, shrt);
    const int64_t tiles = (static_cast<int64_t>(Lk) + kBN - 1) / kBN;
    if (2 * blocks > slots || tiles < 8) return;
    int64_t per_min;                                  // tiles per range at least
    if (blocks <= 32)
        per_min = 4;
    else if (blocks <= 128 && tiles >= 32)
        per_min = 8;
    else if (blocks <= 256 && tiles >= 128)
        per_min = 16;
    else
        return;
    int64_t n = (2 * slots + blocks - 1) / blocks;
    if (n > tiles / per_min) n = tiles / per_min;
    if (n > 32) n = 32;
    if (n < 2) return;
    const int64_t per = (tiles + n - 1) / n;          // tiles per range
    *split_len = static_cast<int>(per * kBN);
    *n_split = static_cast<int>((tiles + per - 1) / per);
}

size_t prefill_mfma_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, bool window,
                                    bool docs) {
    int len, n;
    prefill_mfma_plan(B, Hq, Hkv, Lq, Lk, D, window, docs, &len, &n);
    if (n <= 1) return 0;
    return static_cast<size_t>(B) * Hq * Lq * n * record_stride(D) * sizeof(float);
}

// Workspace bytes of the staged K/V copies (head dims that are not a
// multiple of 8; 0 otherwise), shape only; 256-byte multiple.
size_t prefill_mfma_stage_bytes(int B, int Hkv, int Lk, int D) {
    if (D % 8 == 0 || Lk == 0) return 0;
    const size_t one = static_cast<size_t>(B) * Hkv * Lk * ((D + 7) / 8 * 8) * 2;
    return (2 * one + 255) / 256 * 256;
}

bool prefill_mfma_supported(const Params& p, DType dt) {
    if (dt != DType::BF16 && dt != DType::F16) return false;
    if (p.D < 1 || p.D > 256) return false;
    const bool staged = p.D % 8 != 0;
    // 16-byte loads of Q/K/V rows and 8-byte stores of O need aligned rows;
    // a staged problem reads Q and writes O in 2-byte elements and reads K/V from
    // its aligned copies.
    auto al = [](const void* ptr, const Strides& st, int a) {
        return reinterpret_cast<uintptr_t>(ptr) % (2 * a) == 0 && st.sb % a == 0 &&
               st.sh % a == 0 && st.sr % a == 0;
    };
    if (!staged) {
        if (!al(p.q, p.qs, 8) || !al(p.o, p.os, 4)) return false;
        if (p.Lk > 0 && (!al(p.k, p.ks, 8) || !al(p.v, p.vs, 8))) return false;
    }
    // Buffer offsets within one (b, kv head) slice are 32-bit, including the
    // up-to-one-tile overrun past the key length.
    const int64_t ksr = staged ? (p.D + 7) / 8 * 8 : p.ks.sr;
    const int64_t vsr = staged ? (p.D + 7) / 8 * 8 : p.vs.sr;
    if (ksr >= (1 << 24) || vsr >= (1 << 24)) return false;
    if ((static_cast<int64_t>(p.Lk) + kBN) * ksr * 2 >= (int64_t(1) << 31) ||
        (static_cast<int64_t>(p.Lk) + kBN) * vsr * 2 >= (int64_t(1) << 31))
        return false;
    return block_count(p) * p.n_split < (int64_t(1) << 31);
}

hipError_t launch_prefill_mfma(const Params& p_in, DType dt, hipStream_t s) {
    Params p = p_in;
    if (p.D % 8 != 0 && p.Lk > 0) {   // stage K/V with the head dim padded to a multiple of 8
        const int dp8 = (p.D + 7) / 8 * 8;
        uint16_t* kd = static_cast<uint16_t*>(p.stage);
        uint16_t* vd = kd + static_cast<int64_t>(p.B) * p.Hkv * p.Lk * dp8;
        const int64_t chunks = static_cast<int64_t>(p.B) * p.Hkv * p.Lk * (dp8 / 8);
        // Widest element group that divides D and keeps every access aligned.
        auto fits = [&](int w) {
            auto al = [&](const void* ptr, const Strides& st) {
                return reinterpret_cast<uintptr_t>(ptr) % (2 * w) == 0 && st.sb % w == 0 &&
                       st.sh % w == 0 && st.sr % w == 0;
            };
            return p.D % w == 0 && al(p.k, p.ks) && al(p.v, p.vs);
        };
        const dim3 grid(static_cast<uint32_t>((chunks + 255) / 256));
        if (fits(4))
            hipLaunchKernelGGL(prefill_stage_kv_kernel<4>, grid, dim3(256), 0, s, p, kd, vd, dp8);
        else if (fits(2))
            hipLaunchKernelGGL(prefill_stage_kv_kernel<2>, grid, dim3(256), 0, s, p, kd, vd, dp8);
        else
            hipLaunchKernelGGL(prefill_stage_kv_kernel<1>, grid, dim3(256), 0, s, p, kd, vd, dp8);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.k = kd;
        p.v = vd;
        p.ks = {static_cast<int64_t>(p.Hkv) * p.Lk * dp8, static_cast<int64_t>(p.Lk) * dp8, dp8};
        p.vs = p.ks;
    }
    const int DP = padded_dim(p.D);
    if (dt == DType::BF16) {
        if (DP == 64) return launch_one<true, 64>(p, s);
        return DP == 128 ? launch_one<true, 128>(p, s) : launch_one<true, 256>(p, s);
    }
    if (DP == 64) return launch_one<false, 64>(p, s);
    return DP == 128 ? launch_one<false, 128>(p, s) : launch_one<false, 256>(p, s);
}

}  // namespace sdpa
