// api.cpp -- the C ABI declared in include/sdpa_flash.h: argument validation,
// kernel choice and launch.  Validation runs entirely on the host and before
// any launch, so an error leaves every output untouched.
#include "sdpa_flash.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "attn_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local const char* g_kernel = "";

// Test and debugging override: SDPA_FLASH_KERNEL=generic forces the
// any-shape kernel for every call.
bool force_generic() {
    const char* e = std::getenv("SDPA_FLASH_KERNEL");
    return e && std::strcmp(e, "generic") == 0;
}

attn_status fail(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

size_t elem_size(int32_t dt) { return dt == ATTN_DTYPE_F32 ? 4 : 2; }

bool nonneg(const attn_layout& l) {
    return l.offset >= 0 && l.batch_stride >= 0 && l.head_stride >= 0 && l.row_stride >= 0;
}

// Largest element index a layout touches for (B, H, L, width), +1; in 128
// bits, so that no stride a caller passes can wrap it past the limit check.
__int128 extent(const attn_layout& l, int64_t B, int64_t H, int64_t L, int64_t width) {
    if (B == 0 || H == 0 || L == 0 || width == 0) return 0;
    return static_cast<__int128>(l.offset) + static_cast<__int128>(B - 1) * l.batch_stride +
           static_cast<__int128>(H - 1) * l.head_stride +
           static_cast<__int128>(L - 1) * l.row_stride + width;
}

// check_ptrs = false validates the problem alone (for attn_workspace_size).
attn_status validate(const attn_problem* p, bool check_ptrs, const void* q, const void* k,
                     const void* v, const void* o, const float* mask, const float* lse) {
    if (!p) return fail(ATTN_ERR_INVALID, "problem is NULL");
    if (p->batch < 0 || p->q_len < 0 || p->k_len < 0)
        return fail(ATTN_ERR_INVALID, "batch, q_len and k_len must be >= 0");
    if (p->q_heads < 1 || p->kv_heads < 1)
        return fail(ATTN_ERR_INVALID, "q_heads and kv_heads must be >= 1");
    if (p->q_heads % p->kv_heads != 0)
        return fail(ATTN_ERR_INVALID, "q_heads (%d) is not a multiple of kv_heads (%d)",
                    p->q_heads, p->kv_heads);
    if (p->q_heads > 65535 || p->batch > 65535)
        return fail(ATTN_ERR_UNSUPPORTED, "q_heads and batch are limited to 65535");
    if (p->head_dim < 1 || p->head_dim > 256)
        return fail(ATTN_ERR_INVALID, "head_dim %d outside 1..256", p->head_dim);
    if (p->dtype != ATTN_DTYPE_F32 && p->dtype != ATTN_DTYPE_F16 && p->dtype != ATTN_DTYPE_BF16)
        return fail(ATTN_ERR_INVALID, "unknown dtype %d", p->dtype);
    if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1");
    if (p->masked_rows != ATTN_MASKED_ROWS_NAN && p->masked_rows != ATTN_MASKED_ROWS_ZERO)
        return fail(ATTN_ERR_INVALID, "unknown masked_rows policy %d", p->masked_rows);
    if (!(std::isfinite(p->scale)) || p->scale < 0.f)
        return fail(ATTN_ERR_INVALID, "scale must be finite and >= 0");
    if (p->window < 0) return fail(ATTN_ERR_INVALID, "window must be >= 0");
    if (p->window > 0 && !p->causal)
        return fail(ATTN_ERR_INVALID, "a local window needs the causal rule");
    if (!(std::isfinite(p->softcap)) || p->softcap < 0.f)
        return fail(ATTN_ERR_INVALID, "softcap must be finite and >= 0");
    if (p->sink != 0 && p->sink != 1) return fail(ATTN_ERR_INVALID, "sink must be 0 or 1");
    if (p->head_sink && !p->sink)
        return fail(ATTN_ERR_INVALID, "head_sink given without sink = 1");
    if (p->kv_int8 != 0 && p->kv_int8 != 1) return fail(ATTN_ERR_INVALID, "kv_int8 must be 0 or 1");
    if (p->kv_int8) {
        auto qok = [](int32_t m) {
            return m == ATTN_QUANT_PER_TENSOR || m == ATTN_QUANT_PER_CHANNEL;
        };
        if (!qok(p->k_quant) || !qok(p->v_quant))
            return fail(ATTN_ERR_INVALID, "an int8 cache needs k_quant and v_quant per tensor or "
                                          "per channel");
        if (check_ptrs && (!p->k_scale || !p->v_scale))
            return fail(ATTN_ERR_INVALID, "an int8 cache needs k_scale and v_scale");
    } else if (p->k_quant || p->v_quant || p->k_scale || p->v_scale) {
        return fail(ATTN_ERR_INVALID, "quantization fields set without kv_int8 = 1");
    }
    if (!nonneg(p->q) || !nonneg(p->k) || !nonneg(p->v) || !nonneg(p->o))
        return fail(ATTN_ERR_INVALID, "layout offsets and strides must be >= 0");
    if (!check_ptrs) {
        mask = nullptr;
        lse = nullptr;
    }
    if (mask && !nonneg(p->mask)) return fail(ATTN_ERR_INVALID, "mask strides must be >= 0");
    if (lse && !nonneg(p->lse)) return fail(ATTN_ERR_INVALID, "lse strides must be >= 0");
    const bool work = check_ptrs && p->batch > 0 && p->q_len > 0;
    if (work && (!q || !o)) return fail(ATTN_ERR_INVALID, "q and o must be non-NULL");
    if (work && p->k_len > 0 && (!k || !v))
        return fail(ATTN_ERR_INVALID, "k and v must be non-NULL when k_len > 0");
    const int64_t D = p->head_dim;
    // 64-bit element offsets are used everywhere; reject extents past 2^62.
    const __int128 lim = static_cast<__int128>(1) << 62;
    if (extent(p->q, p->batch, p->q_heads, p->q_len, D) > lim ||
        extent(p->o, p->batch, p->q_heads, p->q_len, D) > lim ||
        extent(p->k, p->batch, p->kv_heads, p->k_len, D) > lim ||
        extent(p->v, p->batch, p->kv_heads, p->k_len, D) > lim)
        return fail(ATTN_ERR_INVALID, "tensor extent too large");
    if (mask && extent(p->mask, p->batch, p->q_heads, p->q_len, p->k_len) > lim)
        return fail(ATTN_ERR_INVALID, "mask extent too large");
    if (lse && extent(p->lse, p->batch, p->q_heads, p->q_len, 1) > lim)
        return fail(ATTN_ERR_INVALID, "lse extent too large");
    return ATTN_OK;
}

sdpa::Params make_params(const attn_problem* p, const void* q, const void* k, const void* v,
                         void* o, const float* mask, const int32_t* key_lens, float* lse) {
    sdpa::Params r{};
    r.n_split = 1;
    const size_t es = elem_size(p->dtype);
    auto adv = [&](const void* base, int64_t off) -> const void* {
        return base ? static_cast<const char*>(base) + off * static_cast<int64_t>(es) : nullptr;
    };
    const size_t kes = p->kv_int8 ? 1 : es;       // K/V element size
    auto adv_kv = [&](const void* base, int64_t off) -> const void* {
        return base ? static_cast<const char*>(base) + off * static_cast<int64_t>(kes) : nullptr;
    };
    r.q = adv(q, p->q.offset);
    r.k = adv_kv(k, p->k.offset);
    r.v = adv_kv(v, p->v.offset);
    r.o = const_cast<void*>(adv(o, p->o.offset));
    r.mask = mask ? mask + p->mask.offset : nullptr;
    r.lens = key_lens;
    r.lse = lse ? lse + p->lse.offset : nullptr;
    r.qs = {p->q.batch_stride, p->q.head_stride, p->q.row_stride};
    r.ks = {p->k.batch_stride, p->k.head_stride, p->k.row_stride};
    r.vs = {p->v.batch_stride, p->v.head_stride, p->v.row_stride};
    r.os = {p->o.batch_stride, p->o.head_stride, p->o.row_stride};
    r.ms = {p->mask.batch_stride, p->mask.head_stride, p->mask.row_stride};
    r.ls = {p->lse.batch_stride, p->lse.head_stride, p->lse.row_stride};
    r.B = p->batch;
    r.Hq = p->q_heads;
    r.Hkv = p->kv_heads;
    r.Lq = p->q_len;
    r.Lk = p->k_len;
    r.D = p->head_dim;
    r.group = p->q_heads / p->kv_heads;
    r.causal = p->causal;
    r.masked_zero = p->masked_rows == ATTN_MASKED_ROWS_ZERO;
    r.delta_end = p->causal_offset == ATTN_CAUSAL_OFFSET_KEY_END;
    r.delta = (p->causal_offset == ATTN_CAUSAL_OFFSET_DEFAULT || r.delta_end)
                  ? static_cast<int64_t>(p->k_len) - p->q_len
                  : p->causal_offset;
    const double scale = p->scale != 0.f ? static_cast<double>(p->scale)
                                         : 1.0 / std::sqrt(static_cast<double>(p->head_dim));
    r.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
    r.scale = static_cast<float>(scale);
    r.window = p->window;
    r.softcap = p->softcap;
    r.sink = p->sink;
    r.head_sink = p->head_sink;
    r.kv_int8 = p->kv_int8;
    r.k_quant = p->k_quant;
    r.v_quant = p->v_quant;
    r.k_scale = p->k_scale;
    r.v_scale = p->v_scale;
    r.doc_start = p->doc_start;
    return r;
}

attn_status launched(hipError_t e) {
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return ATTN_OK;
}

}  // namespace

attn_status sdpa::set_error(attn_status status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

extern "C" {

const char* attn_last_error(void) { return g_err; }

const char* attn_last_kernel(void) { return g_kernel; }

const char* attn_version(void) { return "sdpa_flash 0.1 (gfx950)"; }

// Workspace of the split decode path; depends on the shape only.
size_t decode_split_ws(const attn_problem* p) {
    const bool half = (p->dtype == ATTN_DTYPE_BF16 || p->dtype == ATTN_DTYPE_F16) &&
                      p->head_dim >= 8 && p->head_dim <= 256 &&
                      p->head_dim % (p->kv_int8 ? 16 : 8) == 0;
    const bool f32 = p->dtype == ATTN_DTYPE_F32 && !p->kv_int8 && p->head_dim >= 4 &&
                     p->head_dim <= 128 && p->head_dim % 4 == 0;
    const bool shape_ok = (half || f32) && p->q_len == 1 && p->k_len > 0;
    return shape_ok ? sdpa::decode_workspace_bytes(p->batch, p->q_heads, p->kv_heads, p->head_dim)
                    : 0;
}

// Workspace of the prefill paths' key-range splits (fp32 kernel; bf16/fp16
// matrix-core kernel on small grids), and with one query row of the decode
// kernels that such a call runs on; shape only.
size_t forward_ws(const attn_problem* p) {
    const size_t dec = decode_split_ws(p);
    if (p->dtype == ATTN_DTYPE_F32) {
        const size_t pre = sdpa::prefill_f32_workspace_bytes(p->batch, p->q_heads, p->kv_heads,
                                                             p->q_len, p->k_len, p->head_dim);
        return pre > dec ? pre : dec;
    }
    // Staged K/V copies (head dims not a multiple of 8) first, then the
    // key-range split's records.
    const size_t pre =
        sdpa::prefill_mfma_stage_bytes(p->batch, p->kv_heads, p->k_len, p->head_dim) +
        sdpa::prefill_mfma_workspace_bytes(p->batch, p->q_heads, p->kv_heads, p->q_len, p->k_len,
                                           p->head_dim, p->causal && p->window > 0,
                                           p->doc_start != nullptr);
    return pre > dec ? pre : dec;
}

// attn_decode runs the split decode path when the shape and the buffers allow
// it and the forward path otherwise, so its workspace covers both (shape only).
size_t decode_ws(const attn_problem* p) {
    const size_t a = decode_split_ws(p);
    const size_t b = p->kv_int8 ? 0 : forward_ws(p);
    return a > b ? a : b;
}

// One query row per (batch entry, head) on the decode kernels (the caller has
// checked sdpa::decode_split_supported): the split mode with its merge, or
// one workgroup per unit.  The workspace is checked in both modes, so that
// whether a call needs one never depends on the mode the shape picks.
attn_status run_decode(const attn_problem* p, sdpa::Params& prm, sdpa::DType dt, hipStream_t s,
                       void* workspace, size_t workspace_bytes) {
    const size_t need = decode_split_ws(p);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : size_t(0));
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");
    prm.ws = workspace;
    // SDPA_FLASH_KERNEL=decode_unit / decode_splitk picks the mode (tests
    // run every case through both); by default the shape decides.
    const char* km = std::getenv("SDPA_FLASH_KERNEL");
    const bool unit = (km && std::strcmp(km, "decode_unit") == 0)     ? true
                      : (km && std::strcmp(km, "decode_splitk") == 0) ? false
                                                                       : sdpa::decode_unit_preferred(prm, dt);
    if (unit)
        g_kernel = p->kv_int8 ? "decode_unit_int8" : "decode_unit";
    else
        g_kernel = p->kv_int8 ? "decode_splitk_int8" : "decode_splitk";
    return launched(sdpa::launch_decode_split(prm, dt, s, unit));
}

attn_status attn_workspace_size(const attn_problem* p, int32_t op, size_t* bytes) {
    if (!bytes) return fail(ATTN_ERR_INVALID, "bytes is NULL");
    *bytes = 0;
    attn_status st = validate(p, false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    if (st != ATTN_OK) return st;
    if (op != ATTN_OP_FORWARD && op != ATTN_OP_DECODE)
        return fail(ATTN_ERR_INVALID, "unknown op %d", op);
    *bytes = (op == ATTN_OP_DECODE) ? decode_ws(p) : forward_ws(p);
    return ATTN_OK;
}

attn_status attn_forward(const attn_problem* p, const void* q, const void* k, const void* v,
                         void* o, const float* mask, const int32_t* key_lens, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
    attn_status st = validate(p, true, q, k, v, o, mask, lse);
    if (st != ATTN_OK) return st;
    if (p->batch == 0 || p->q_len == 0) {
        g_err[0] = '\0';
        g_kernel = "";
        return ATTN_OK;
    }
    if (p->kv_int8)
        return fail(ATTN_ERR_UNSUPPORTED, "an int8 key/value cache runs through attn_decode only");
    sdpa::Params prm = make_params(p, q, k, v, o, mask, key_lens, lse);
    const auto dt = static_cast<sdpa::DType>(p->dtype);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // One query row (a cross-attention step, or decode called as a forward):
    // the decode kernels read each live K/V row once for a whole head group,
    // where a prefill tile would fill one of its rows.  Except small fp32
    // problems without head groups (fewer than 64 kv heads in all): there
    // the fp32 prefill kernel's key ranges spread the few heads wider than
    // the decode kernels, whose fp32 steps cost 16 columns of matrix work
    // for the one head (the Whisper cross-attention step, 12 heads of 1500
    // keys: 18.9 us against 21.3).
    const bool small_mha_f32 = dt == sdpa::DType::F32 && p->q_heads == p->kv_heads &&
                               static_cast<int64_t>(p->batch) * p->kv_heads < 64;
    if (!force_generic() && p->q_len == 1 && !small_mha_f32 &&
        sdpa::decode_split_supported(prm, dt))
        return run_decode(p, prm, dt, s, workspace, workspace_bytes);
    if (!force_generic() && (dt == sdpa::DType::BF16 || dt == sdpa::DType::F16)) {
        sdpa::prefill_mfma_plan(p->batch, p->q_heads, p->kv_heads, p->q_len, p->k_len,
                                p->head_dim, p->causal && p->window > 0, p->doc_start != nullptr,
                                &prm.split_len, &prm.n_split);
        if (sdpa::prefill_mfma_supported(prm, dt)) {
            const size_t need = forward_ws(p);
            if (need > 0) {
                if (!workspace || workspace_bytes < need)
                    return fail(ATTN_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu",
                                need, workspace ? workspace_bytes : size_t(0));
                if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
                    return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");
                const size_t stage =
                    sdpa::prefill_mfma_stage_bytes(p->batch, p->kv_heads, p->k_len, p->head_dim);
                prm.stage = workspace;
                prm.ws = static_cast<char*>(workspace) + stage;
            }
            g_kernel = "prefill_mfma";
            return launched(sdpa::launch_prefill_mfma(prm, dt, s));
        }
        prm.n_split = 1;
        prm.split_len = 0;
    }
    sdpa::prefill_f32_plan(p->batch, p->q_heads, p->kv_heads, p->q_len, p->k_len, p->head_dim,
                           &prm.split_len, &prm.n_split);
    if (!force_generic() && sdpa::prefill_f32_supported(prm, dt)) {
        if (prm.n_split > 1) {
            const size_t need = forward_ws(p);
            if (!workspace || workspace_bytes < need)
                return fail(ATTN_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need,
                            workspace ? workspace_bytes : size_t(0));
            if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
                return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");
            prm.ws = workspace;
        }
        g_kernel = "prefill_f32";
        return launched(sdpa::launch_prefill_f32(prm, dt, s));
    }
    g_kernel = "generic";
    return launched(sdpa::launch_generic(prm, dt, s));
}

attn_status attn_decode(const attn_problem* p, const void* q, const void* k, const void* v,
                        void* o, const float* mask, const int32_t* key_lens, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
    attn_status st = validate(p, true, q, k, v, o, mask, lse);
    if (st != ATTN_OK) return st;
    if (p->q_len != 1) return fail(ATTN_ERR_INVALID, "decode needs q_len == 1");
    if (p->batch == 0) {
        g_err[0] = '\0';
        g_kernel = "";
        return ATTN_OK;
    }
    sdpa::Params prm = make_params(p, q, k, v, o, mask, key_lens, lse);
    const auto dt = static_cast<sdpa::DType>(p->dtype);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!force_generic() && sdpa::decode_split_supported(prm, dt))
        return run_decode(p, prm, dt, s, workspace, workspace_bytes);
    if (p->kv_int8)
        return fail(ATTN_ERR_UNSUPPORTED, "int8 cache decode needs fp16/bf16, a head_dim that is "
                                          "a multiple of 16 up to 256 and 16-byte aligned K/V rows");
    return attn_forward(p, q, k, v, o, mask, key_lens, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
