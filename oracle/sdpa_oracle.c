/*
 * sdpa_oracle.c -- plain CPU oracle for fused scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP path.
 *
 * What it computes is the plain definition, in float64, by three passes over
 * each query row (no tiling, no online normaliser, no reordering):
 *
 *   O = softmax(scale * Q K^T + Mask) V            (OneGPU "Attention", intro)
 *
 * following the classic three-pass softmax (llm.istanbul 05_attention,
 * section "Online Softmax - Niye?": max, then sum of exp(s - m), then divide),
 * with the visibility and special-value rules of OneGPU "Attention":
 *   - "What it covers" table: grouped heads, per-batch key lengths, causal with
 *     an offset whose default is KLen - QLen, a broadcast additive float mask;
 *   - "Special values": hidden keys weigh 0; a row with no visible key gives
 *     NaN (or zeros under the Zero policy); a NaN or +inf score gives NaN.
 * GQA mapping: query head h reads kv head h / (Hq / Hkv) (llm.istanbul,
 * section "GQA", and line-by-line step 1).
 * LSE = m + log(l) (llm.istanbul, "Online Softmax Algoritmasi", final step).
 *
 * Readings taken where the pages are silent:
 *   - key lengths are clamped to [0, KLen]; the default causal offset is
 *     relative to the problem's KLen, not the per-batch length;
 *   - the end-aligned offset (mode 2) is, per batch entry, the clamped key
 *     length minus QLen: the last query row lines up with the entry's last
 *     live key, as for a chunk of new tokens appended to a cache whose live
 *     length differs per entry (ONNX GroupQueryAttention README,
 *     "Implementation variants": causal tiles bounded by each entry's live
 *     length, right-aligned; "Inputs": per-sample total sequence lengths);
 *   - a row with a NaN or +inf score is NaN under both policies, LSE NaN;
 *     this check comes before the empty-row check;
 *   - an empty row (no visible key, or every visible score -inf) has LSE -inf
 *     under both policies;
 *   - the mask is added after scaling; keys hidden by length or by the causal
 *     rule are never evaluated (so garbage there cannot leak in).
 *
 * Score-rule variants (ONNX GroupQueryAttention README, "Attributes" and
 * "Inputs"; readings):
 *   - local window W >= 0 (causal only): the row at position p = i + offset
 *     also needs j >= p - W, i.e. W keys to its left and itself ("left window
 *     size for causal local attention"); -1 disables it;
 *   - softcap c > 0: the scaled score becomes c * tanh(score / c), before the
 *     additive mask is added (so a -inf mask entry still hides its key);
 *   - sink: one more term exp(sink_h) in each row's softmax denominator, a
 *     key of score sink_h with no value ("per-head smooth factor added to the
 *     softmax denominator"; smooth softmax without per-head values uses 0).
 *     A row then always has weight somewhere: with no visible key O = 0 and
 *     LSE = sink_h under both policies; a NaN / +inf score, the sink's own
 *     included, still gives NaN.
 *
 * Document masks (llm.istanbul "05_attention", line-by-line steps "Phase 0"
 * and "K-block iteration"): packed documents give each query row the index
 * of its document's first key, doc_start[b * Lq + i]; keys before it are
 * hidden (row i sees j >= doc_start, together with the other rules).
 *
 * Quantized key/value cache (ONNX GroupQueryAttention README, "Inputs":
 * k_scale / v_scale; "Attributes": k_quant_type / v_quant_type, cache bit
 * width 8): a cache element is a signed 8-bit integer and its value is that
 * integer times a float32 scale -- one scale for the whole tensor (per
 * tensor), or one per (kv head, head-dim index), stored at g * D + d (per
 * channel).  Reading: symmetric, no zero point; Q and the output keep the
 * problem's element type.
 *
 * Inputs are read in their storage type and decoded exactly to double
 * (float32 widened; float16 and bfloat16 bit patterns decoded from their IEEE
 * definitions), as the OneGPU "Tolerances" section describes its reference
 * ("reference in double on the CPU, inputs rounded to half first").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* Strides are in elements; the innermost (head-dim / key) stride is 1. */
typedef struct oracle_problem {
    int64_t batch, q_heads, kv_heads, q_len, k_len, head_dim;
    int32_t dtype;          /* ORACLE_F32 / ORACLE_F16 / ORACLE_BF16            */
    int32_t causal;         /* 0 or 1                                           */
    int32_t has_offset;     /* 0: offset k_len - q_len; 1: causal_offset;
                               2: per batch entry, clamped key length - q_len   */
    int32_t masked_zero;    /* 0: empty rows are NaN, 1: empty rows are zero    */
    int64_t causal_offset;  /* used when has_offset == 1                        */
    double scale;           /* 0: 1/sqrt(head_dim)                              */
    int64_t qs[3], ks[3], vs[3]; /* batch, head, row strides                     */
    int64_t ms[3];          /* mask batch, head, row strides (0 = broadcast)    */
    int32_t window;         /* -1: none; W >= 0: causal rows need j >= i+delta-W */
    int32_t sink;           /* 0: none; 1: exp(sink_h) joins the denominator     */
    double softcap;         /* 0: none; c > 0: score -> c * tanh(score / c)      */
    int32_t kv_int8;        /* 0: K/V in dtype; 1: int8 cache with scales        */
    int32_t k_quant;        /* with kv_int8: 1 per tensor, 2 per channel         */
    int32_t v_quant;        /* likewise for V                                    */
} oracle_problem;

/* float16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);  /* (1 + f/1024) * 2^(e-15)     */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_decode_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* base, int32_t dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float*)base)[idx];
    if (dtype == ORACLE_F16)
        return oracle_decode_f16(((const uint16_t*)base)[idx]);
    return oracle_decode_bf16(((const uint16_t*)base)[idx]);
}

/* Element d of a K or V row: the stored value, or for an int8 cache the
 * integer times its scale (per tensor: scale[0]; per channel: scale[g*D+d]). */
static double load_kv(const oracle_problem* p, const void* base, const float* scale, int32_t quant,
                      int64_t g, int64_t idx, int64_t d)
{
    if (!p->kv_int8)
        return load_elem(base, p->dtype, idx);
    const double x = (double)((const int8_t*)base)[idx];
    return x * (double)(quant == 1 ? scale[0] : scale[g * p->head_dim + d]);
}

/* One query row (b, h, i).  s is scratch of k_len doubles. */
static void one_row(const oracle_problem* p, const void* q, const void* k, const void* v,
                    const float* mask, const int32_t* key_lens, const float* head_sink,
                    const float* k_scale, const float* v_scale, const int32_t* doc_start,
                    int64_t b, int64_t h, int64_t i, double* s, unsigned char* vis,
                    double* o_row, double* lse_out)
{
    const int64_t D = p->head_dim;
    const int64_t group = p->q_heads / p->kv_heads;
    const int64_t g = h / group;
    const double scale = p->scale != 0.0 ? p->scale : 1.0 / sqrt((double)D);

    int64_t kv_len = p->k_len;
    if (key_lens) {
        int64_t L = key_lens[b];
        kv_len = L < 0 ? 0 : (L > p->k_len ? p->k_len : L);
    }
    const int64_t delta = p->has_offset == 1   ? p->causal_offset
                          : p->has_offset == 2 ? kv_len - p->q_len
                                               : p->k_len - p->q_len;

    const int64_t qbase = b * p->qs[0] + h * p->qs[1] + i * p->qs[2];
    const int64_t first_key = doc_start ? (int64_t)doc_start[b * p->q_len + i] : 0;

    /* Scores of the visible keys. */
    for (int64_t j = 0; j < p->k_len; ++j) {
        vis[j] = (j < kv_len) && j >= first_key &&
                 (!p->causal || (j <= i + delta && (p->window < 0 || j >= i + delta - p->window)));
        if (!vis[j])
            continue;
        const int64_t kbase = b * p->ks[0] + g * p->ks[1] + j * p->ks[2];
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += load_elem(q, p->dtype, qbase + d) *
                   load_kv(p, k, k_scale, p->k_quant, g, kbase + d, d);
        double sj = scale * dot;
        if (p->softcap > 0.0)
            sj = p->softcap * tanh(sj / p->softcap);
        if (mask)
            sj += (double)mask[b * p->ms[0] + h * p->ms[1] + i * p->ms[2] + j];
        s[j] = sj;
    }

    /* The sink is one more softmax term with no value vector. */
    const double sink = p->sink ? (head_sink ? (double)head_sink[h] : 0.0) : -INFINITY;

    /* Pass 1: maximum, and whether any score is NaN or +inf. */
    double m = -INFINITY;
    int bad = isnan(sink) || sink == INFINITY;
    for (int64_t j = 0; j < p->k_len; ++j) {
        if (!vis[j])
            continue;
        if (isnan(s[j]) || s[j] == INFINITY)
            bad = 1;
        else if (s[j] > m)
            m = s[j];
    }
    if (bad) {
        for (int64_t d = 0; d < D; ++d)
            o_row[d] = NAN;
        *lse_out = NAN;
        return;
    }
    if (sink > m)
        m = sink;
    if (m == -INFINITY) {
        /* No visible key with a finite score: the masked-row policy. */
        for (int64_t d = 0; d < D; ++d)
            o_row[d] = p->masked_zero ? 0.0 : NAN;
        *lse_out = -INFINITY;
        return;
    }

    /* Pass 2: normaliser. */
    double l = p->sink ? exp(sink - m) : 0.0;
    for (int64_t j = 0; j < p->k_len; ++j)
        if (vis[j])
            l += exp(s[j] - m);

    /* Pass 3: weights times values. */
    for (int64_t d = 0; d < D; ++d)
        o_row[d] = 0.0;
    for (int64_t j = 0; j < p->k_len; ++j) {
        if (!vis[j])
            continue;
        const double w = exp(s[j] - m) / l;
        const int64_t vbase = b * p->vs[0] + g * p->vs[1] + j * p->vs[2];
        for (int64_t d = 0; d < D; ++d)
            o_row[d] += w * load_kv(p, v, v_scale, p->v_quant, g, vbase + d, d);
    }
    *lse_out = m + log(l);
}

/*
 * Computes the rows listed in `rows` (n_rows triples b, h, i), or every row in
 * (b, h, i) order when rows is NULL (then n_rows must be B*Hq*Lq).
 * o: n_rows * head_dim doubles, lse: n_rows doubles (may be NULL).
 * Returns 0, or -1 on a malformed problem.
 */
int oracle_attention(const oracle_problem* p, const void* q, const void* k, const void* v,
                     const float* mask, const int32_t* key_lens, const float* head_sink,
                     const float* k_scale, const float* v_scale, const int32_t* doc_start,
                     const int64_t* rows, int64_t n_rows, double* o, double* lse,
                     int n_threads)
{
    if (!p || p->q_heads <= 0 || p->kv_heads <= 0 || p->q_heads % p->kv_heads != 0 ||
        p->head_dim <= 0 || p->batch < 0 || p->q_len < 0 || p->k_len < 0)
        return -1;
    if (!rows && n_rows != p->batch * p->q_heads * p->q_len)
        return -1;
    if (p->kv_int8 && (!k_scale || !v_scale || p->k_quant < 1 || p->k_quant > 2 ||
                       p->v_quant < 1 || p->v_quant > 2))
        return -1;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        const int64_t kl = p->k_len > 0 ? p->k_len : 1;
        double* s = (double*)malloc(sizeof(double) * kl);
        unsigned char* vis = (unsigned char*)malloc(kl);
        if (!s || !vis) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !vis)
                continue;
            int64_t b, h, i;
            if (rows) {
                b = rows[3 * r];
                h = rows[3 * r + 1];
                i = rows[3 * r + 2];
            } else {
                b = r / (p->q_heads * p->q_len);
                h = (r / p->q_len) % p->q_heads;
                i = r % p->q_len;
            }
            double lse_r;
            one_row(p, q, k, v, mask, key_lens, head_sink, k_scale, v_scale, doc_start, b, h, i,
                    s, vis, o + r * p->head_dim, &lse_r);
            if (lse)
                lse[r] = lse_r;
        }
        free(s);
        free(vis);
    }
    return failed ? -1 : 0;
}

/* Thread count OpenMP would use (reported with the CPU baseline). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
