/*
 * sdpa_flash.h -- C ABI of the MI355X fused scaled-dot-product attention library.
 *
 * Computes, for every batch entry b, query head h and query row i,
 *
 *     O[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,g,j,:] + Mask[b,h,i,j] ) V[b,g,j,:]
 *
 * with g = h / (q_heads / kv_heads), in one pass over the keys with the online
 * normaliser, so the score matrix is never written to memory.
 *   - Definition and the running max / running sum / rescaled accumulator:
 *     OneGPU "Attention" page, introduction; llm.istanbul "05_attention",
 *     section "Online Softmax Algoritmasi" (also the LSE = m + log l output).
 *   - Problem description (batch, heads, query and key lengths, head dim, one
 *     layout per tensor with offset and batch/head/row strides, elements of a
 *     row contiguous): OneGPU "Attention", code sample and "What it covers".
 *   - Grouped heads: llm.istanbul "05_attention", section "GQA".
 *   - Key lengths, causal rule with an offset (default KLen - QLen), additive
 *     float32 mask broadcast over batch/heads/rows: OneGPU "What it covers".
 *   - Masked rows (NaN or zero) and NaN/+inf scores: OneGPU "Special values".
 *   - Key-range split with partials merged in range order, scratch sized by
 *     the shape: OneGPU "Accuracy at long key lengths", last paragraph.
 *   - Default scale 1/sqrt(head_dim) when scale is 0: ONNX GroupQueryAttention
 *     README, "Attributes" table (scale).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no pointer after the call returns and allocates no device memory.
 *     Buffers must stay valid until the work queued on `stream` completes.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the null stream) and the call returns without synchronising.
 *   - Layout fields are in ELEMENTS.  A row's head_dim elements (or a mask
 *     row's k_len elements) are contiguous.  Strides must be >= 0; a stride of
 *     0 broadcasts (used for the mask).
 *   - Every argument is validated before anything is launched: an error
 *     status means nothing was enqueued and no output was written.
 *     attn_last_error() then returns a message (thread-local).
 *   - Every element of O (and of LSE when requested) is written exactly once,
 *     masked rows included.  Two identical calls give identical bits (fixed
 *     summation order, no atomics).
 *   - Values in device memory are never trapped on: key lengths are clamped
 *     to [0, k_len]; keys at or beyond a batch entry's length are never read.
 */
#ifndef SDPA_FLASH_H
#define SDPA_FLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,      /* malformed problem or pointer                  */
    ATTN_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented               */
    ATTN_ERR_WORKSPACE = 3,    /* workspace missing or too small                */
    ATTN_ERR_HIP = 4           /* the HIP runtime refused a launch              */
} attn_status;

typedef enum attn_dtype {
    ATTN_DTYPE_F32 = 0,        /* float32 Q/K/V/O                               */
    ATTN_DTYPE_F16 = 1,        /* IEEE binary16 Q/K/V/O, float32 accumulation   */
    ATTN_DTYPE_BF16 = 2        /* bfloat16 Q/K/V/O, float32 accumulation        */
} attn_dtype;

typedef enum attn_masked_rows {
    ATTN_MASKED_ROWS_NAN = 0,  /* a row with no visible key is NaN (0/0)        */
    ATTN_MASKED_ROWS_ZERO = 1  /* ... or all zeros                              */
} attn_masked_rows;

typedef enum attn_quant {
    ATTN_QUANT_NONE = 0,
    ATTN_QUANT_PER_TENSOR = 1,
    ATTN_QUANT_PER_CHANNEL = 2
} attn_quant;

typedef enum attn_op {
    ATTN_OP_FORWARD = 0,
    ATTN_OP_DECODE = 1
} attn_op;

/* Sentinel for attn_problem.causal_offset: use k_len - q_len (OneGPU
 * "Attention", "What it covers": the default offset, the cached-decoder case). */
#define ATTN_CAUSAL_OFFSET_DEFAULT INT64_MIN

/* Sentinel for attn_problem.causal_offset: per batch entry, that entry's key
 * length (key_lens[b] clamped to [0, k_len]) minus q_len, so the last query
 * row lines up with the entry's last live key -- a chunk of q_len new rows
 * appended to a cache whose live length differs per entry (ONNX
 * GroupQueryAttention README, "Implementation variants": causal tiles bounded
 * by each entry's live length, right-aligned).  Without key_lens it equals
 * the default.                                                               */
#define ATTN_CAUSAL_OFFSET_KEY_END (INT64_MIN + 1)

/* Element (b, h, r, d) of a tensor lives at
 *   base + offset + b*batch_stride + h*head_stride + r*row_stride + d.
 * Positions-first [B, L, H, D] contiguous: batch_stride = L*H*D,
 *   head_stride = D, row_stride = H*D.
 * Heads-first [B, H, L, D] contiguous: batch_stride = H*L*D,
 *   head_stride = L*D, row_stride = D.
 * Offsets and strides are in elements and must be >= 0; a layout (Q/K/V/O,
 * and the mask and LSE when given) whose largest element index reaches 2^62
 * is rejected with ATTN_ERR_INVALID.                                          */
typedef struct attn_layout {
    int64_t offset;
    int64_t batch_stride;
    int64_t head_stride;
    int64_t row_stride;
} attn_layout;

typedef struct attn_problem {
    int32_t batch;       /* >= 0                                                 */
    int32_t q_heads;     /* >= 1                                                 */
    int32_t kv_heads;    /* >= 1, divides q_heads                                */
    int32_t q_len;       /* >= 0 (decode: exactly 1)                             */
    int32_t k_len;       /* >= 0; for decode, the cache capacity                 */
    int32_t head_dim;    /* 1..256                                               */
    int32_t dtype;       /* attn_dtype, shared by Q, K, V and O                  */
    int32_t causal;      /* 0 or 1: key j visible to row i iff j <= i + offset   */
    int64_t causal_offset; /* a value, ATTN_CAUSAL_OFFSET_DEFAULT or _KEY_END     */
    float scale;         /* 0 selects 1/sqrt(head_dim)                           */
    int32_t masked_rows; /* attn_masked_rows                                     */
    attn_layout q, k, v, o;
    /* float32 additive mask: element (b, h, i, j) at
     * mask + offset + b*batch_stride + h*head_stride + i*row_stride + j.
     * Use stride 0 to broadcast an axis.  Ignored when mask == NULL.          */
    attn_layout mask;
    /* float32 LSE: element (b, h, i) at
     * lse + offset + b*batch_stride + h*head_stride + i*row_stride.
     * Ignored when lse == NULL.                                               */
    attn_layout lse;
    /* Score-rule variants (ONNX GroupQueryAttention README, "Attributes" and
     * "Inputs").  A zero-filled tail selects none of them.                    */
    /* Local window: 0 = none; W >= 1 (causal only) = a row sees at most the W
     * keys ending at its own position i + offset, i.e. keys j with
     * i + offset - W < j <= i + offset.  The README's local_window_size L
     * (keys to the left of the position) is W = L + 1.                        */
    int32_t window;
    /* Softcap: 0 = none; c > 0 = the scaled score s becomes c * tanh(s / c)
     * before the additive mask is added (a -inf mask entry still hides).      */
    float softcap;
    /* Sink: 0 = none; 1 = each row's softmax denominator gets one more term
     * exp(sink_h), a key of score sink_h with no value: sink_h = head_sink[h]
     * (device float32[q_heads]) or 0 when head_sink is NULL (smooth softmax).
     * A row with no visible key then gives O = 0 and LSE = sink_h under both
     * masked-row policies; a NaN or +inf sink_h gives a NaN row.              */
    int32_t sink;
    const float* head_sink;
    /* Quantized key/value cache (GroupQueryAttention README, "Inputs":
     * k_scale / v_scale; "Attributes": k_quant_type / v_quant_type, cache bit
     * width 8).  kv_int8 = 0: K and V are in dtype.  kv_int8 = 1: K and V are
     * signed 8-bit integers (layout strides count elements, i.e. bytes) whose
     * value is the integer times a float32 scale: k_quant / v_quant =
     * ATTN_QUANT_PER_TENSOR uses scale[0], ATTN_QUANT_PER_CHANNEL uses
     * scale[g * head_dim + d] for kv head g.  k_scale / v_scale are device
     * pointers.  Only attn_decode runs int8 caches (fp16 or bf16 Q/O,
     * head_dim a multiple of 16 up to 256; K/V rows and strides 16-byte
     * aligned); other problems return ATTN_ERR_UNSUPPORTED.                   */
    int32_t kv_int8;
    int32_t k_quant;
    int32_t v_quant;
    const float* k_scale;
    const float* v_scale;
    /* Document mask (llm.istanbul "05_attention", line-by-line steps "Phase
     * 0" and "K-block iteration"): NULL, or device int32[batch * q_len] whose
     * element b * q_len + i is the first key of the document holding query
     * row i; keys before it are hidden for that row (with every other rule).
     * Blocks of keys below a block's first document start are skipped.       */
    const int32_t* doc_start;
} attn_problem;

/*
 * attn_forward -- fused attention over all query rows (prefill / training
 * forward / cross-attention).
 *   p          problem description (host memory, read during the call only).
 *   q, k, v    device input tensors of p->dtype, laid out per p->q/k/v.
 *              k and v may be NULL only when k_len == 0.
 *   o          device output of p->dtype per p->o (may not alias the inputs).
 *   mask       device float32 additive mask or NULL.  -inf hides a key.
 *   key_lens   device int32[batch] of real key lengths or NULL (= k_len).
 *   lse        device float32 log-sum-exp of each row's scores or NULL;
 *              -inf for a row with no visible key, NaN for a NaN row.
 *   workspace  device scratch of at least attn_workspace_size(p, FORWARD)
 *              bytes, 16-byte aligned (NULL allowed when that size is 0).
 *              It is needed when the query rows give too few workgroups to
 *              fill the GPU (bf16/fp16: at most half of its resident
 *              workgroup slots; fp32: few row blocks): the keys are then cut
 *              into ranges whose partial (max, sum, accumulator) records go
 *              to the workspace, and a second kernel merges each row's
 *              ranges in order (OneGPU "Attention", "Accuracy at long key
 *              lengths", last paragraph).  bf16/fp16 head dims that are not
 *              a multiple of 8 also keep copies of K and V there, padded to
 *              one (OneGPU "Attention", "What it covers": other head dims
 *              are padded up).  A problem with q_len == 1 that attn_decode's
 *              kernels take runs on them (for instance a cross-attention
 *              step) and needs their workspace.  The size depends on the
 *              shape only; the contents need no initialisation and are
 *              scratch.
 *   stream     hipStream_t to enqueue on.
 * Returns ATTN_OK, or an error with nothing enqueued (ATTN_ERR_WORKSPACE
 * when a needed workspace is missing or too small).
 */
attn_status attn_forward(const attn_problem* p, const void* q, const void* k, const void* v,
                         void* o, const float* mask, const int32_t* key_lens, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode -- one query row per (batch, head) against a key/value cache
 * (llm.istanbul "05_attention", section "attention_decode Farki"; ONNX
 * GroupQueryAttention README, split-K decode variants and BNSH caches).
 * Same arguments and semantics as attn_forward, with p->q_len == 1 and
 * p->k_len the cache capacity; key_lens gives the live length of each batch
 * entry.  Two modes, chosen from the shape: for large calls the live keys of
 * all (batch entry, kv head) pairs are cut, on the device from key_lens, into
 * equal contiguous shares over a fixed set of waves; each share's partial
 * (max, sum, accumulator) goes to the workspace (whose size depends on the
 * shape only) and a second kernel merges a row's partials in key order.  For
 * small calls (a few 32-key steps per wave) one workgroup takes each (batch
 * entry, kv head) pair, folds its waves' partials in key order on chip and
 * writes the outputs; the workspace is then unused.  Both modes take
 * bf16/fp16 Q/K/V (or an int8 cache) with head dims that are whole 16-byte
 * chunks up to 256, and fp32 Q/K/V with head dims that are multiples of 4 up
 * to 128.  Shapes or buffers that neither mode takes (other head dims,
 * unaligned rows) run as attn_forward would;
 * attn_workspace_size(p, ATTN_OP_DECODE) covers every case.
 */
attn_status attn_decode(const attn_problem* p, const void* q, const void* k, const void* v,
                        void* o, const float* mask, const int32_t* key_lens, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as attn_decode without the
 * workspace: the partial records go to a fixed 32 MiB device array that the
 * library keeps on every GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call there, with that device
 * current).  The call allocates nothing.  A problem whose
 * attn_workspace_size(p, ATTN_OP_DECODE) exceeds 32 MiB returns
 * ATTN_ERR_WORKSPACE.  All calls on one GPU share the array and need no
 * clearing between them (every record is written before it is read), but
 * calls that overlap in time on one GPU -- on different streams, or from
 * different threads -- race on it and must be serialised by the caller.
 */
attn_status attn_decode_noalloc(const attn_problem* p, const void* q, const void* k,
                                const void* v, void* o, const float* mask,
                                const int32_t* key_lens, float* lse, void* stream);

/*
 * attn_workspace_size -- bytes of device workspace the call `op` needs for
 * problem p (0 when it needs none).  Host-only: touches no device.
 * Returns ATTN_ERR_INVALID for a malformed problem.
 */
attn_status attn_workspace_size(const attn_problem* p, int32_t op, size_t* bytes);

/* Message for the last error on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Name of the kernel family the last successful call on this thread launched
 * ("prefill_mfma", "prefill_f32", "decode_splitk", "decode_unit" (each with
 * "_int8" for an int8 cache), "generic", or "" when the call had no work).
 * For tests and profiling; the string is static.  The environment variable
 * SDPA_FLASH_KERNEL=generic sends every call to the any-shape kernel, and
 * =decode_splitk or =decode_unit fixes the decode mode.                    */
const char* attn_last_kernel(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_FLASH_H */
