// attn_internal.h -- kernel parameter block and launcher declarations shared by
// the host dispatch (api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_flash.h"

namespace sdpa {

// Element strides of one tensor: (b, h, r) -> b*sb + h*sh + r*sr (+ d).
struct Strides {
    int64_t sb, sh, sr;
};

// Everything a kernel needs, passed by value.  Base pointers already include
// the layout offsets.  All scores are handled in base-2 units:
// t = s * log2(e), so exp(s - m) = exp2(t - m2).
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const float* mask;     // nullable
    const int32_t* lens;   // nullable
    float* lse;            // nullable
    void* ws;              // workspace (split partials), nullable
    Strides qs, ks, vs, os, ms, ls;
    int32_t B, Hq, Hkv, Lq, Lk, D;
    int32_t group;         // Hq / Hkv
    int32_t causal;
    int32_t masked_zero;
    int64_t delta;         // causal offset (resolved), unless delta_end
    int32_t delta_end;     // 1: offset per batch entry = its clamped key length - Lq
    float scale_log2;      // scale * log2(e)
    float scale;           // scale (natural units)
    int32_t window;        // 0, or W: keys i + delta - W < j <= i + delta (causal)
    float softcap;         // 0, or c: s -> c * tanh(s / c) on scaled scores
    int32_t sink;          // 1: a sink term joins each denominator
    const float* head_sink;   // per query head sink scores (nullable: 0)
    int32_t kv_int8;       // 1: K/V are int8 with scales
    int32_t k_quant, v_quant;   // 1 per tensor, 2 per channel (g * D + d)
    const float* k_scale;
    const float* v_scale;
    const int32_t* doc_start;   // nullable: per (b, i) first visible key
    void* stage;           // workspace part for staged K/V copies (head dims not a multiple of 8)
    int32_t n_split;       // key ranges per row block (1: no split); 16-byte aligned ws
    int32_t split_len;     // keys per range (multiple of the kernel's tile)
};

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

// Records a printf-style message for attn_last_error() on this thread and
// returns `status`.
attn_status set_error(attn_status status, const char* fmt, ...);

// Launchers return the hipError_t of the launch.
hipError_t launch_generic(const Params& p, DType dt, hipStream_t s);

// window: a causal local window is set; docs: document starts are given.
void prefill_mfma_plan(int B, int Hq, int Hkv, int Lq, int Lk, int D, bool window, bool docs,
                       int* split_len, int* n_split);
size_t prefill_mfma_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, bool window,
                                    bool docs);
size_t prefill_mfma_stage_bytes(int B, int Hkv, int Lk, int D);
bool prefill_mfma_supported(const Params& p, DType dt);
bool decode_split_supported(const Params& p, DType dt);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D);
// unit: one workgroup per (entry, kv head, head slice), no workspace and no
// merge; otherwise the split over equal shares of all steps plus the merge.
bool decode_unit_preferred(const Params& p, DType dt);
hipError_t launch_decode_split(const Params& p, DType dt, hipStream_t s, bool unit);

void prefill_f32_plan(int B, int Hq, int Hkv, int Lq, int Lk, int D, int* split_len,
                      int* n_split);
size_t prefill_f32_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D);
bool prefill_f32_supported(const Params& p, DType dt);
hipError_t launch_prefill_f32(const Params& p, DType dt, hipStream_t s);
hipError_t launch_prefill_mfma(const Params& p, DType dt, hipStream_t s);

}  // namespace sdpa
