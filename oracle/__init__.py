"""Plain float64 CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product package never imports it.  It shares no code
with the HIP path.

The arithmetic lives in ``sdpa_oracle.c`` (three-pass softmax attention in
double, one query row at a time).  This module only marshals numpy arrays into
that C function.  Semantics (OneGPU "Attention": intro formula, "What it
covers", "Special values"; llm.istanbul 05_attention: "GQA", "Online Softmax -
Niye?", LSE in "Online Softmax Algoritmasi") are documented in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdpa_oracle.c")
_LIB = os.path.join(_HERE, "libsdpa_oracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("q_heads", ctypes.c_int64),
        ("kv_heads", ctypes.c_int64),
        ("q_len", ctypes.c_int64),
        ("k_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("has_offset", ctypes.c_int32),
        ("masked_zero", ctypes.c_int32),
        ("causal_offset", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("qs", ctypes.c_int64 * 3),
        ("ks", ctypes.c_int64 * 3),
        ("vs", ctypes.c_int64 * 3),
        ("ms", ctypes.c_int64 * 3),
        ("window", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("softcap", ctypes.c_double),
        ("kv_int8", ctypes.c_int32),
        ("k_quant", ctypes.c_int32),
        ("v_quant", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [
            ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().oracle_max_threads()


def decode_f16(bits: int) -> float:
    return _load().oracle_decode_f16(bits)


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(bits)


def _bhs_strides(a: np.ndarray, layout: str):
    """Element strides (batch, head, row) of a 4-D array; innermost must be 1."""
    es = [s // a.itemsize for s in a.strides]
    if a.shape[3] > 1 and es[3] != 1:
        raise ValueError("innermost dimension must be contiguous")
    if layout == "bshd":      # [B, L, H, D] (positions first)
        return es[0], es[2], es[1]
    if layout == "bhsd":      # [B, H, L, D] (heads first)
        return es[0], es[1], es[2]
    raise ValueError("layout must be 'bshd' or 'bhsd'")


def _dims(a: np.ndarray, layout: str):
    if layout == "bshd":
        return a.shape[0], a.shape[2], a.shape[1], a.shape[3]   # B, H, L, D
    return a.shape[0], a.shape[1], a.shape[2], a.shape[3]


def attention(q, k, v, *, dtype: str, layout: str = "bshd", kv_layout: str | None = None,
              causal: bool = False, causal_offset: int | str | None = None,
              scale: float | None = None, mask: np.ndarray | None = None,
              key_lens: np.ndarray | None = None, masked_rows: str = "nan",
              window: int = -1, softcap: float = 0.0, sink: bool = False,
              head_sink: np.ndarray | None = None,
              k_scale: np.ndarray | None = None, v_scale: np.ndarray | None = None,
              doc_start: np.ndarray | None = None,
              rows: np.ndarray | None = None, threads: int = 0):
    """Reference attention in float64.

    q, k, v: numpy arrays in storage form (float32, float16, or uint16 holding
    bfloat16 bits), 4-D in ``layout`` ('bshd' = [B, L, H, D], 'bhsd' =
    [B, H, L, D]); ``kv_layout`` defaults to ``layout``.
    mask: float32, 4-D [B|1, Hq|1, Lq|1, Lk] (size-1 axes broadcast).
    key_lens: int32 [B] (real lengths, clamped to [0, Lk]).
    causal_offset: None (Lk - Lq), an int, or "end": per batch entry the
    clamped key length minus Lq (the last query row sees the last live key).
    window: -1, or W >= 0 keys left of each causal row's position.
    softcap: 0, or c > 0 (score -> c*tanh(score/c) before the mask).
    sink: add exp(head_sink[h]) (0 without head_sink) to each denominator;
    head_sink: float32 [Hq] or None.
    k, v may be int8 (a quantized cache); then k_scale / v_scale are float32
    of size 1 (per tensor) or Hkv * D (per channel, index g * D + d) and an
    element's value is the integer times its scale.
    doc_start: int32 [B, Lq] or None: row i of entry b sees only keys
    j >= doc_start[b, i] (its document's first key).
    rows: optional int64 [n, 3] of (b, h, i) to compute; default every row.

    Returns (O, LSE): O is [B, Hq, Lq, D] (or [n, D] with ``rows``) float64,
    LSE is [B, Hq, Lq] (or [n]).
    """
    kv_layout = kv_layout or layout
    st = STORAGE[dtype]
    kv_int8 = k.dtype == np.int8
    keep_scales = []
    for name, a in (("q", q), ("k", k), ("v", v)):
        want = np.int8 if (kv_int8 and name != "q") else st
        if a.dtype != want or a.ndim != 4:
            raise TypeError("%s must be a 4-D %s array" % (name, np.dtype(want)))
    B, Hq, Lq, D = _dims(q, layout)
    Bk, Hkv, Lk, Dk = _dims(k, kv_layout)
    if _dims(v, kv_layout) != (Bk, Hkv, Lk, Dk) or Bk != B or Dk != D:
        raise ValueError("inconsistent shapes")
    p = _Problem()
    p.batch, p.q_heads, p.kv_heads, p.q_len, p.k_len, p.head_dim = B, Hq, Hkv, Lq, Lk, D
    p.dtype = DTYPES[dtype]
    p.causal = 1 if causal else 0
    if causal_offset is None:
        p.has_offset, p.causal_offset = 0, 0
    elif isinstance(causal_offset, str):
        if causal_offset != "end":
            raise ValueError("causal_offset must be an int, None or 'end'")
        p.has_offset, p.causal_offset = 2, 0
    else:
        p.has_offset, p.causal_offset = 1, int(causal_offset)
    p.masked_zero = {"nan": 0, "zero": 1}[masked_rows]
    p.scale = 0.0 if scale is None else float(scale)
    p.window = int(window)
    p.softcap = float(softcap)
    p.sink = 1 if sink else 0
    scale_ptrs = [None, None]
    if kv_int8:
        p.kv_int8 = 1
        modes = []
        for j, sc in enumerate((k_scale, v_scale)):
            if sc is None:
                raise ValueError("an int8 cache needs k_scale and v_scale")
            sc = np.ascontiguousarray(sc, dtype=np.float32).reshape(-1)
            if sc.size == 1:
                modes.append(1)
            elif sc.size == Hkv * D:
                modes.append(2)
            else:
                raise ValueError("a scale has 1 or Hkv*D entries")
            keep_scales.append(sc)
            scale_ptrs[j] = sc.ctypes.data
        p.k_quant, p.v_quant = modes
    p.qs[:] = _bhs_strides(q, layout)
    p.ks[:] = _bhs_strides(k, kv_layout)
    p.vs[:] = _bhs_strides(v, kv_layout)
    keep = [q, k, v]
    mask_ptr = None
    if mask is not None:
        mask = np.asarray(mask)
        if (mask.dtype != np.float32 or mask.ndim != 4 or mask.shape[3] != Lk
                or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, Hq)
                or mask.shape[2] not in (1, Lq)):
            raise TypeError("mask must be float32 [B|1, Hq|1, Lq|1, Lk]")
        if mask.shape[3] > 1 and mask.strides[3] != 4:
            mask = np.ascontiguousarray(mask)
        ms = [s // 4 if n > 1 else 0 for s, n in zip(mask.strides, mask.shape)]
        p.ms[:] = ms[:3]
        keep.append(mask)
        mask_ptr = mask.ctypes.data
    lens_ptr = None
    if key_lens is not None:
        key_lens = np.ascontiguousarray(key_lens, dtype=np.int32)
        if key_lens.shape != (B,):
            raise ValueError("key_lens must be int32 [B]")
        keep.append(key_lens)
        lens_ptr = key_lens.ctypes.data
    sink_ptr = None
    if head_sink is not None:
        head_sink = np.ascontiguousarray(head_sink, dtype=np.float32)
        if head_sink.shape != (Hq,):
            raise ValueError("head_sink must be float32 [Hq]")
        keep.append(head_sink)
        sink_ptr = head_sink.ctypes.data
    doc_ptr = None
    if doc_start is not None:
        doc_start = np.ascontiguousarray(doc_start, dtype=np.int32)
        if doc_start.shape != (B, Lq):
            raise ValueError("doc_start must be int32 [B, Lq]")
        keep.append(doc_start)
        doc_ptr = doc_start.ctypes.data
    if rows is None:
        n = B * Hq * Lq
        rows_ptr = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        if n and ((rows < 0).any() or (rows[:, 0] >= B).any() or (rows[:, 1] >= Hq).any()
                  or (rows[:, 2] >= Lq).any()):
            raise ValueError("rows out of range")
        keep.append(rows)
        rows_ptr = rows.ctypes.data
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attention(ctypes.byref(p), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                  mask_ptr, lens_ptr, sink_ptr, scale_ptrs[0], scale_ptrs[1],
                                  doc_ptr, rows_ptr, n, o.ctypes.data,
                                  lse.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle rejected the problem")
    if rows is None:
        return o.reshape(B, Hq, Lq, D), lse.reshape(B, Hq, Lq)
    return o, lse
