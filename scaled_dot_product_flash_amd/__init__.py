"""MI355X-native fused scaled-dot-product attention.

Thin Python binding over the C ABI in include/sdpa_flash.h (libsdpa_flash.so,
built in-tree by ``python -m scaled_dot_product_flash_amd.build``).  This
module only marshals arguments: torch tensors supply device pointers, strides
and the current HIP stream, and torch allocates the outputs and the
workspace.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and calls fail loudly when the library
is missing or a tensor is not on the GPU.

    o = forward(q, k, v, causal=True)                       # [B, L, H, D] tensors
    o, lse = forward(q, k, v, causal=True, return_lse=True)
    o = decode(q, k_cache, v_cache, key_lens, kv_layout="bhsd")
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["forward", "decode", "decode_noalloc", "workspace_size", "AttnError", "lib_path", "load_library",
           "Problem", "Layout", "SYMBOLS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsdpa_flash.so")

# Every symbol include/sdpa_flash.h declares.
SYMBOLS = ("attn_forward", "attn_decode", "attn_decode_noalloc", "attn_workspace_size",
           "attn_last_error", "attn_last_kernel", "attn_version")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
MASKED_NAN, MASKED_ZERO = 0, 1
QUANT_PER_TENSOR, QUANT_PER_CHANNEL = 1, 2
OP_FORWARD, OP_DECODE = 0, 1
_OP_DECODE_NOALLOC = 2     # binding-side tag: attn_decode_noalloc (no workspace argument)
CAUSAL_OFFSET_DEFAULT = -(1 << 63)
CAUSAL_OFFSET_KEY_END = -(1 << 63) + 1


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("attn status %d: %s" % (status, message))
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("k_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("causal_offset", ctypes.c_int64),
        ("scale", ctypes.c_float), ("masked_rows", ctypes.c_int32),
        ("q", Layout), ("k", Layout), ("v", Layout), ("o", Layout),
        ("mask", Layout), ("lse", Layout),
        ("window", ctypes.c_int32), ("softcap", ctypes.c_float),
        ("sink", ctypes.c_int32), ("head_sink", ctypes.c_void_p),
        ("kv_int8", ctypes.c_int32), ("k_quant", ctypes.c_int32), ("v_quant", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("doc_start", ctypes.c_void_p),
    ]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsdpa_flash.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libsdpa_flash.so is not built; run "
                           "`python -m scaled_dot_product_flash_amd.build` first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    call = [ctypes.POINTER(Problem), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    for name in ("attn_forward", "attn_decode"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = call
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [ctypes.POINTER(Problem), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_workspace_size.restype = ctypes.c_int
    lib.attn_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_last_kernel.restype = ctypes.c_char_p
    lib.attn_last_kernel.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().attn_last_error().decode()


def last_kernel() -> str:
    """Kernel family the last call on this thread launched."""
    return load_library().attn_last_kernel().decode()


_last_ws = 0


def last_workspace_bytes() -> int:
    """Workspace bytes the last forward/decode call of this module asked the
    library for (nonzero when it split the keys into ranges)."""
    return _last_ws


def _check(status: int):
    if status != OK:
        raise AttnError(status, last_error())


def workspace_size(problem: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().attn_workspace_size(ctypes.byref(problem), op, ctypes.byref(n)))
    return n.value


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return codes[t.dtype]


def _layout_of(t, layout: str) -> Layout:
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor, got shape %s" % (tuple(t.shape),))
    st = t.stride()
    if t.shape[3] > 1 and st[3] != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    if layout == "bshd":
        return Layout(0, st[0], st[2], st[1])
    if layout == "bhsd":
        return Layout(0, st[0], st[1], st[2])
    raise ValueError("layout must be 'bshd' or 'bhsd'")


def _dims(t, layout: str):
    if layout == "bshd":
        return t.shape[0], t.shape[2], t.shape[1], t.shape[3]   # B, H, L, D
    return t.shape[0], t.shape[1], t.shape[2], t.shape[3]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(op: int, q, k, v, *, layout: str, kv_layout: str | None, causal: bool,
         causal_offset, scale, mask, key_lens, masked_rows: str, return_lse: bool,
         local_window: int = -1, softcap: float = 0.0, sink: bool = False, head_sink=None,
         k_scale=None, v_scale=None, doc_start=None, out=None, stream=None):
    torch = _torch()
    kv_layout = kv_layout or layout
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors (there is no CPU path)")
    kv_int8 = k.dtype == torch.int8
    if kv_int8:
        if v.dtype != torch.int8 or k_scale is None or v_scale is None:
            raise TypeError("an int8 cache needs int8 k and v and both k_scale and v_scale")
    elif not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    B, Hq, Lq, D = _dims(q, layout)
    Bk, Hkv, Lk, Dk = _dims(k, kv_layout)
    if _dims(v, kv_layout) != (Bk, Hkv, Lk, Dk) or Bk != B or Dk != D:
        raise ValueError("inconsistent q/k/v shapes")
    p = Problem()
    p.batch, p.q_heads, p.kv_heads, p.q_len, p.k_len, p.head_dim = B, Hq, Hkv, Lq, Lk, D
    p.dtype = _dtype_code(q)
    p.causal = 1 if causal else 0
    if causal_offset is None:
        p.causal_offset = CAUSAL_OFFSET_DEFAULT
    elif isinstance(causal_offset, str):
        if causal_offset != "end":
            raise ValueError("causal_offset must be an int, None or 'end'")
        p.causal_offset = CAUSAL_OFFSET_KEY_END
    else:
        p.causal_offset = int(causal_offset)
    p.scale = 0.0 if scale is None else float(scale)
    p.masked_rows = {"nan": MASKED_NAN, "zero": MASKED_ZERO}[masked_rows]
    if local_window is None or local_window < 0:
        p.window = 0
    else:
        p.window = int(local_window) + 1      # keys ending at the row's own position
    p.softcap = float(softcap)
    p.sink = 1 if sink else 0
    if head_sink is not None:
        if (head_sink.dtype != torch.float32 or not head_sink.is_cuda
                or head_sink.shape != (Hq,)):
            raise TypeError("head_sink must be a float32 GPU tensor of shape [Hq]")
        head_sink = head_sink.contiguous()
        p.head_sink = head_sink.data_ptr()
    if doc_start is not None:
        if (doc_start.dtype != torch.int32 or not doc_start.is_cuda
                or doc_start.numel() != B * Lq):
            raise TypeError("doc_start must be an int32 GPU tensor of B*Lq values")
        doc_start = doc_start.contiguous()
        p.doc_start = doc_start.data_ptr()
    if kv_int8:
        p.kv_int8 = 1
        modes = []
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc.dtype != torch.float32 or not sc.is_cuda or sc.numel() not in (1, Hkv * D):
                raise TypeError("%s must be a float32 GPU tensor of 1 or Hkv*D values" % name)
            modes.append(QUANT_PER_TENSOR if sc.numel() == 1 else QUANT_PER_CHANNEL)
        k_scale, v_scale = k_scale.contiguous(), v_scale.contiguous()
        p.k_quant, p.v_quant = modes
        p.k_scale, p.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    p.q = _layout_of(q, layout)
    p.k = _layout_of(k, kv_layout)
    p.v = _layout_of(v, kv_layout)
    if out is None:
        shape = (B, Lq, Hq, D) if layout == "bshd" else (B, Hq, Lq, D)
        out = torch.empty(shape, dtype=q.dtype, device=q.device)
    elif out.dtype != q.dtype or _dims(out, layout) != (B, Hq, Lq, D):
        raise ValueError("out has the wrong dtype or shape")
    p.o = _layout_of(out, layout)
    if mask is not None:
        if mask.dtype != torch.float32 or mask.dim() != 4 or not mask.is_cuda:
            raise TypeError("mask must be a float32 GPU tensor [B|1, Hq|1, Lq|1, Lk]")
        if (mask.shape[3] != Lk or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, Hq)
                or mask.shape[2] not in (1, Lq)):
            raise ValueError("mask shape %s does not broadcast to [%d, %d, %d, %d]"
                             % (tuple(mask.shape), B, Hq, Lq, Lk))
        if Lk > 1 and mask.stride(3) != 1:
            mask = mask.contiguous()
        ms = [s if n > 1 else 0 for s, n in zip(mask.stride(), mask.shape)]
        p.mask = Layout(0, ms[0], ms[1], ms[2])
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.shape != (B,):
            raise TypeError("key_lens must be an int32 GPU tensor of shape [B]")
        key_lens = key_lens.contiguous()
    lse = None
    if return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
        p.lse = Layout(0, Hq * Lq, Lq, 1)
    lib = load_library()
    global _last_ws
    ws = None
    if op != _OP_DECODE_NOALLOC:
        ws_bytes = workspace_size(p, op)
        _last_ws = ws_bytes
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    with torch.cuda.device(q.device):
        cur = torch.cuda.current_stream(q.device)
        s = stream if stream is not None else cur
        if op == _OP_DECODE_NOALLOC:
            _check(lib.attn_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                           _ptr(mask), _ptr(key_lens), _ptr(lse),
                                           ctypes.c_void_p(s.cuda_stream)))
        else:
            fn = lib.attn_forward if op == OP_FORWARD else lib.attn_decode
            _check(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(mask),
                      _ptr(key_lens), _ptr(lse), _ptr(ws), ws_bytes,
                      ctypes.c_void_p(s.cuda_stream)))
        if s != cur:
            # Blocks allocated here (workspace, contiguous copies, outputs) were
            # taken on the current stream; keep them from being reused there
            # before the work on `s` has finished.
            for t in (ws, out, lse, mask, key_lens, head_sink, doc_start, k_scale, v_scale):
                if t is not None:
                    t.record_stream(s)
    return (out, lse) if return_lse else out


def forward(q, k, v, *, layout: str = "bshd", kv_layout: str | None = None,
            causal: bool = False, causal_offset: int | str | None = None,
            scale: float | None = None, mask=None, key_lens=None, masked_rows: str = "nan",
            return_lse: bool = False, local_window: int = -1, softcap: float = 0.0,
            sink: bool = False, head_sink=None, doc_start=None, out=None, stream=None):
    """Fused attention.  q: [B, Lq, Hq, D] ('bshd') or [B, Hq, Lq, D] ('bhsd');
    k, v likewise in ``kv_layout`` (default ``layout``).  Returns O in q's layout
    (and the float32 LSE [B, Hq, Lq] with ``return_lse``).

    causal_offset: None (Lk - Lq), an int, or "end": per batch entry its key
    length minus Lq, for a chunk of Lq new rows at the end of a cache.
    local_window: -1, or L >= 0 keys left of each causal row's position.
    softcap: 0, or c > 0 (scaled score -> c*tanh(score/c) before the mask).
    sink: add exp(head_sink[h]) (float32 GPU [Hq]; 0 when None) to each
    row's softmax denominator.
    doc_start: int32 GPU [B, Lq]: row i of entry b sees only keys
    j >= doc_start[b, i] (packed documents)."""
    return _run(OP_FORWARD, q, k, v, layout=layout, kv_layout=kv_layout, causal=causal,
                causal_offset=causal_offset, scale=scale, mask=mask, key_lens=key_lens,
                masked_rows=masked_rows, return_lse=return_lse, local_window=local_window,
                softcap=softcap, sink=sink, head_sink=head_sink, doc_start=doc_start, out=out,
                stream=stream)


def decode(q, k_cache, v_cache, key_lens=None, *, layout: str = "bshd", kv_layout: str = "bhsd",
           scale: float | None = None, mask=None, masked_rows: str = "nan",
           return_lse: bool = False, local_window: int = -1, softcap: float = 0.0,
           sink: bool = False, head_sink=None, k_scale=None, v_scale=None, doc_start=None,
           out=None, stream=None):
    """One query row per (batch, head) against a K/V cache of capacity Lk with
    live lengths ``key_lens`` (int32 [B]).  The row is the newest position of
    its entry (end-aligned causal offset), so every live key is visible and a
    local window counts back from the entry's last live key.  An int8 cache
    (k_cache / v_cache int8) takes float32 k_scale / v_scale of 1 value (per
    tensor) or Hkv*D values (per channel, index g*D + d)."""
    return _run(OP_DECODE, q, k_cache, v_cache, layout=layout, kv_layout=kv_layout,
                causal=True, causal_offset="end", scale=scale, mask=mask, key_lens=key_lens,
                masked_rows=masked_rows, return_lse=return_lse, local_window=local_window,
                softcap=softcap, sink=sink, head_sink=head_sink, k_scale=k_scale,
                v_scale=v_scale, doc_start=doc_start, out=out, stream=stream)


def decode_noalloc(q, k_cache, v_cache, key_lens=None, *, layout: str = "bshd",
                   kv_layout: str = "bhsd", scale: float | None = None, mask=None,
                   masked_rows: str = "nan", return_lse: bool = False, local_window: int = -1,
                   softcap: float = 0.0, sink: bool = False, head_sink=None, k_scale=None,
                   v_scale=None, doc_start=None, out=None, stream=None):
    """decode() through attn_decode_noalloc: the library takes no workspace
    and allocates nothing (its partial records go to a fixed device array it
    holds per GPU).  Pass ``out`` (and no ``return_lse``) for a call that
    allocates nothing on the torch side either."""
    return _run(_OP_DECODE_NOALLOC, q, k_cache, v_cache, layout=layout, kv_layout=kv_layout,
                causal=True, causal_offset="end", scale=scale, mask=mask, key_lens=key_lens,
                masked_rows=masked_rows, return_lse=return_lse, local_window=local_window,
                softcap=softcap, sink=sink, head_sink=head_sink, k_scale=k_scale,
                v_scale=v_scale, doc_start=doc_start, out=out, stream=stream)
