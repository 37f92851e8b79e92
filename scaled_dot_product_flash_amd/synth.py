"""Seeded synthetic inputs for attention problems.

This module holds no attention arithmetic: it only draws inputs.  Both the
HIP path (through the tests and the benchmark) and the float64 oracle are fed
from it, so the two sides see identical bits.

Recipe (the same for every workload): numpy PCG64 ``default_rng(seed)``;
draw order Q, K, V, then key lengths, then the mask, then per-head sink
scores, then int8-cache scales, then document starts; values are i.i.d.
N(0, 1) in float32 (sink
scores 2 * N(0, 1)), rounded to nearest-even into the storage type (float16
via numpy, bfloat16 by bit rounding, kept as uint16 bit patterns).  An int8
cache keeps K and V as float32 draws and quantizes them at the end: scale
4/127 per tensor, or (0.5 + U[0, 1)) * 4/127 per (kv head, head-dim)
channel; value = clip(round_half_even(x / scale), -127, 127).  Packed
documents: lengths uniform in [1, 2 * doc_mean) placed back to back until
the entry's q_len positions are filled (doc_start = each position's
document's first index); 'random' starts are uniform in [0, k_len].
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Union

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


@dataclass(frozen=True)
class Spec:
    """Shape and options of one attention problem.

    Layout tags: 'bshd' = [batch, positions, heads, head_dim] (positions
    first), 'bhsd' = [batch, heads, positions, head_dim] (heads first).
    ``q_layout`` applies to Q and O, ``kv_layout`` to K and V.
    """
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    q_len: int
    k_len: int
    head_dim: int
    dtype: str
    seed: int
    q_layout: str = "bshd"
    kv_layout: str = "bshd"
    causal: bool = False
    causal_offset: Optional[Union[int, str]] = None   # None, an int or 'end'
    lse: bool = False
    decode: bool = False
    lens: Optional[str] = None        # None, 'uniform' (in [1, k_len]), 'full', 'cross' or
                                      # 'chunk' (in [q_len, k_len]: the chunk fits)
    mask: Optional[str] = None        # None or 'keys' ([B,1,1,Lk], 10% -inf)
    masked_rows: str = "nan"
    lens_zero_at: int = 5             # 'cross' lengths: this batch entry has length 0
    lens_full_at: int = 7             # ... and this one has the full k_len
    mask_all_at: int = 2              # 'keys' mask: this batch entry is fully -inf
    mask_p: float = 0.1
    local_window: int = -1            # -1, or keys left of each causal row's position
    softcap: float = 0.0              # 0, or c > 0
    sink: Optional[str] = None        # None, 'zero' (smooth softmax) or 'heads' (drawn)
    docs: Optional[str] = None        # None, 'packed' or 'random' (doc_start per row)
    doc_mean: int = 512
    kv_quant: Optional[str] = None    # int8 cache: None, 'tensor', 'channel' or 'mixed'
                                      # ('mixed': K per tensor, V per channel)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)

    @property
    def flops(self) -> float:
        """4*B*Hq*Lq*Lk*D, halved under the causal rule."""
        f = 4.0 * self.batch * self.q_heads * self.q_len * self.k_len * self.head_dim
        return f / 2 if self.causal and not self.decode else f


# The five workloads the measurements and parity tests are built on.
TINY_F32 = Spec("tiny fp32 MHA B1 H2 L64 D32", 1, 2, 2, 64, 64, 32, "f32", seed=1)
CAUSAL_GQA_F32 = Spec("fp32 causal GQA prefill B2 H12/4 L512 D64", 2, 12, 4, 512, 512, 64,
                      "f32", seed=2, causal=True, causal_offset=0, lse=True)
CAUSAL_GQA_BF16 = Spec("bf16 causal GQA prefill B4 H32/8 L4096 D128", 4, 32, 8, 4096, 4096,
                       128, "bf16", seed=3, causal=True, causal_offset=0, lse=True)
DECODE_F16 = Spec("fp16 decode B64 H32/8 cache8192 D128", 64, 32, 8, 1, 8192, 128, "f16",
                  seed=4, kv_layout="bhsd", causal=True, decode=True, lens="uniform")
# A chunk of 128 new query rows per entry at the end of a cache whose live
# length differs per entry (end-aligned causal rule).
CHUNK_F16 = Spec("fp16 chunked prefill B16 H32/8 Lq128 cache8192 D128", 16, 32, 8, 128, 8192,
                 128, "f16", seed=6, kv_layout="bhsd", causal=True, causal_offset="end",
                 lse=True, lens="chunk")
CROSS_MASK_F16 = Spec("fp16 cross-attention B8 H16 Lq1024 Lk2048 D64 mask+lens", 8, 16, 16,
                      1024, 2048, 64, "f16", seed=5, q_layout="bhsd", kv_layout="bhsd",
                      lens="cross", mask="keys")

WORKLOADS = {
    "tiny_f32": TINY_F32,
    "causal_gqa_f32": CAUSAL_GQA_F32,
    "causal_gqa_bf16": CAUSAL_GQA_BF16,
    "decode_f16": DECODE_F16,
    "cross_mask_f16": CROSS_MASK_F16,
}

# Score-rule variants on the prefill and decode shapes: a 1024-key causal
# local window; softcap 30 with per-head sinks.
WINDOW_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D128, local window 1023", local_window=1023,
    seed=7)
SOFTCAP_SINK_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D128, softcap 30, head sinks", softcap=30.0,
    sink="heads", seed=8)
DECODE_WINDOW_F16 = DECODE_F16.replace(
    name="fp16 decode B64 H32/8 cache8192 D128, local window 2047, head sinks",
    local_window=2047, sink="heads", seed=9)

# The decode workload with an int8 cache and per-channel scales.
DECODE_INT8_F16 = DECODE_F16.replace(
    name="fp16 decode B64 H32/8 cache8192 D128, int8 cache, per-channel scales",
    kv_quant="channel", seed=10)

# Packed documents (mean length 512) on the bf16 causal prefill shape.
DOCS_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D128, packed documents (mean 512)",
    docs="packed", doc_mean=512, seed=11)

# One long sequence: a chunk of 512 new rows at the end of a 32768-key cache
# (64 query blocks, a quarter of the GPU's workgroup slots: the keys are cut
# into ranges).
LONG_CHUNK_BF16 = Spec("bf16 chunked prefill B1 H32/8 Lq512 cache32768 D128", 1, 32, 8, 512,
                       32768, 128, "bf16", seed=14, kv_layout="bhsd", causal=True,
                       causal_offset="end", lse=True)

# Head dims beyond 64 / 128 on the matrix cores (96 runs padded to 128).
D256_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D256", head_dim=256, seed=12)
D96_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D96", head_dim=96, seed=13)

# Head dims that are not a multiple of 8 (bf16, run padded to 128 with K/V
# staged) and an fp32 head dim between the fp32 kernel's tiles (96 -> 128).
D100_BF16 = CAUSAL_GQA_BF16.replace(
    name="bf16 causal GQA prefill B4 H32/8 L4096 D100", head_dim=100, seed=15)
D96_F32 = CAUSAL_GQA_BF16.replace(
    name="fp32 causal GQA prefill B4 H32/8 L4096 D96", dtype="f32", head_dim=96, seed=16)
# Decode at a head dim below 128 (run padded to 128 by the split decode path).
DECODE_D96_F16 = DECODE_F16.replace(name="fp16 decode B64 H32/8 cache8192 D96", head_dim=96,
                                    seed=17)
# The decode shape with fp32 Q/K/V.
DECODE_F32 = DECODE_F16.replace(name="fp32 decode B64 H32/8 cache8192 D128", dtype="f32", seed=18)

# Workloads of the extensions beyond the five (measured and tested the same way).
EXTRA_WORKLOADS = {
    "chunk_f16": CHUNK_F16,
    "long_chunk_bf16": LONG_CHUNK_BF16,
    "window_bf16": WINDOW_BF16,
    "softcap_sink_bf16": SOFTCAP_SINK_BF16,
    "decode_window_f16": DECODE_WINDOW_F16,
    "decode_int8_f16": DECODE_INT8_F16,
    "docs_bf16": DOCS_BF16,
    "d256_bf16": D256_BF16,
    "d96_bf16": D96_BF16,
    "d100_bf16": D100_BF16,
    "d96_f32": D96_F32,
    "decode_d96_f16": DECODE_D96_F16,
    "decode_f32": DECODE_F32,
}

# The model shapes the OneGPU "Attention" page times (its "Performance"
# tables): 12 heads throughout, no mask; MiniLM with head dim 32, BERT-base
# and Whisper-small with 64.  The page does not state the Whisper batch;
# 1 is taken.  The Whisper decoder row is read as one new query row against
# 448 cached keys, the cross-attention row as one query row against the
# encoder's 1500 keys.  Random inputs of those shapes: no trained weights.
MINILM_B8 = Spec("MiniLM B8 S128 H12 D32", 8, 12, 12, 128, 128, 32, "f32", seed=20)
BERT_B8_S512 = Spec("BERT-base B8 S512 H12 D64", 8, 12, 12, 512, 512, 64, "f32", seed=21)
WHISPER_ENC = Spec("Whisper-small encoder B1 H12 L1500 D64", 1, 12, 12, 1500, 1500, 64, "f32",
                   seed=22)
WHISPER_DEC = Spec("Whisper-small decoder step B1 H12 cache448 D64", 1, 12, 12, 1, 448, 64,
                   "f32", seed=23, kv_layout="bhsd", causal=True, decode=True, lens="full")
WHISPER_CROSS = Spec("Whisper-small cross-attention B1 H12 Lq1 Lk1500 D64", 1, 12, 12, 1, 1500,
                     64, "f32", seed=24)


def _both(spec: Spec):
    return [spec, spec.replace(name=spec.name + " fp16", dtype="f16", seed=spec.seed + 100)]


PAGE_SHAPES = {s.name: s for base in (MINILM_B8, BERT_B8_S512, WHISPER_ENC, WHISPER_DEC,
                                      WHISPER_CROSS) for s in _both(base)}


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN kept NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return round_bf16_bits(x)
    raise ValueError(dtype)


def shape_of(spec: Spec, which: str):
    """Array shape of 'q'/'o' or 'k'/'v' in the spec's layout."""
    if which in ("q", "o"):
        L, H, lay = spec.q_len, spec.q_heads, spec.q_layout
    else:
        L, H, lay = spec.k_len, spec.kv_heads, spec.kv_layout
    if lay == "bshd":
        return (spec.batch, L, H, spec.head_dim)
    return (spec.batch, H, L, spec.head_dim)


@dataclass
class Case:
    spec: Spec
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    key_lens: Optional[np.ndarray]
    mask: Optional[np.ndarray]
    head_sink: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    doc_start: Optional[np.ndarray] = None


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORAGE[dtype])
    step = 1 << 26
    for s in range(0, n, step):          # chunked: keeps the float32 staging small
        m = min(step, n - s)
        out[s:s + m] = to_storage(rng.standard_normal(m, dtype=np.float32), dtype)
    return out.reshape(shape)


def generate(spec: Spec) -> Case:
    rng = np.random.default_rng(spec.seed)
    q = _normal(rng, shape_of(spec, "q"), spec.dtype)
    kv_dtype = "f32" if spec.kv_quant else spec.dtype
    k = _normal(rng, shape_of(spec, "k"), kv_dtype)
    v = _normal(rng, shape_of(spec, "v"), kv_dtype)
    lens = None
    if spec.lens == "uniform":
        lens = rng.integers(1, spec.k_len + 1, size=spec.batch).astype(np.int32)
    elif spec.lens == "cross":
        lens = rng.integers(1, spec.k_len + 1, size=spec.batch).astype(np.int32)
        if spec.lens_zero_at < spec.batch:
            lens[spec.lens_zero_at] = 0
        if spec.lens_full_at < spec.batch:
            lens[spec.lens_full_at] = spec.k_len
    elif spec.lens == "full":
        lens = np.full(spec.batch, spec.k_len, dtype=np.int32)
    elif spec.lens == "chunk":
        lens = rng.integers(min(spec.q_len, spec.k_len), spec.k_len + 1,
                            size=spec.batch).astype(np.int32)
    elif spec.lens is not None:
        raise ValueError(spec.lens)
    mask = None
    if spec.mask == "keys":
        hide = rng.random((spec.batch, spec.k_len)) < spec.mask_p
        mask = np.where(hide, np.float32(-np.inf), np.float32(0.0)).astype(np.float32)
        if spec.mask_all_at < spec.batch:
            mask[spec.mask_all_at, :] = -np.inf
        mask = mask.reshape(spec.batch, 1, 1, spec.k_len)
    elif spec.mask is not None:
        raise ValueError(spec.mask)
    head_sink = None
    if spec.sink == "heads":
        head_sink = (2.0 * rng.standard_normal(spec.q_heads, dtype=np.float32)).astype(np.float32)
    elif spec.sink not in (None, "zero"):
        raise ValueError(spec.sink)
    k_scale = v_scale = None
    if spec.kv_quant:
        if spec.kv_quant not in ("tensor", "channel", "mixed"):
            raise ValueError(spec.kv_quant)
        base = np.float32(4.0 / 127.0)
        n_ch = spec.kv_heads * spec.head_dim
        chan = ((0.5 + rng.random(2 * n_ch, dtype=np.float32)) * base).astype(np.float32)
        k_scale = (np.array([base], np.float32) if spec.kv_quant in ("tensor", "mixed")
                   else chan[:n_ch])
        v_scale = np.array([base], np.float32) if spec.kv_quant == "tensor" else chan[n_ch:]
        k = _quantize(k, k_scale, spec)
        v = _quantize(v, v_scale, spec)
    doc_start = None
    if spec.docs == "packed":
        doc_start = np.empty((spec.batch, spec.q_len), np.int32)
        for b in range(spec.batch):
            pos = 0
            while pos < spec.q_len:
                n = int(rng.integers(1, 2 * spec.doc_mean))
                doc_start[b, pos:pos + n] = pos
                pos += n
    elif spec.docs == "random":
        doc_start = rng.integers(0, spec.k_len + 1, size=(spec.batch, spec.q_len)).astype(np.int32)
    elif spec.docs is not None:
        raise ValueError(spec.docs)
    return Case(spec, q, k, v, lens, mask, head_sink, k_scale, v_scale, doc_start)


def _quantize(x: np.ndarray, scale: np.ndarray, spec: Spec) -> np.ndarray:
    """float32 cache -> int8 codes with a per-tensor or per-channel scale."""
    if scale.size == 1:
        s = scale[0]
    else:
        s = scale.reshape(spec.kv_heads, spec.head_dim)
        s = s[None, None] if spec.kv_layout == "bshd" else s[None, :, None, :]
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8)
