"""Helpers for the GPU parity tests: move synthetic cases to the device, run
the HIP path through the binding, run the oracle, and compare by the rule

  * oracle NaN            -> GPU NaN
  * oracle empty row      -> GPU exactly 0 (zero policy) / NaN (NaN policy),
                             LSE exactly -inf
  * otherwise             -> GPU finite and |GPU - oracle| <= tol

with tol = 1e-4 (fp32), 5e-3 (fp16), 2e-2 (bf16) max-abs on unit-variance
inputs.

LSE has bounds of its own, derived from the arithmetic rather than from the
output tolerance.  On the bf16/fp16 paths the running sum l adds the
probabilities after they are rounded to the element type (OneGPU "Attention",
"Matrix hardware": numerator and denominator see the same rounded p), so
l_gpu = sum_j p_j (1 + e_j) with |e_j| <= 2^-9 (bf16) or 2^-12 (fp16), and
|LSE_gpu - LSE| <= -ln(1 - 2^-9) = 1.96e-3 (bf16), 2.4e-4 (fp16), plus fp32
rounding of the sums and of exp2/log2.  The rounding of m*c cancels between
the exponents and the epilogue's m*c + log2 l.  The bounds below are those
figures with 2x (bf16) and 4x (fp16) slack; fp32 does not round p.
"""
from __future__ import annotations

import numpy as np

import oracle
import scaled_dot_product_flash_amd as sdpa
from scaled_dot_product_flash_amd import synth

TOL = {"f32": 1e-4, "f16": 5e-3, "bf16": 2e-2}
LSE_TOL = {"f32": 1e-4, "f16": 1e-3, "bf16": 4e-3}

# Largest errors seen in this session, per dtype (reported by conftest.py at
# the end of a run, so the measured margins can be quoted).
MAX_SEEN = {"o": {}, "lse": {}}


def _note(kind: str, dtype: str, err: float):
    d = MAX_SEEN[kind]
    if err > d.get(dtype, 0.0):
        d[dtype] = float(err)


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray, dtype: str):
    torch = torch_mod()
    if a.dtype == np.int8:
        return torch.from_numpy(a).to("cuda")
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def canon(o: np.ndarray, layout: str) -> np.ndarray:
    """[B, L, H, D] or [B, H, L, D] -> [B, H, L, D]."""
    return np.transpose(o, (0, 2, 1, 3)) if layout == "bshd" else o


def run_hip(case: synth.Case, policy: str = "nan", *, return_lse=None, tensors=None):
    """Returns (O [B,Hq,Lq,D] float64, LSE [B,Hq,Lq] float64 or None, raw tensors)."""
    s = case.spec
    torch = torch_mod()
    if tensors is None:
        tensors = dict(q=to_dev(case.q, s.dtype), k=to_dev(case.k, s.dtype),
                       v=to_dev(case.v, s.dtype),
                       mask=None if case.mask is None else torch.from_numpy(case.mask).cuda(),
                       lens=None if case.key_lens is None else torch.from_numpy(case.key_lens).cuda(),
                       sink=None if case.head_sink is None else torch.from_numpy(case.head_sink).cuda(),
                       docs=None if case.doc_start is None else torch.from_numpy(case.doc_start).cuda())
    var = dict(local_window=s.local_window, softcap=s.softcap, sink=s.sink is not None,
               head_sink=tensors.get("sink"), doc_start=tensors.get("docs"))
    dvar = {}
    if case.k_scale is not None:
        dvar = dict(k_scale=torch.from_numpy(case.k_scale).cuda(),
                    v_scale=torch.from_numpy(case.v_scale).cuda())
    want_lse = s.lse if return_lse is None else return_lse
    if s.decode:
        r = sdpa.decode(tensors["q"], tensors["k"], tensors["v"], tensors["lens"],
                        layout=s.q_layout, kv_layout=s.kv_layout, mask=tensors["mask"],
                        masked_rows=policy, return_lse=want_lse, **var, **dvar)
    else:
        r = sdpa.forward(tensors["q"], tensors["k"], tensors["v"], layout=s.q_layout,
                         kv_layout=s.kv_layout, causal=s.causal, causal_offset=s.causal_offset,
                         mask=tensors["mask"], key_lens=tensors["lens"], masked_rows=policy,
                         return_lse=want_lse, **var)
    torch.cuda.synchronize()
    o, lse = (r if want_lse else (r, None))
    O = canon(to_f64(o), s.q_layout)
    L = None if lse is None else lse.cpu().numpy().astype(np.float64)
    return O, L, (o, lse, tensors)


def run_oracle(case: synth.Case, policy: str = "nan", rows=None):
    s = case.spec
    # Decode rows are the newest position of their entry (end-aligned offset).
    off = "end" if s.decode else s.causal_offset
    return oracle.attention(case.q, case.k, case.v, dtype=s.dtype, layout=s.q_layout,
                            kv_layout=s.kv_layout, causal=s.causal, causal_offset=off,
                            mask=case.mask, key_lens=case.key_lens, masked_rows=policy,
                            window=s.local_window, softcap=s.softcap, sink=s.sink is not None,
                            head_sink=case.head_sink, k_scale=case.k_scale,
                            v_scale=case.v_scale, doc_start=case.doc_start, rows=rows)


def compare(gpu_o, ref_o, gpu_lse, ref_lse, dtype: str, policy: str, what: str = ""):
    """Raise AssertionError with a description on the first violated rule.
    gpu_o/ref_o: [..., D]; *_lse: [...] (same leading shape) or None."""
    tol = TOL[dtype]
    ref_nan = np.isnan(ref_o)
    gpu_nan = np.isnan(gpu_o)
    if not (gpu_nan[ref_nan]).all():
        n = int((~gpu_nan[ref_nan]).sum())
        raise AssertionError("%s: %d outputs should be NaN" % (what, n))
    fin = ~ref_nan
    if (gpu_nan & fin).any():
        raise AssertionError("%s: %d unexpected NaN outputs" % (what, int((gpu_nan & fin).sum())))
    if not np.isfinite(gpu_o[fin]).all():
        raise AssertionError("%s: non-finite outputs where the oracle is finite" % what)
    err = np.abs(gpu_o[fin] - ref_o[fin]).max(initial=0.0)
    _note("o", dtype, err)
    if err > tol:
        idx = np.unravel_index(np.argmax(np.where(fin, np.abs(gpu_o - ref_o), -1)), ref_o.shape)
        raise AssertionError("%s: max |gpu - oracle| = %.3g > %.1g at %s (gpu %r, oracle %r)"
                             % (what, err, tol, idx, gpu_o[idx], ref_o[idx]))
    if ref_lse is not None:
        empty = ref_lse == -np.inf
        if policy == "zero" and empty.any():
            z = gpu_o[empty]
            if not (z == 0).all():
                raise AssertionError("%s: zero-policy rows are not exactly 0" % what)
        if gpu_lse is not None:
            if not (np.isnan(gpu_lse) == np.isnan(ref_lse)).all():
                raise AssertionError("%s: LSE NaN pattern differs" % what)
            if not (gpu_lse[empty] == -np.inf).all():
                raise AssertionError("%s: LSE of empty rows is not -inf" % what)
            ok = np.isfinite(ref_lse)
            if not np.isfinite(gpu_lse[ok]).all():
                raise AssertionError("%s: non-finite LSE where the oracle is finite" % what)
            lerr = np.abs(gpu_lse[ok] - ref_lse[ok]).max(initial=0.0)
            _note("lse", dtype, lerr)
            if lerr > LSE_TOL[dtype]:
                raise AssertionError("%s: LSE error %.3g > %.1g" % (what, lerr, LSE_TOL[dtype]))
    return err


def sample_rows(spec: synth.Spec, n: int, seed: int = 0) -> np.ndarray:
    """Deterministic sample of (b, h, i) rows: random ones plus the corners."""
    rng = np.random.default_rng(1000 + seed)
    B, H, L = spec.batch, spec.q_heads, spec.q_len
    rows = [(0, 0, 0), (B - 1, H - 1, L - 1), (0, H - 1, L // 2), (B - 1, 0, 0)]
    rows += [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(L))) for _ in range(n)]
    return np.array(rows, dtype=np.int64)
