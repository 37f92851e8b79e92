"""Seeded random problems through the HIP path against the oracle.

Each case draws, from its own fixed seed: the dtype, head dim (multiples of 8
and odd ones), grouped heads, layouts, lengths, causal offset, additive mask,
score-rule variants (local window, softcap, sink), document starts, and
decode against a cache (fp16/bf16, or int8 with scales). Both masked-row
policies alternate over the cases. A failure names its case index, which
reproduces it exactly.
"""
import numpy as np
import pytest

from scaled_dot_product_flash_amd import synth
import parity_util as pu

pytestmark = pytest.mark.gpu

N_CASES = 96


def draw(i: int) -> synth.Spec:
    rng = np.random.default_rng(7000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = pick(["bf16", "f16", "f32"])
    decode = dtype != "f32" and rng.random() < 0.3
    Hkv = pick([1, 2, 3, 4])
    Hq = Hkv * pick([1, 2, 3, 4, 8])
    D = pick([8, 16, 24, 32, 40, 64, 72, 96, 128, 136, 192, 256, 17, 33, 100])
    big = i >= 48                      # the second half draws longer rows and more entries
    B = int(rng.integers(1, 7 if big else 5))
    kw = dict(q_layout=pick(["bshd", "bhsd"]), lse=True, masked_rows=pick(["nan", "zero"]))
    if decode:
        Lk = int(rng.integers(1, 1200 if big else 700))
        spec = synth.Spec("random %d" % i, B, Hq, Hkv, 1, Lk, D, dtype, seed=i, kv_layout="bhsd",
                          causal=True, decode=True, lens="uniform", **kw)
    else:
        Lq = int(rng.integers(1, 600 if big else 300))
        Lk = int(rng.integers(0, 1000 if big else 400)) if rng.random() < 0.9 else 0
        causal = bool(rng.random() < 0.6)
        off = None
        if causal:
            off = pick([None, None, "end", int(rng.integers(-Lq, Lk + 1))])
        spec = synth.Spec("random %d" % i, B, Hq, Hkv, Lq, Lk, D, dtype, seed=i,
                          kv_layout=pick(["bshd", "bhsd"]), causal=causal, causal_offset=off,
                          lens=pick([None, "uniform", "cross"]) if Lk > 0 else None, **kw)
    var = {}
    if Hq * D > 0 and spec.k_len > 0:
        if spec.causal and rng.random() < 0.25:
            var["local_window"] = int(rng.integers(0, 200))
        if rng.random() < 0.2:
            var["softcap"] = float(pick([5.0, 30.0]))
        if rng.random() < 0.2:
            var["sink"] = pick(["zero", "heads"])
        if rng.random() < 0.15:
            var["docs"] = "random"
        if not decode and rng.random() < 0.25:
            var["mask"] = "keys"
    if decode and D in (64, 128) and rng.random() < 0.35:
        var["kv_quant"] = pick(["tensor", "channel", "mixed"])
    return spec.replace(**var)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(i):
    spec = draw(i)
    case = synth.generate(spec)
    policy = spec.masked_rows
    o, lse, _ = pu.run_hip(case, policy)
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what="random case %d: %s" % (i, spec))


N_STRIDED = 24


def _padded_view(torch, a, dtype, layout, pad_h, pad_d):
    """A device view of array a ([B, L, H, D] or [B, H, L, D]) inside a buffer
    with pad_h extra heads and pad_d extra elements per row."""
    t = pu.to_dev(a, dtype)
    shape = list(t.shape)
    h_ax = 2 if layout == "bshd" else 1
    shape[h_ax] += pad_h
    shape[3] += pad_d
    buf = torch.full(shape, float("nan"), dtype=t.dtype, device=t.device) if t.is_floating_point() \
        else torch.zeros(shape, dtype=t.dtype, device=t.device)
    idx = [slice(None)] * 4
    idx[h_ax] = slice(0, t.shape[h_ax])
    idx[3] = slice(0, t.shape[3])
    view = buf[tuple(idx)]
    view.copy_(t)
    return view


@pytest.mark.parametrize("i", range(N_STRIDED))
def test_random_strided_layouts(i):
    """Q/K/V/O as views into buffers padded in the head count and the head
    dim (NaN in the padding, never read), and a full per-row mask
    [B, Hq, Lq, Lk] with hidden keys, against the oracle on the plain arrays."""
    import scaled_dot_product_flash_amd as sdpa
    torch = pu.torch_mod()
    rng = np.random.default_rng(9000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = pick(["bf16", "f16", "f32"])
    decode = dtype != "f32" and rng.random() < 0.3
    Hkv = pick([1, 2, 4])
    Hq = Hkv * pick([1, 2, 4])
    D = pick([32, 64, 96, 128, 256, 40])
    B = int(rng.integers(1, 4))
    Lq = 1 if decode else int(rng.integers(1, 260))
    Lk = int(rng.integers(1, 500))
    q_layout, kv_layout = pick(["bshd", "bhsd"]), "bhsd" if decode else pick(["bshd", "bhsd"])
    causal = decode or bool(rng.random() < 0.5)
    spec = synth.Spec("strided %d" % i, B, Hq, Hkv, Lq, Lk, D, dtype, seed=100 + i,
                      q_layout=q_layout, kv_layout=kv_layout, causal=causal, decode=decode,
                      lens="uniform" if (decode or rng.random() < 0.5) else None, lse=True)
    case = synth.generate(spec)
    mask = None
    if not decode and rng.random() < 0.6:
        mask = rng.standard_normal((B, Hq, Lq, Lk)).astype(np.float32)
        mask[rng.random(mask.shape) < 0.2] = -np.inf
        case = synth.Case(spec, case.q, case.k, case.v, case.key_lens, mask)
    pad_d = pick([0, 8, 16]) if dtype != "f32" else pick([0, 4, 8])
    q = _padded_view(torch, case.q, dtype, q_layout, pick([0, 1, 3]), pad_d)
    k = _padded_view(torch, case.k, dtype, kv_layout, pick([0, 1]), pad_d)
    v = _padded_view(torch, case.v, dtype, kv_layout, pick([0, 2]), pad_d)
    out = _padded_view(torch, np.zeros_like(case.q), dtype, q_layout, pick([0, 1]), pad_d)
    lens = None if case.key_lens is None else torch.from_numpy(case.key_lens).cuda()
    mt = None if mask is None else torch.from_numpy(mask).cuda()
    policy = pick(["nan", "zero"])
    if decode:
        o, lse = sdpa.decode(q, k, v, lens, layout=q_layout, kv_layout=kv_layout, mask=mt,
                             masked_rows=policy, return_lse=True, out=out)
    else:
        o, lse = sdpa.forward(q, k, v, layout=q_layout, kv_layout=kv_layout, causal=causal,
                              key_lens=lens, mask=mt, masked_rows=policy, return_lse=True, out=out)
    torch.cuda.synchronize()
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(pu.canon(pu.to_f64(o), q_layout), ro, lse.cpu().numpy().astype(np.float64), rl,
               dtype, policy, what="strided case %d (%s, last kernel %s)" % (i, spec, sdpa.last_kernel()))
