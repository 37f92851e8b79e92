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
