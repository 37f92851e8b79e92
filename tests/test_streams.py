"""Stream and graph use of the binding: a call enqueued on a caller's stream,
and calls captured in a HIP graph and replayed.  Both must give the same bits
as the same call made eagerly on the current stream (the kernels are
deterministic and the key-range plan depends on the shape only).
"""
import numpy as np
import pytest

import scaled_dot_product_flash_amd as sdpa
from scaled_dot_product_flash_amd import synth
import parity_util as pu

pytestmark = pytest.mark.gpu

# A prefill whose query blocks are too few for the GPU (the keys are cut into
# ranges: workspace + merge kernel), a split decode (workspace + merge) and a
# small decode (one workgroup per unit, folding in LDS).
CASES = {
    "chunk_split_f16": synth.CHUNK_F16.replace(batch=2, q_heads=8, kv_heads=2, q_len=64,
                                               k_len=2048, lens="cross", lens_zero_at=9,
                                               lens_full_at=1, seed=21),
    "decode_split_f16": synth.DECODE_F16.replace(batch=8, k_len=8192, seed=23),
    "decode_unit_f16": synth.DECODE_F16.replace(batch=8, k_len=1000, seed=22),
}
KERNEL = {"chunk_split_f16": "prefill_mfma", "decode_split_f16": "decode_splitk",
          "decode_unit_f16": "decode_unit"}


def _call(case, t, **kw):
    s = case.spec
    if s.decode:
        return sdpa.decode(t["q"], t["k"], t["v"], t["lens"], layout=s.q_layout,
                           kv_layout=s.kv_layout, return_lse=True, **kw)
    return sdpa.forward(t["q"], t["k"], t["v"], layout=s.q_layout, kv_layout=s.kv_layout,
                        causal=s.causal, causal_offset=s.causal_offset, key_lens=t["lens"],
                        return_lse=True, **kw)


def _tensors(case):
    s = case.spec
    torch = pu.torch_mod()
    return dict(q=pu.to_dev(case.q, s.dtype), k=pu.to_dev(case.k, s.dtype),
                v=pu.to_dev(case.v, s.dtype), lens=torch.from_numpy(case.key_lens).cuda())


@pytest.mark.parametrize("name", sorted(CASES))
def test_caller_stream_matches_current_stream(name):
    torch = pu.torch_mod()
    case = synth.generate(CASES[name])
    t = _tensors(case)
    o_ref, l_ref = _call(case, t)
    assert sdpa.last_kernel() == KERNEL[name]
    assert sdpa.last_workspace_bytes() > 0
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse = _call(case, t, stream=side)
    # Work on the current stream that would reuse freed blocks right away.
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), name
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), name


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    torch = pu.torch_mod()
    case = synth.generate(CASES[name])
    t = _tensors(case)
    _call(case, t)                       # library loaded, first launch done
    assert sdpa.last_kernel() == KERNEL[name]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, l_g = _call(case, t)
    rng = np.random.default_rng(5)
    for rep in range(4):
        # New query values in place, then the eager result for them.
        fresh = rng.standard_normal(t["q"].shape).astype(np.float32)
        t["q"].copy_(torch.from_numpy(fresh).to(t["q"].dtype).cuda())
        o_e, l_e = _call(case, t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), (name, rep)
        assert torch.equal(l_g.view(torch.int32), l_e.view(torch.int32)), (name, rep)
        # The eager outputs agree with the oracle on these inputs too.
        if rep == 0:
            case.q[...] = synth.to_storage(fresh, case.spec.dtype).reshape(case.q.shape)
            ref_o, ref_l = pu.run_oracle(case, "nan")
            pu.compare(pu.canon(pu.to_f64(o_e), case.spec.q_layout), ref_o,
                       l_e.cpu().numpy().astype(np.float64), ref_l, case.spec.dtype, "nan",
                       what=name)
