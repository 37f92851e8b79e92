"""attn_decode_noalloc (the decode entry point that allocates nothing) against
attn_decode on the same inputs: two calls in a row on the same GPU, the second
with a smaller problem, each bit-identical to the workspace entry point."""
import numpy as np
import pytest

import scaled_dot_product_flash_amd as sdpa
from scaled_dot_product_flash_amd import synth
import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("small_mode", ["decode_splitk", "decode_unit"])
def test_noalloc_decode_matches_decode(dtype, small_mode, monkeypatch):
    """The large call runs the split mode (records in the fixed array); the
    smaller one runs the split mode too, or the unit mode, which needs no
    scratch at all."""
    torch = pu.torch_mod()
    shapes = [(64, 8192, 4, "decode_splitk"), (5, 300, 41, small_mode)]   # second call smaller
    for B, Lk, seed, mode in shapes:
        monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
        spec = synth.DECODE_F16.replace(dtype=dtype, batch=B, k_len=Lk, seed=seed)
        case = synth.generate(spec)
        q, k, v = (pu.to_dev(x, dtype) for x in (case.q, case.k, case.v))
        lens = torch.from_numpy(case.key_lens).cuda()
        want, want_lse = sdpa.decode(q, k, v, lens, kv_layout="bhsd", return_lse=True)
        assert sdpa.last_kernel() == mode
        out = torch.full_like(q, float("nan"))
        got, got_lse = sdpa.decode_noalloc(q, k, v, lens, kv_layout="bhsd", return_lse=True,
                                           out=out)
        assert sdpa.last_kernel() == mode
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (B, Lk)
        assert torch.equal(got_lse.view(torch.int32), want_lse.view(torch.int32)), (B, Lk)
        if B <= 8:   # the small call against the oracle too
            ro, rl = pu.run_oracle(case, "nan")
            pu.compare(pu.canon(pu.to_f64(got), "bshd"), ro,
                       got_lse.cpu().numpy().astype(np.float64), rl, dtype, "nan",
                       what="noalloc %s B%d" % (dtype, B))


def test_noalloc_rejects_oversized_workspace():
    """A problem whose decode workspace exceeds the fixed array is refused
    before anything runs (the ABI check needs no data)."""
    torch = pu.torch_mod()
    B, Hq, Hkv, D = 4096, 64, 4, 128       # 16-head slots: far beyond 32 MiB
    q = torch.zeros(B, 1, Hq, D, dtype=torch.float16, device="cuda")
    k = torch.zeros(B, Hkv, 64, D, dtype=torch.float16, device="cuda")
    lens = torch.full((B,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(sdpa.AttnError) as ei:
        sdpa.decode_noalloc(q, k, k, lens, kv_layout="bhsd")
    assert ei.value.status == sdpa.ERR_WORKSPACE
