"""GPU parity: the HIP path against the float64 oracle, element by element.

Reduced versions of the five workloads (several tiles and a ragged tail each)
are compared in full; the full-size workloads are compared on sampled rows
the oracle computes one by one, plus properties that hold at any size.
"""
import dataclasses

import numpy as np
import pytest

import scaled_dot_product_flash_amd as sdpa
from scaled_dot_product_flash_amd import synth
import parity_util as pu

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny_f32": synth.TINY_F32,
    "causal_gqa_f32": synth.CAUSAL_GQA_F32,
    "causal_gqa_bf16_L333": synth.CAUSAL_GQA_BF16.replace(batch=1, q_heads=8, kv_heads=2,
                                                          q_len=333, k_len=333),
    "decode_f16_cache1000": synth.DECODE_F16.replace(batch=8, k_len=1000),
    "cross_mask_f16_100x300": synth.CROSS_MASK_F16.replace(q_len=100, k_len=300),
    "causal_gqa_f16_D64_L200": synth.CAUSAL_GQA_BF16.replace(dtype="f16", batch=2, q_heads=6,
                                                             kv_heads=3, q_len=200, k_len=200,
                                                             head_dim=64, seed=11),
    "cross_bf16_D128_lens": synth.CROSS_MASK_F16.replace(dtype="bf16", head_dim=128, q_len=130,
                                                         k_len=257, seed=12),
    # End-aligned chunks: lengths include 0, the capacity, and values below
    # q_len (leading rows with no visible key).
    "chunk_f16_70x300": synth.CHUNK_F16.replace(batch=8, q_heads=8, kv_heads=2, q_len=70,
                                                k_len=300, lens="cross"),
    "chunk_bf16_D64": synth.CHUNK_F16.replace(dtype="bf16", batch=4, q_heads=6, kv_heads=3,
                                              q_len=100, k_len=257, head_dim=64, lens="cross",
                                              lens_zero_at=1, lens_full_at=2, seed=13),
    "chunk_f32": synth.CHUNK_F16.replace(dtype="f32", batch=3, q_heads=4, kv_heads=2, q_len=40,
                                         k_len=130, head_dim=64, lens="cross", lens_zero_at=0,
                                         lens_full_at=1, seed=14),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_reduced_workload_full_compare(name, policy):
    spec = REDUCED[name]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what=name)


def _full_case(name):
    spec = synth.WORKLOADS[name]
    return spec, synth.generate(spec)


@pytest.mark.parametrize("name", ["tiny_f32", "causal_gqa_f32"])
def test_small_workloads_at_full_size(name):
    spec, case = _full_case(name)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=name)


def test_causal_gqa_bf16_full_size_sampled():
    spec, case = _full_case("causal_gqa_bf16")
    o, lse, _ = pu.run_hip(case, "nan")
    assert np.isfinite(o).all() and np.isfinite(lse).all()   # every row sees key 0
    rows = pu.sample_rows(spec, 96)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what="bf16 causal GQA 4x32x4096x128")


def test_chunk_f16_full_size_sampled():
    """128 new rows per entry at the end of an 8192-key cache, lengths in
    [128, 8192]: every row sees at least one key."""
    spec = synth.EXTRA_WORKLOADS["chunk_f16"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = pu.sample_rows(spec, 96, seed=6)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what="fp16 chunk 16x32x128 cache 8192")


def test_long_chunk_bf16_full_size_sampled():
    """512 new rows at the end of a 32768-key cache, batch 1: too few query
    blocks for the GPU, so the keys are cut into ranges and merged."""
    import scaled_dot_product_flash_amd as sdpa
    spec = synth.EXTRA_WORKLOADS["long_chunk_bf16"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan")
    assert sdpa.last_workspace_bytes() > 0
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = pu.sample_rows(spec, 48, seed=14)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what="bf16 chunk 1x32x512 cache 32768")


def test_decode_f16_full_size_every_row():
    spec, case = _full_case("decode_f16")
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what="fp16 decode 64x32 cache 8192")


@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_cross_mask_f16_full_size(policy):
    spec, case = _full_case("cross_mask_f16")
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    # Batch entry 2 is fully masked and entry 5 has no keys: whole rows follow the policy.
    for b in (spec.mask_all_at, spec.lens_zero_at):
        if policy == "nan":
            assert np.isnan(o[b]).all()
        else:
            assert (o[b] == 0).all()
        assert (lse[b] == -np.inf).all()
    rows = pu.sample_rows(spec, 160)
    rows = np.concatenate([rows, [[2, 3, 7], [5, 0, 1023], [7, 15, 512]]])
    ro, rl = pu.run_oracle(case, policy, rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, policy, what="fp16 cross 8x16x1024x2048")


# ---------------------------------------------------------------------------
# Edge cases and properties.

EDGE = [
    # dtype, B, Hq, Hkv, Lq, Lk, D, causal, offset
    ("f32", 1, 1, 1, 1, 1, 1, False, None),
    ("f16", 2, 3, 1, 5, 7, 3, True, None),
    ("bf16", 1, 2, 2, 65, 129, 256, False, None),
    ("f16", 1, 4, 2, 33, 64, 128, True, 0),
    ("bf16", 2, 4, 1, 129, 65, 64, True, -5),
    ("f32", 1, 2, 1, 40, 300, 33, True, 1000),
    ("f16", 1, 1, 1, 1, 1, 128, False, None),
    ("bf16", 1, 8, 8, 256, 256, 128, True, 0),
    ("f16", 3, 2, 2, 64, 64, 64, True, None),
    ("bf16", 1, 2, 1, 17, 1, 32, False, None),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes(cfg):
    dtype, B, Hq, Hkv, Lq, Lk, D, causal, offset = cfg
    spec = synth.Spec("edge", B, Hq, Hkv, Lq, Lk, D, dtype, seed=Lq * 7 + Lk, causal=causal,
                      causal_offset=offset, lse=True)
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "zero")
    ro, rl = pu.run_oracle(case, "zero")
    pu.compare(o, ro, lse, rl, dtype, "zero", what=str(cfg))


@pytest.mark.parametrize("policy", ["nan", "zero"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_zero_key_length_problem(policy, dtype):
    spec = synth.Spec("klen0", 2, 4, 2, 9, 0, 64, dtype, seed=3, lse=True)
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, policy)
    assert (np.isnan(o) if policy == "nan" else (o == 0)).all()
    assert (lse == -np.inf).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_special_values(dtype):
    """NaN in one visible K element -> NaN row; +inf mask entry -> NaN row; NaN in
    K beyond the key length, and garbage V rows beyond it, never leak."""
    torch = pu.torch_mod()
    spec = synth.Spec("special", 2, 2, 1, 70, 150, 64, dtype, seed=9, causal=True, lse=True,
                      lens="uniform")
    case = synth.generate(spec)
    case.key_lens[:] = [120, 150]
    k = case.k.copy()
    v = case.v.copy()
    nanbits = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}
    k[0, 120:, :, :] = nanbits[dtype]        # beyond batch 0's length: never read
    v[0, 120:, :, :] = nanbits[dtype]
    k[1, 30, 0, 5] = nanbits[dtype]          # visible to batch 1 rows i >= 30 (offset 80)
    mask = np.zeros((2, 1, 70, 150), np.float32)
    mask[0, :, 10, 3] = np.inf               # batch 0, row 10 -> NaN row
    case = synth.Case(spec, case.q, k, v, case.key_lens, mask)
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        ro, rl = pu.run_oracle(case, policy)
        assert np.isnan(ro[0, :, 10]).all() and np.isnan(ro[1, :, 0]).all()
        pu.compare(o, ro, lse, rl, dtype, policy, what="special %s" % policy)
    del torch


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_one_hot_is_bit_exact(dtype):
    """All keys but j0 hidden by -inf: O equals V[j0] bit for bit."""
    torch = pu.torch_mod()
    spec = synth.Spec("onehot", 1, 4, 2, 80, 200, 128 if dtype != "f32" else 64, dtype, seed=4)
    case = synth.generate(spec)
    mask = np.full((1, 1, 1, 200), -np.inf, np.float32)
    mask[..., 137] = 0.5
    case = synth.Case(spec, case.q, case.k, case.v, None, mask)
    o, _, (ot, _, tens) = pu.run_hip(case, "nan", return_lse=False)
    vt = tens["v"]
    for h in range(4):
        assert torch.equal(ot[0, :, h, :], vt[0, 137, h // 2, :].expand(80, -1))


def test_gqa_map_exact():
    """V of kv head g is g+1 everywhere -> O of query head h is exactly h//(Hq/Hkv)+1."""
    spec = synth.Spec("gqa", 2, 12, 4, 96, 96, 64, "bf16", seed=5, causal=True)
    case = synth.generate(spec)
    v = np.empty_like(case.v)
    for g in range(4):
        v[:, :, g, :] = synth.to_storage(np.full(1, g + 1, np.float32), "bf16")[0]
    case = synth.Case(spec, case.q, case.k, v, None, None)
    o, _, _ = pu.run_hip(case, "nan", return_lse=False)
    for h in range(12):
        assert (o[:, h] == h // 3 + 1).all()


def test_strided_packed_qkv_and_broadcast_mask():
    """Q/K/V as slices of one packed projection [B, L, Hq+2*Hkv, D]; mask [B,1,Lq,Lk]."""
    torch = pu.torch_mod()
    B, L, Hq, Hkv, D = 2, 150, 8, 2, 128
    rng = np.random.default_rng(21)
    packed = synth.to_storage(rng.standard_normal((B, L, Hq + 2 * Hkv, D)).astype(np.float32), "f16")
    mask = rng.standard_normal((B, 1, L, L)).astype(np.float32)
    pt = pu.to_dev(packed, "f16")
    q, k, v = pt[:, :, :Hq], pt[:, :, Hq:Hq + Hkv], pt[:, :, Hq + Hkv:]
    mt = torch.from_numpy(mask).cuda()
    o, lse = __import__("scaled_dot_product_flash_amd").forward(q, k, v, causal=True, mask=mt,
                                                                return_lse=True)
    torch.cuda.synchronize()
    import oracle
    ro, rl = oracle.attention(packed[:, :, :Hq], packed[:, :, Hq:Hq + Hkv],
                              packed[:, :, Hq + Hkv:], dtype="f16", causal=True, mask=mask)
    pu.compare(pu.canon(pu.to_f64(o), "bshd"), ro, lse.cpu().numpy().astype(np.float64), rl,
               "f16", "nan", what="packed qkv")


@pytest.mark.parametrize("name", ["causal_gqa_bf16_L333", "decode_f16_cache1000",
                                  "cross_mask_f16_100x300", "causal_gqa_f32"])
def test_two_runs_bit_identical(name):
    torch = pu.torch_mod()
    case = synth.generate(REDUCED[name])
    _, _, (o1, l1, tens) = pu.run_hip(case, "nan", return_lse=True)
    _, _, (o2, l2, _) = pu.run_hip(case, "nan", return_lse=True, tensors=tens)
    assert torch.equal(o1.view(torch.int16) if o1.dtype != torch.float32 else o1.view(torch.int32),
                       o2.view(torch.int16) if o2.dtype != torch.float32 else o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_empty_batch_is_a_no_op():
    torch = pu.torch_mod()
    import scaled_dot_product_flash_amd as sdpa
    q = torch.zeros(0, 4, 2, 64, dtype=torch.float16, device="cuda")
    o = sdpa.forward(q, q, q)
    assert o.shape == q.shape


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f16", 128), ("bf16", 64)])
def test_matrix_core_path_is_used_and_matches_generic(dtype, D, monkeypatch):
    """The MFMA kernel serves bf16/fp16 at D = 64/128; it agrees with the
    any-shape kernel (forced through SDPA_FLASH_KERNEL=generic) within tolerance."""
    import scaled_dot_product_flash_amd as sdpa
    spec = synth.Spec("mfma", 2, 8, 2, 300, 300, D, dtype, seed=31, causal=True, lse=True,
                      lens="uniform")
    case = synth.generate(spec)
    o1, l1, (_, _, tens) = pu.run_hip(case, "zero")
    assert sdpa.last_kernel() == "prefill_mfma"
    monkeypatch.setenv("SDPA_FLASH_KERNEL", "generic")
    o2, l2, _ = pu.run_hip(case, "zero", tensors=tens)
    assert sdpa.last_kernel() == "generic"
    pu.compare(o1, o2, l1, l2, dtype, "zero", what="mfma vs generic")
    ro, rl = pu.run_oracle(case, "zero")
    pu.compare(o1, ro, l1, rl, dtype, "zero", what="mfma vs oracle")


# Key ranges of 1 to 5 tiles of 64 around each head dim's staging plan (how
# many K / V tiles are loaded ahead and into how many buffers), with ragged
# per-entry lengths ("cross": one entry empty, one full), so that prologues
# shorter than the prefetch distance, the last tiles' waits and the buffer
# rotation all run; the windowed cases start the key loop past tile 0.
STAGING = [(dt, D, Lk, win) for (dt, D) in (("f16", 64), ("bf16", 128), ("f16", 128), ("bf16", 256))
           for Lk in (1, 64, 65, 128, 129, 192, 193, 256, 320) for win in (-1,)]
STAGING += [("bf16", 128, 320, 70), ("f16", 64, 320, 70), ("bf16", 256, 257, 100)]


@pytest.mark.parametrize("cfg", STAGING, ids=lambda c: "x".join(map(str, c)))
def test_staging_tile_counts(cfg):
    import scaled_dot_product_flash_amd as sdpa
    dtype, D, Lk, win = cfg
    spec = synth.Spec("staging", 4, 8, 2, 70 if win < 0 else Lk, Lk, D, dtype, seed=Lk + D,
                      causal=win >= 0, lens="cross", lens_zero_at=1, lens_full_at=2,
                      local_window=win, lse=True)
    case = synth.generate(spec)
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        assert sdpa.last_kernel() == "prefill_mfma"
        ro, rl = pu.run_oracle(case, policy)
        pu.compare(o, ro, lse, rl, dtype, policy, what=str(cfg))


# Prefill grids too small for the GPU: each row block's keys are cut into
# ranges whose partial records a second kernel merges in order (checked to be
# the path taken through the workspace the call asked for).  Long caches,
# ragged and zero lengths, both policies, mask, window, sink and documents.
SPLIT = {
    "bf16_D128_chunk_end": synth.CHUNK_F16.replace(dtype="bf16", batch=2, q_heads=8, kv_heads=2,
                                                   q_len=100, k_len=8192, lens="cross",
                                                   lens_zero_at=1, seed=41),
    "f16_D64_mask_lens": synth.CROSS_MASK_F16.replace(batch=2, q_heads=4, kv_heads=4, q_len=300,
                                                      k_len=3000, seed=42),
    "bf16_D256_window_sink": synth.CHUNK_F16.replace(dtype="bf16", batch=1, q_heads=2,
                                                     kv_heads=1, q_len=64, k_len=2048,
                                                     head_dim=256, lens=None, local_window=700,
                                                     sink="heads", seed=43),
    "bf16_D96_docs": synth.CAUSAL_GQA_BF16.replace(batch=1, q_heads=4, kv_heads=1, q_len=2100,
                                                   k_len=2100, head_dim=96, docs="packed",
                                                   doc_mean=300, seed=44),
    "f16_D128_softcap_sink_zero": synth.CHUNK_F16.replace(batch=3, q_heads=4, kv_heads=1,
                                                          q_len=2, k_len=5000, softcap=10.0,
                                                          sink="zero", lens="cross",
                                                          lens_zero_at=0, seed=45),
}


@pytest.mark.parametrize("policy", ["nan", "zero"])
@pytest.mark.parametrize("name", sorted(SPLIT))
def test_prefill_key_range_split(name, policy):
    import scaled_dot_product_flash_amd as sdpa
    spec = SPLIT[name]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, policy)
    assert sdpa.last_kernel() == "prefill_mfma"
    assert sdpa.last_workspace_bytes() > 0
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what=name)


# Without causality, workgroups with per-entry key lengths are ordered
# longest entry first (ranks computed on the device; ties by index): tied and
# zero lengths, unit counts that do and do not split over the 8 XCDs, and
# more than 64 entries (the plain order).
LEN_ORDER = [
    ("f16", 64, [300, 300, 0]),
    ("bf16", 128, [5, 300, 300, 1, 0, 299, 64, 65]),
    ("f16", 128, [17, 300, 0, 0, 250, 300, 1, 128, 129]),
    ("bf16", 64, list(np.random.default_rng(3).integers(0, 301, size=65))),
]


@pytest.mark.parametrize("cfg", LEN_ORDER, ids=lambda c: "%s_D%d_B%d" % (c[0], c[1], len(c[2])))
def test_length_ordered_workgroups(cfg):
    import scaled_dot_product_flash_amd as sdpa
    dtype, D, lens = cfg
    spec = synth.Spec("lenorder", len(lens), 4, 2, 200, 300, D, dtype, seed=len(lens) + D,
                      lens="uniform", lse=True)
    case = synth.generate(spec)
    case = dataclasses.replace(case, key_lens=np.asarray(lens, dtype=np.int32))
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        assert sdpa.last_kernel() == "prefill_mfma"
        ro, rl = pu.run_oracle(case, policy)
        pu.compare(o, ro, lse, rl, dtype, policy, what=str(lens))


DECODE = [
    # dtype, B, Hq, Hkv, cap, D, lens
    ("f16", 6, 32, 8, 3000, 128, [1, 3000, 0, 257, 1024, 2999]),
    ("bf16", 5, 8, 8, 700, 64, [700, 1, 128, 129, 0]),
    ("f16", 3, 32, 1, 513, 128, [513, 256, 255]),
    ("bf16", 2, 6, 2, 9000, 128, [9000, 4097]),
    # head dims below 128 that are whole 16-byte chunks run padded to 64/128
    ("f16", 4, 16, 4, 600, 96, [600, 1, 300, 0]),
    ("bf16", 3, 8, 2, 500, 40, [500, 17, 250]),
    ("f16", 2, 4, 4, 300, 8, [300, 33]),
    ("bf16", 2, 32, 8, 1000, 112, [1000, 999]),
    ("f16", 3, 8, 4, 700, 256, [700, 64, 333]),
    ("bf16", 2, 16, 2, 400, 200, [400, 1]),
    # fp32 Q/K/V: head dims that are whole 16-byte chunks up to 128 (padded to 64/128)
    ("f32", 4, 16, 4, 900, 128, [900, 1, 450, 0]),
    ("f32", 3, 8, 8, 700, 64, [700, 65, 0]),
    ("f32", 2, 32, 1, 513, 100, [513, 300]),
    ("f32", 2, 4, 2, 300, 4, [300, 33]),
    ("f32", 2, 48, 2, 2100, 96, [2100, 1000]),
]


# The two decode modes: the split over equal shares of all steps with its
# ordered merge, and one workgroup per unit folding in LDS.
DECODE_MODES = ["decode_splitk", "decode_unit"]


@pytest.mark.parametrize("cfg", DECODE, ids=lambda c: "x".join(map(str, c[:6])))
@pytest.mark.parametrize("policy", ["nan", "zero"])
@pytest.mark.parametrize("mode", DECODE_MODES)
def test_decode_split_path(cfg, policy, mode, monkeypatch):
    """Decode in each mode against the oracle and the any-shape kernel."""
    import scaled_dot_product_flash_amd as sdpa
    dtype, B, Hq, Hkv, cap, D, lens = cfg
    spec = synth.Spec("decode", B, Hq, Hkv, 1, cap, D, dtype, seed=cap + B, kv_layout="bhsd",
                      causal=True, decode=True, lens="uniform", lse=True)
    case = synth.generate(spec)
    case.key_lens[:] = lens
    monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
    o1, l1, (_, _, tens) = pu.run_hip(case, policy)
    assert sdpa.last_kernel() == mode
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o1, ro, l1, rl, dtype, policy, what="decode %s" % (cfg,))
    monkeypatch.setenv("SDPA_FLASH_KERNEL", "generic")
    o2, l2, _ = pu.run_hip(case, policy, tensors=tens)
    assert sdpa.last_kernel() == "generic"
    pu.compare(o1, o2, l1, l2, dtype, policy, what="decode vs generic")


def test_decode_with_mask_and_garbage_beyond_length():
    """Per-head mask rows; NaN cache rows past each length are never read."""
    torch = pu.torch_mod()
    spec = synth.Spec("decode-mask", 4, 8, 2, 1, 1500, 128, "f16", seed=77, kv_layout="bhsd",
                      causal=True, decode=True, lens="uniform", lse=True)
    case = synth.generate(spec)
    case.key_lens[:] = [1500, 700, 3, 1]
    k, v = case.k.copy(), case.v.copy()
    for b, L in enumerate(case.key_lens):
        k[b, :, L:] = np.float16(np.nan)
        v[b, :, L:] = np.float16(np.nan)
    rng = np.random.default_rng(5)
    mask = rng.standard_normal((4, 8, 1, 1500)).astype(np.float32)
    mask[rng.random(mask.shape) < 0.2] = -np.inf
    mask[3, :, :, 0] = -np.inf                  # batch 3: its only key hidden -> empty rows
    case = synth.Case(spec, case.q, k, v, case.key_lens, mask)
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        ro, rl = pu.run_oracle(case, policy)
        assert (rl[3] == -np.inf).all()
        pu.compare(o, ro, lse, rl, "f16", policy, what="decode mask %s" % policy)
    del torch


F32 = [
    # B, Hq, Hkv, Lq, Lk, D, causal, offset, lens, mask
    (1, 2, 2, 64, 64, 32, False, None, False, False),
    (2, 12, 4, 512, 512, 64, True, 0, False, False),
    (1, 4, 1, 100, 700, 128, True, None, True, True),
    (3, 2, 2, 17, 1000, 64, False, None, True, True),
    (1, 1, 1, 1, 1, 32, True, None, False, False),
    # head dims padded to 32 / 64 / 96 / 128 / 256, odd ones (per-element
    # loads), and the key-range split at several paddings
    (2, 4, 2, 70, 70, 1, True, None, False, False),
    (2, 4, 2, 90, 130, 17, False, None, True, True),
    (2, 6, 3, 100, 100, 33, True, 0, True, False),
    (2, 12, 4, 512, 512, 80, True, 0, False, False),
    (2, 12, 4, 512, 512, 96, True, 0, False, False),
    (1, 4, 2, 60, 900, 100, True, None, True, True),
    (2, 4, 2, 130, 130, 160, True, None, False, False),
    (1, 4, 4, 50, 700, 256, False, None, True, True),
    (2, 4, 2, 100, 100, 256, True, 0, False, False),
]


@pytest.mark.parametrize("cfg", F32, ids=lambda c: "x".join(map(str, c[:6])))
def test_fp32_vector_path(cfg, monkeypatch):
    """fp32 runs on the vector-FMA kernel (with the key-range split when the row
    blocks are few) and matches the oracle and the any-shape kernel."""
    import scaled_dot_product_flash_amd as sdpa
    B, Hq, Hkv, Lq, Lk, D, causal, offset, lens, mask = cfg
    spec = synth.Spec("f32", B, Hq, Hkv, Lq, Lk, D, "f32", seed=Lq + Lk + D, causal=causal,
                      causal_offset=offset, lse=True, lens="uniform" if lens else None)
    case = synth.generate(spec)
    if mask:
        rng = np.random.default_rng(3)
        m = rng.standard_normal((B, 1, Lq, Lk)).astype(np.float32)
        m[rng.random(m.shape) < 0.2] = -np.inf
        case = synth.Case(spec, case.q, case.k, case.v, case.key_lens, m)
    for policy in ("nan", "zero"):
        o1, l1, (_, _, tens) = pu.run_hip(case, policy)
        # (The one-row case is a small problem without head groups, which
        # stays on this kernel rather than the decode kernels.)
        assert sdpa.last_kernel() == "prefill_f32"
        ro, rl = pu.run_oracle(case, policy)
        pu.compare(o1, ro, l1, rl, "f32", policy, what="f32 %s" % (cfg,))
    monkeypatch.setenv("SDPA_FLASH_KERNEL", "generic")
    o2, l2, _ = pu.run_hip(case, "zero", tensors=tens)
    pu.compare(o1, o2, l1, l2, "f32", "zero", what="f32 vs generic")


@pytest.mark.parametrize("lens", [[1, 0, 3, 2], [0, 0, 0, 0], [33, 0, 0, 64]])
def test_decode_tiny_totals(lens):
    """Fewer live steps than decode waves: most waves own nothing, and entries
    with no live key are skipped by the cut."""
    spec = synth.Spec("decode-tiny", 4, 8, 2, 1, 64, 64, "bf16", seed=8, kv_layout="bhsd",
                      causal=True, decode=True, lens="uniform", lse=True)
    case = synth.generate(spec)
    case.key_lens[:] = lens
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        ro, rl = pu.run_oracle(case, policy)
        pu.compare(o, ro, lse, rl, "bf16", policy, what="decode tiny %s" % lens)


@pytest.mark.parametrize("B,cap", [(150, 300), (300, 2000)])
def test_decode_many_entries_trailing_empty(B, cap):
    """More entries than one wave's lanes (the per-entry step sums run in
    chunks of 64), about a third of them empty, the last ones included, with
    fewer (150 x 300) and more (300 x 2000) live steps than decode waves."""
    spec = synth.Spec("decode-many", B, 4, 2, 1, cap, 64, "f16", seed=B, kv_layout="bhsd",
                      causal=True, decode=True, lens="uniform", lse=True)
    case = synth.generate(spec)
    rng = np.random.default_rng(B)
    lens = rng.integers(1, cap + 1, size=B).astype(np.int32)
    lens[rng.random(B) < 0.3] = 0
    lens[-5:] = 0
    lens[0] = cap
    case.key_lens[:] = lens
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy)
        ro, rl = pu.run_oracle(case, policy)
        pu.compare(o, ro, lse, rl, "f16", policy, what="decode many %d" % B)


@pytest.mark.parametrize("which", ["decode_f16", "prefill_bf16", "prefill_f32"])
def test_largest_batch(which):
    """The largest batch the library accepts (65535 entries; the fp32 kernel's
    grid depth is exactly its limit), short rows, a third of the key lengths
    zero."""
    B = 65535
    if which == "decode_f16":
        spec = synth.Spec("max-batch", B, 2, 1, 1, 40, 64, "f16", seed=91, kv_layout="bhsd",
                          causal=True, decode=True, lens="uniform", lse=True)
    else:
        spec = synth.Spec("max-batch", B, 2, 1, 5, 7, 64, which[-4:].lstrip("_"), seed=92,
                          causal=True, causal_offset="end", lens="uniform", lse=True)
    case = synth.generate(spec)
    rng = np.random.default_rng(93)
    case.key_lens[rng.random(B) < 0.33] = 0
    o, lse, _ = pu.run_hip(case, "nan")
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what="largest batch %s" % which)


# --------------------------------------------------------------------------
# Score-rule variants: local window, softcap, sink (GroupQueryAttention
# README attributes), on every kernel that runs them.

VARIANTS = {
    "window50_bf16_L333": (synth.CAUSAL_GQA_BF16.replace(
        batch=1, q_heads=8, kv_heads=2, q_len=333, k_len=333, local_window=50, seed=21),
        "prefill_mfma"),
    "window0_f16_D64": (synth.CAUSAL_GQA_BF16.replace(
        dtype="f16", batch=2, q_heads=6, kv_heads=3, q_len=200, k_len=260, head_dim=64,
        local_window=0, seed=22), "prefill_mfma"),
    "softcap5_bf16_mask_lens": (synth.CROSS_MASK_F16.replace(
        dtype="bf16", head_dim=128, q_len=130, k_len=257, softcap=5.0, seed=23), "prefill_mfma"),
    "sink_heads_f16_chunk": (synth.CHUNK_F16.replace(
        batch=8, q_heads=8, kv_heads=2, q_len=70, k_len=300, lens="cross", sink="heads",
        seed=24), "prefill_mfma"),
    "window_cap_smooth_bf16": (synth.CAUSAL_GQA_BF16.replace(
        batch=2, q_heads=8, kv_heads=4, q_len=300, k_len=300, local_window=77, softcap=20.0,
        sink="zero", seed=25), "prefill_mfma"),
    "window_cap_sink_f32": (synth.CAUSAL_GQA_F32.replace(
        batch=1, q_heads=4, kv_heads=2, q_len=100, k_len=100, local_window=10, softcap=3.0,
        sink="heads", seed=26), "prefill_f32"),
    "window_docs_f32_D96_split": (synth.CAUSAL_GQA_F32.replace(
        batch=1, q_heads=4, kv_heads=2, q_len=60, k_len=900, head_dim=96, local_window=300,
        causal_offset=None, docs="random", sink="zero", seed=30), "prefill_f32"),
    "softcap_f32_D256_mask_lens": (synth.CROSS_MASK_F16.replace(
        dtype="f32", batch=3, q_heads=4, kv_heads=4, q_len=70, k_len=200, head_dim=256,
        softcap=4.0, lens_zero_at=1, lens_full_at=0, mask_all_at=2, seed=31), "prefill_f32"),
    "decode_window_cap_sink": (synth.DECODE_F16.replace(
        batch=8, k_len=1000, local_window=100, softcap=30.0, sink="heads", seed=27),
        "decode"),
    "decode_window0_bf16": (synth.DECODE_F16.replace(
        dtype="bf16", batch=8, k_len=700, head_dim=64, local_window=0, seed=28), "decode"),
    "decode_f32_window_cap_sink": (synth.DECODE_F16.replace(
        dtype="f32", batch=4, k_len=900, local_window=100, softcap=30.0, sink="heads", seed=39),
        "decode"),
    "decode_sink_zero_lens0": (synth.DECODE_F16.replace(
        batch=8, k_len=500, lens="cross", lens_zero_at=3, lens_full_at=4, sink="zero",
        local_window=3000, seed=29), "decode"),
}


def _run_and_compare(spec, kernel, policy, name, monkeypatch):
    """Runs a case on its expected kernel ("decode": in both decode modes)
    and compares it with the oracle."""
    case = synth.generate(spec)
    ro, rl = pu.run_oracle(case, policy)
    for want in (DECODE_MODES if kernel == "decode" else [kernel]):
        if kernel == "decode":
            monkeypatch.setenv("SDPA_FLASH_KERNEL", want)
        o, lse, _ = pu.run_hip(case, policy, return_lse=True)
        assert sdpa.last_kernel() == want
        pu.compare(o, ro, lse, rl, spec.dtype, policy, what="%s %s" % (name, want))


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_score_variants_full_compare(name, policy, monkeypatch):
    spec, kernel = VARIANTS[name]
    _run_and_compare(spec, kernel, policy, name, monkeypatch)


def test_sink_rows_without_keys_are_zero():
    """Rows that see no key put all weight on the sink: O = 0, LSE = sink."""
    spec = synth.CHUNK_F16.replace(batch=4, q_heads=8, kv_heads=2, q_len=64, k_len=128,
                                   lens="cross", lens_zero_at=0, lens_full_at=1, sink="heads",
                                   seed=30)
    case = synth.generate(spec)
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy, return_lse=True)
        assert (o[0] == 0).all()
        # LSE = sink, up to the fp32 round trip through base 2.
        want = np.broadcast_to(case.head_sink.astype(np.float64)[:, None], lse[0].shape)
        assert np.abs(lse[0] - want).max() < 1e-6


@pytest.mark.parametrize("name", ["window_bf16", "softcap_sink_bf16"])
def test_variant_prefill_full_size_sampled(name):
    spec = synth.EXTRA_WORKLOADS[name]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = pu.sample_rows(spec, 96, seed=7)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what=spec.name)


@pytest.mark.parametrize("mode", [None] + DECODE_MODES)
def test_variant_decode_full_size_every_row(mode, monkeypatch):
    """The window + sink decode workload at full size, in the mode its shape
    picks (the window bounds every unit to 64 steps: one workgroup per unit)
    and in each mode forced."""
    spec = synth.EXTRA_WORKLOADS["decode_window_f16"]
    case = synth.generate(spec)
    if mode:
        monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() == (mode or "decode_unit")
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=spec.name)


# --------------------------------------------------------------------------
# int8 key/value cache with float32 scales (decode).

INT8 = {
    "i8_tensor_f16": synth.DECODE_F16.replace(batch=8, k_len=1000, kv_quant="tensor", seed=31),
    "i8_channel_bf16_D64": synth.DECODE_F16.replace(dtype="bf16", batch=8, k_len=777,
                                                    head_dim=64, kv_quant="channel", seed=32),
    "i8_mixed_window_cap_sink": synth.DECODE_F16.replace(
        batch=8, k_len=900, kv_quant="mixed", local_window=300, softcap=20.0, sink="heads",
        seed=33),
    "i8_channel_lens0_mask": synth.DECODE_F16.replace(
        batch=8, k_len=600, kv_quant="channel", lens="cross", lens_zero_at=2, lens_full_at=3,
        mask="keys", mask_all_at=5, seed=34),
    # padded head dims (multiples of 16 below 128): per-channel scales indexed by the true dim
    "i8_channel_D96": synth.DECODE_F16.replace(batch=6, k_len=800, head_dim=96,
                                               kv_quant="channel", seed=35),
    "i8_tensor_bf16_D48": synth.DECODE_F16.replace(dtype="bf16", batch=5, k_len=500, head_dim=48,
                                                   kv_quant="mixed", lens="cross", lens_zero_at=1,
                                                   lens_full_at=0, seed=36),
    "i8_channel_D256_window": synth.DECODE_F16.replace(batch=4, k_len=900, head_dim=256,
                                                       kv_quant="channel", local_window=500,
                                                       seed=37),
}


@pytest.mark.parametrize("name", sorted(INT8))
@pytest.mark.parametrize("policy", ["nan", "zero"])
@pytest.mark.parametrize("mode", DECODE_MODES)
def test_int8_cache_decode(name, policy, mode, monkeypatch):
    spec = INT8[name]
    case = synth.generate(spec)
    monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    assert sdpa.last_kernel() == mode + "_int8"
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what=name)


def test_decode_d96_full_size_every_row():
    """Decode at head dim 96 (padded to 128 on the split path) at full size."""
    spec = synth.EXTRA_WORKLOADS["decode_d96_f16"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() == "decode_splitk"
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=spec.name)


def test_decode_f32_full_size_every_row():
    """fp32 decode at the decode workload's shape (split mode) on every row."""
    spec = synth.EXTRA_WORKLOADS["decode_f32"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() == "decode_splitk"
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=spec.name)


def test_int8_cache_decode_full_size_every_row():
    spec = synth.EXTRA_WORKLOADS["decode_int8_f16"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=spec.name)


# --------------------------------------------------------------------------
# Document masks (packed documents; arbitrary per-row starts too).

DOCS = {
    "docs_bf16_L333": (synth.CAUSAL_GQA_BF16.replace(
        batch=2, q_heads=8, kv_heads=2, q_len=333, k_len=333, docs="packed", doc_mean=40,
        seed=41), "prefill_mfma"),
    "docs_random_f16_D64_lens": (synth.CAUSAL_GQA_BF16.replace(
        dtype="f16", batch=3, q_heads=6, kv_heads=3, q_len=200, k_len=260, head_dim=64,
        docs="random", lens="cross", lens_zero_at=1, lens_full_at=2, seed=42), "prefill_mfma"),
    "docs_window_sink_bf16": (synth.CAUSAL_GQA_BF16.replace(
        batch=1, q_heads=8, kv_heads=4, q_len=300, k_len=300, docs="packed", doc_mean=70,
        local_window=50, sink="heads", seed=43), "prefill_mfma"),
    "docs_noncausal_f16_mask": (synth.CROSS_MASK_F16.replace(
        q_len=100, k_len=300, docs="random", seed=44), "prefill_mfma"),
    "docs_f32": (synth.CAUSAL_GQA_F32.replace(
        batch=2, q_heads=4, kv_heads=2, q_len=90, k_len=90, docs="packed", doc_mean=12,
        seed=45), "prefill_f32"),
    "docs_f32_D33_sink_split": (synth.CAUSAL_GQA_F32.replace(
        batch=1, q_heads=2, kv_heads=1, q_len=40, k_len=800, head_dim=33, docs="random",
        causal_offset=None, sink="heads", seed=47), "prefill_f32"),
    "docs_decode": (synth.DECODE_F16.replace(
        batch=8, k_len=700, docs="random", seed=46), "decode"),
}


@pytest.mark.parametrize("name", sorted(DOCS))
@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_doc_masks_full_compare(name, policy, monkeypatch):
    spec, kernel = DOCS[name]
    _run_and_compare(spec, kernel, policy, name, monkeypatch)


def test_docs_bf16_full_size_sampled():
    spec = synth.EXTRA_WORKLOADS["docs_bf16"]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = pu.sample_rows(spec, 96, seed=11)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what=spec.name)


# --------------------------------------------------------------------------
# Head dims beyond 64 / 128 on the matrix cores (multiples of 8 run padded
# to 64, 128 or 256; odd dims stay on the any-shape kernel).

HEAD_DIMS = [
    # D, dtype, q_len, k_len, extra
    (8, "bf16", 130, 130, {}),
    (32, "f16", 200, 200, {}),
    (40, "bf16", 97, 150, dict(lens="cross", lens_zero_at=1, lens_full_at=0)),
    (80, "f16", 150, 150, {}),
    (96, "bf16", 150, 200, dict(local_window=40, sink="heads")),
    (160, "f16", 100, 100, dict(softcap=10.0)),
    (256, "bf16", 200, 200, {}),
    (256, "f16", 70, 300, dict(causal=False, mask="keys", lens="cross", lens_zero_at=1,
                               lens_full_at=0, mask_all_at=2)),
    (256, "bf16", 120, 120, dict(docs="packed", doc_mean=30)),
]


@pytest.mark.parametrize("cfg", HEAD_DIMS, ids=lambda c: "D%d-%s-%dx%d" % c[:4])
@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_head_dims_on_matrix_cores(cfg, policy):
    D, dtype, lq, lk, extra = cfg
    spec = synth.CAUSAL_GQA_BF16.replace(dtype=dtype, batch=3, q_heads=8, kv_heads=2, q_len=lq,
                                         k_len=lk, head_dim=D, seed=50 + D, **extra)
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    assert sdpa.last_kernel() == "prefill_mfma"
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what="D=%d %s" % (D, dtype))


# Head dims that are not a multiple of 8: K/V staged into the workspace
# padded to one, Q read and O written per element (through LDS, one row at
# a time, at the padded dims 128 and 256), then the matrix-core
# kernel at the padded dim (OneGPU "Attention", "What it covers").
ODD_DIMS = [
    # D, dtype, B, Hq, Hkv, Lq, Lk, extra
    (1, "bf16", 2, 4, 2, 70, 70, {}),
    (17, "bf16", 3, 8, 2, 150, 150, dict(lens="cross", lens_zero_at=1, lens_full_at=0)),
    (33, "f16", 2, 4, 2, 40, 40, {}),
    (100, "bf16", 2, 8, 2, 200, 260, dict(local_window=60, sink="heads")),
    (100, "f16", 2, 4, 4, 90, 300, dict(causal=False, mask="keys", lens="cross",
                                        lens_zero_at=1, lens_full_at=0, mask_all_at=5)),
    (255, "bf16", 2, 4, 2, 100, 100, dict(docs="packed", doc_mean=20, softcap=8.0)),
    (130, "f16", 1, 8, 2, 64, 2000, dict(causal_offset=None)),   # key-range split
]


@pytest.mark.parametrize("cfg", ODD_DIMS, ids=lambda c: "D%d-%s-%dx%d" % (c[0], c[1], c[5], c[6]))
@pytest.mark.parametrize("policy", ["nan", "zero"])
def test_odd_head_dims_on_matrix_cores(cfg, policy):
    D, dtype, B, Hq, Hkv, lq, lk, extra = cfg
    spec = synth.CAUSAL_GQA_BF16.replace(dtype=dtype, batch=B, q_heads=Hq, kv_heads=Hkv,
                                         q_len=lq, k_len=lk, head_dim=D, seed=60 + D, **extra)
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    assert sdpa.last_kernel() == "prefill_mfma"
    assert sdpa.last_workspace_bytes() > 0      # the staged K/V copies
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what="D=%d %s" % (D, dtype))


def test_odd_head_dim_decode_runs_staged():
    """Decode at a head dim the split decode path does not take runs as the
    forward path does, staged K/V included."""
    spec = synth.DECODE_F16.replace(batch=8, k_len=700, head_dim=100, seed=67)
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() == "prefill_mfma"
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what="decode D=100")


@pytest.mark.parametrize("name,kernel", [("d256_bf16", "prefill_mfma"),
                                         ("d96_bf16", "prefill_mfma"),
                                         ("d100_bf16", "prefill_mfma"),
                                         ("d96_f32", "prefill_f32")])
def test_head_dim_workloads_full_size_sampled(name, kernel):
    spec = synth.EXTRA_WORKLOADS[name]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan")
    assert sdpa.last_kernel() == kernel
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = pu.sample_rows(spec, 64, seed=12)
    ro, rl = pu.run_oracle(case, "nan", rows=rows)
    go = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    pu.compare(go, ro, gl, rl, spec.dtype, "nan", what=spec.name)


# Causal offsets that put each row's key bounds far outside the tile or on
# either side of a 64-key tile edge, with ragged lengths and tails, with and
# without a local window: the per-score visibility test compares each score's
# offset inside its tile with the lane's bounds clamped to [0, 64].
@pytest.mark.parametrize("window", [-1, 37])
@pytest.mark.parametrize("off", [-(1 << 40), -151, -150, -149, -65, -64, -63, -1, 0, 1, 63, 64,
                                 65, 127, 1 << 40])
def test_causal_offsets_at_tile_edges(off, window):
    spec = synth.Spec("offset %d window %d" % (off, window), 2, 8, 2, 150, 203, 128, "bf16",
                      seed=31, causal=True, causal_offset=off, lens="uniform", lse=True,
                      local_window=window, masked_rows="zero")
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "zero")
    ro, rl = pu.run_oracle(case, "zero")
    pu.compare(o, ro, lse, rl, "bf16", "zero", what=str(spec))


# Large finite mask values (the float32-minimum "masked" convention, -1e30,
# a huge positive entry): they are values, not -inf, so a row whose visible
# keys all carry the same such value is the plain mean of those V rows
# (OneGPU "Attention", "Special values": only -inf keys weigh nothing), and a
# row mixing them with ordinary keys gives them weight 0.  Every kernel:
# matrix-core prefill (one pass and key-range split), fp32, decode and the
# any-shape kernel.
FMIN = np.finfo(np.float32).min


def _large_mask_rows(rng, n_rows, Lk):
    m = (rng.standard_normal((n_rows, Lk)) * 2).astype(np.float32)
    pats = [np.full(Lk, FMIN, np.float32),                                  # all finfo.min
            np.where(np.arange(Lk) % 2 == 0, 0.0, FMIN).astype(np.float32), # half of them
            np.full(Lk, -1e30, np.float32),                                 # all -1e30
            np.where(np.arange(Lk) % 3 == 0, -np.inf, FMIN).astype(np.float32),
            np.full(Lk, -np.inf, np.float32),                               # empty row
            np.where(np.arange(Lk) == Lk // 3, 3e38, 0.0).astype(np.float32)]
    for r, pat in enumerate(pats):
        if r < n_rows:
            m[r] = pat
    return m


def _compare_large(o, lse, ro, rl, dtype, policy, what):
    pu.compare(o, ro, None, None, dtype, policy, what=what)
    # LSE of rows near the float range: fp32 cannot hold ln(count) beside
    # 3.4e38, so those compare relatively.
    fin = np.isfinite(rl)
    assert (np.isnan(lse) == np.isnan(rl)).all() and (lse[rl == -np.inf] == -np.inf).all()
    err = np.abs(lse[fin] - rl[fin])
    assert (err <= pu.LSE_TOL[dtype] + 2.0 ** -22 * np.abs(rl[fin])).all(), what


LARGE = [("bf16", 128, "mfma"), ("f16", 64, "mfma"), ("f16", 128, "split"),
         ("f32", 64, "f32"), ("f32", 64, "f32split"), ("bf16", 72, "generic")]


@pytest.mark.parametrize("cfg", LARGE, ids=lambda c: "_".join(map(str, c)))
def test_large_finite_mask(cfg, monkeypatch):
    import scaled_dot_product_flash_amd as sdpa
    dtype, D, path = cfg
    Lq, Lk = (100, 3000) if path == "split" else ((40, 700) if path == "f32split" else (70, 200))
    B, Hq, Hkv = (1, 4, 4) if path in ("split", "f32split") else (2, 4, 2)
    spec = synth.Spec("large", B, Hq, Hkv, Lq, Lk, D, dtype, seed=51 + D, lse=True)
    case = synth.generate(spec)
    rng = np.random.default_rng(77)
    mask = _large_mask_rows(rng, Lq, Lk)[None, None].repeat(B, axis=0)
    case = synth.Case(spec, case.q, case.k, case.v, None, np.ascontiguousarray(mask))
    if path == "generic":
        monkeypatch.setenv("SDPA_FLASH_KERNEL", "generic")
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy, return_lse=True)
        want = {"mfma": "prefill_mfma", "split": "prefill_mfma", "f32": "prefill_f32",
                "f32split": "prefill_f32", "generic": "generic"}[path]
        assert sdpa.last_kernel() == want
        if path in ("split", "f32split"):
            assert sdpa.last_workspace_bytes() > 0
        ro, rl = pu.run_oracle(case, policy)
        assert np.isfinite(ro[:, :, :4]).all() and np.isfinite(ro[:, :, 5]).all()
        _compare_large(o, lse, ro, rl, dtype, policy, what="%s %s" % (cfg, policy))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("mode", DECODE_MODES)
def test_large_finite_mask_decode(dtype, mode, monkeypatch):
    import scaled_dot_product_flash_amd as sdpa
    spec = synth.DECODE_F16.replace(dtype=dtype, batch=6, k_len=300, seed=61)
    case = synth.generate(spec)
    case.key_lens[:] = [300, 150, 77, 300, 33, 256]
    rng = np.random.default_rng(78)
    mask = _large_mask_rows(rng, 6, 300)[:, None, None, :]
    case = synth.Case(spec, case.q, case.k, case.v, case.key_lens, np.ascontiguousarray(mask))
    monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
    for policy in ("nan", "zero"):
        o, lse, _ = pu.run_hip(case, policy, return_lse=True)
        assert sdpa.last_kernel() == mode
        ro, rl = pu.run_oracle(case, policy)
        _compare_large(o, lse, ro, rl, dtype, policy, what="decode %s %s" % (dtype, policy))


# fp32 at long key lengths (OneGPU "Attention", "Accuracy at long key
# lengths": a single running sum lost accuracy at thousands of keys; the fp32
# kernel sums each tile into zero-started partials).  Q is scaled so the
# scores spread with standard deviation 3 to 12 (natural units).  The scaled
# error (max |gpu - oracle| / max |oracle|) is printed beside the page's 1e-5
# fp32 figure; the bound is the fp32 tolerance.
@pytest.mark.parametrize("lk,spread", [(4096, 3.0), (4096, 12.0), (8192, 6.0)])
def test_fp32_long_keys_accuracy(lk, spread):
    import scaled_dot_product_flash_amd as sdpa
    spec = synth.Spec("f32-long", 1, 4, 2, 64, lk, 64, "f32", seed=70 + lk % 97, causal=False,
                      lse=True)
    case = synth.generate(spec)
    # score std = |q| |k| scale: scale q so that scale * |q| * |k| ~ spread
    q = (case.q * np.float32(spread)).astype(np.float32)
    case = synth.Case(spec, q, case.k, case.v, None, None)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() == "prefill_f32"
    ro, rl = pu.run_oracle(case, "nan")
    err = pu.compare(o, ro, lse, rl, "f32", "nan", what="f32 Lk=%d spread %g" % (lk, spread))
    print("fp32 Lk=%d score std %.0f: max|err| %.3g, scaled %.3g (page: 1e-5 bound)"
          % (lk, spread, err, err / np.abs(ro).max()))


# The model shapes the OneGPU "Attention" page times ("Performance"), fp32
# and fp16, compared in full against the oracle: MiniLM (head 32), BERT-base
# B8 S512, the Whisper-small encoder (1500 keys), a decoder step against 448
# cached keys and one-query cross-attention over the 1500 encoder keys.
@pytest.mark.parametrize("name", sorted(synth.PAGE_SHAPES))
def test_page_model_shapes(name):
    spec = synth.PAGE_SHAPES[name]
    case = synth.generate(spec)
    o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
    assert sdpa.last_kernel() != "generic"
    ro, rl = pu.run_oracle(case, "nan")
    pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=name)


def test_decode_mode_chosen_by_shape():
    """Small decodes (each wave a few steps) run one workgroup per unit with
    no merge; long caches run the split over equal shares plus the merge."""
    small = synth.PAGE_SHAPES["Whisper-small decoder step B1 H12 cache448 D64 fp16"]
    small32 = synth.PAGE_SHAPES["Whisper-small decoder step B1 H12 cache448 D64"]
    long = synth.DECODE_F16.replace(batch=2, q_heads=8, kv_heads=2, k_len=8192, seed=62)
    long32 = long.replace(dtype="f32", seed=63)
    for spec, want in ((small, "decode_unit"), (small32, "decode_unit"), (long, "decode_splitk"),
                       (long32, "decode_splitk")):
        case = synth.generate(spec)
        o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
        assert sdpa.last_kernel() == want, spec.name
        ro, rl = pu.run_oracle(case, "nan")
        pu.compare(o, ro, lse, rl, spec.dtype, "nan", what=spec.name)


# Forward calls with one query row run on the decode kernels (both modes):
# non-causal cross-attention, a global causal offset with a window and
# document starts, the per-entry end-aligned rule with softcap and sinks,
# and a broadcast key mask with lengths.
FORWARD_ONE_ROW = {
    "whisper_cross_f16": synth.PAGE_SHAPES["Whisper-small cross-attention B1 H12 Lq1 Lk1500 D64 fp16"],
    "offset_window_docs_bf16": synth.CAUSAL_GQA_BF16.replace(
        batch=3, q_heads=8, kv_heads=2, q_len=1, k_len=500, causal_offset=300, local_window=60,
        docs="random", seed=63),
    "end_softcap_sink_f16": synth.CHUNK_F16.replace(
        batch=6, q_heads=8, kv_heads=2, q_len=1, k_len=900, lens="cross", lens_zero_at=2,
        lens_full_at=3, softcap=10.0, sink="heads", seed=64),
    "mask_lens_bf16_D128": synth.CROSS_MASK_F16.replace(
        dtype="bf16", batch=8, q_heads=8, kv_heads=8, q_len=1, k_len=777, head_dim=128, seed=65),
    "gqa_cross_f32": synth.PAGE_SHAPES["Whisper-small cross-attention B1 H12 Lq1 Lk1500 D64"].replace(
        batch=2, q_heads=16, kv_heads=4, seed=68),
    "mask_lens_f32_D64": synth.CROSS_MASK_F16.replace(
        dtype="f32", batch=6, q_heads=16, kv_heads=4, q_len=1, k_len=555, head_dim=64, seed=66),
    "offset_window_docs_f32": synth.CAUSAL_GQA_F32.replace(
        batch=3, q_heads=8, kv_heads=2, q_len=1, k_len=500, head_dim=128, causal_offset=300,
        local_window=60, docs="random", seed=67),
}


def test_small_mha_f32_one_row_stays_on_the_f32_kernel():
    """fp32 single-row forwards without head groups and with fewer than 64 kv
    heads in all run on the fp32 prefill kernel (its key ranges spread the few
    heads wider); with head groups they run on the decode kernels."""
    cross = synth.PAGE_SHAPES["Whisper-small cross-attention B1 H12 Lq1 Lk1500 D64"]
    for spec, want in ((cross, "prefill_f32"), (cross.replace(q_heads=48, seed=69), "decode_unit")):
        case = synth.generate(spec)
        o, lse, _ = pu.run_hip(case, "nan", return_lse=True)
        assert sdpa.last_kernel() == want, spec
        ro, rl = pu.run_oracle(case, "nan")
        pu.compare(o, ro, lse, rl, spec.dtype, "nan", what="%s %s" % (spec.name, want))


@pytest.mark.parametrize("name", sorted(FORWARD_ONE_ROW))
@pytest.mark.parametrize("policy", ["nan", "zero"])
@pytest.mark.parametrize("mode", DECODE_MODES)
def test_forward_one_query_row_on_decode_kernels(name, policy, mode, monkeypatch):
    spec = FORWARD_ONE_ROW[name]
    assert spec.q_len == 1 and not spec.decode
    case = synth.generate(spec)
    monkeypatch.setenv("SDPA_FLASH_KERNEL", mode)
    o, lse, _ = pu.run_hip(case, policy, return_lse=True)
    assert sdpa.last_kernel() == mode
    ro, rl = pu.run_oracle(case, policy)
    pu.compare(o, ro, lse, rl, spec.dtype, policy, what="%s %s" % (name, mode))
