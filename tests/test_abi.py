"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, its struct layout matches the binding, and malformed calls are
rejected on the host before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import scaled_dot_product_flash_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa_flash.h")


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared_symbols() == sorted(sdpa.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = sdpa.load_library()
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sdpa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b[TW] (attn_\w+)", out))
    assert set(_declared_symbols()) <= exported


def test_version_string():
    assert b"gfx950" in sdpa.load_library().attn_version()


def test_struct_layout_matches_c(tmp_path):
    """sizeof/offsetof from the C compiler equal the ctypes layout."""
    fields = [f[0] for f in sdpa.Problem._fields_]
    src = tmp_path / "layout.c"
    body = "".join('printf("%s %%zu\\n", offsetof(attn_problem, %s));' % (f, f) for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sdpa_flash.h"\n'
                   'int main(void){printf("size %%zu\\n", sizeof(attn_problem));'
                   'printf("layout %%zu\\n", sizeof(attn_layout));%s return 0;}\n' % body)
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)]).decode().splitlines())
    assert int(got["size"]) == ctypes.sizeof(sdpa.Problem)
    assert int(got["layout"]) == ctypes.sizeof(sdpa.Layout)
    for f in fields:
        assert int(got[f]) == getattr(sdpa.Problem, f).offset, f


def _problem(**kw):
    p = sdpa.Problem()
    p.batch, p.q_heads, p.kv_heads, p.q_len, p.k_len, p.head_dim = 1, 4, 2, 8, 8, 64
    p.dtype = sdpa.DTYPE_BF16
    p.causal_offset = sdpa.CAUSAL_OFFSET_DEFAULT
    for lay, H, L in (("q", 4, 8), ("k", 2, 8), ("v", 2, 8), ("o", 4, 8)):
        setattr(p, lay, sdpa.Layout(0, L * H * 64, 64, H * 64))
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation rejects first


@pytest.mark.parametrize("change,status", [
    (dict(q_heads=3), sdpa.ERR_INVALID),
    (dict(kv_heads=0), sdpa.ERR_INVALID),
    (dict(head_dim=0), sdpa.ERR_INVALID),
    (dict(head_dim=257), sdpa.ERR_INVALID),
    (dict(dtype=7), sdpa.ERR_INVALID),
    (dict(causal=2), sdpa.ERR_INVALID),
    (dict(masked_rows=5), sdpa.ERR_INVALID),
    (dict(batch=-1), sdpa.ERR_INVALID),
    (dict(q_len=-3), sdpa.ERR_INVALID),
    (dict(scale=float("nan")), sdpa.ERR_INVALID),
    (dict(scale=-1.0), sdpa.ERR_INVALID),
    (dict(q=sdpa.Layout(0, -1, 64, 256)), sdpa.ERR_INVALID),
    (dict(batch=70000), sdpa.ERR_UNSUPPORTED),
    (dict(window=-1), sdpa.ERR_INVALID),
    (dict(window=4), sdpa.ERR_INVALID),              # a window needs the causal rule
    (dict(softcap=-1.0), sdpa.ERR_INVALID),
    (dict(softcap=float("nan")), sdpa.ERR_INVALID),
    (dict(sink=2), sdpa.ERR_INVALID),
    (dict(head_sink=0x1000), sdpa.ERR_INVALID),      # values without sink = 1
    (dict(q_heads=70000, kv_heads=2), sdpa.ERR_UNSUPPORTED),
    (dict(k=sdpa.Layout(0, 0, 64, 1 << 60)), sdpa.ERR_INVALID),     # extent past 2^62
    (dict(k=sdpa.Layout(0, 0, 64, 1 << 62)), sdpa.ERR_INVALID),     # 7 * 2^62 would wrap int64
    (dict(causal=0, window=0, doc_start=None, k_scale=0x1000), sdpa.ERR_INVALID),  # scale, no int8
])
def test_invalid_problem_rejected_before_launch(change, status):
    lib = sdpa.load_library()
    p = _problem(**change)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None)
    assert rc == status
    assert lib.attn_last_error()
    n = ctypes.c_size_t(123)
    assert lib.attn_workspace_size(ctypes.byref(p), sdpa.OP_FORWARD, ctypes.byref(n)) == status
    assert n.value == 0


def test_null_pointers_rejected():
    lib = sdpa.load_library()
    p = _problem()
    assert lib.attn_forward(None, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None) \
        == sdpa.ERR_INVALID
    assert lib.attn_forward(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, None, None, 0,
                            None) == sdpa.ERR_INVALID
    assert lib.attn_forward(ctypes.byref(p), FAKE, None, FAKE, FAKE, None, None, None, None, 0,
                            None) == sdpa.ERR_INVALID
    assert lib.attn_workspace_size(ctypes.byref(p), 0, None) == sdpa.ERR_INVALID
    assert lib.attn_workspace_size(ctypes.byref(p), 9, ctypes.byref(ctypes.c_size_t())) \
        == sdpa.ERR_INVALID


def test_negative_mask_and_lse_strides_rejected():
    lib = sdpa.load_library()
    p = _problem()
    p.mask = sdpa.Layout(0, 0, -8, 8)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None)
    assert rc == sdpa.ERR_INVALID and b"mask" in lib.attn_last_error()
    p = _problem()
    p.lse = sdpa.Layout(0, -1, 8, 1)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None)
    assert rc == sdpa.ERR_INVALID and b"lse" in lib.attn_last_error()
    # Strides whose products would wrap 64-bit offsets.
    p = _problem()
    p.mask = sdpa.Layout(0, 0, 0, 1 << 62)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None)
    assert rc == sdpa.ERR_INVALID and b"mask" in lib.attn_last_error()
    p = _problem()
    p.lse = sdpa.Layout(0, 0, 1 << 62, 1)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None)
    assert rc == sdpa.ERR_INVALID and b"lse" in lib.attn_last_error()


def test_decode_requires_one_query_row():
    lib = sdpa.load_library()
    p = _problem(q_len=2)
    assert lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0,
                           None) == sdpa.ERR_INVALID
    assert b"q_len" in lib.attn_last_error()


def test_empty_problem_is_a_no_op():
    """batch = 0 or q_len = 0 returns OK without touching the device."""
    lib = sdpa.load_library()
    for change in (dict(batch=0), dict(q_len=0)):
        p = _problem(**change)
        assert lib.attn_forward(ctypes.byref(p), None, None, None, None, None, None, None, None,
                                0, None) == sdpa.OK


def test_workspace_size_is_host_only():
    n = sdpa.workspace_size(_problem(), sdpa.OP_FORWARD)
    assert n >= 0


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 2, 8)
    with pytest.raises(ValueError):
        sdpa.forward(q, q, q)


def test_decode_workspace_is_checked_before_launch():
    lib = sdpa.load_library()
    p = _problem(q_len=1, k_len=4096, dtype=sdpa.DTYPE_F16, head_dim=128)
    for lay, H, L in (("q", 4, 1), ("k", 2, 4096), ("v", 2, 4096), ("o", 4, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * 128, 128, H * 128))
    need = sdpa.workspace_size(p, sdpa.OP_DECODE)
    assert need > 0
    # As a forward problem the same shape is one small workgroup, whose keys
    # are cut into ranges: whole records of (m, l, acc[128]) per query row.
    fwd = sdpa.workspace_size(p, sdpa.OP_FORWARD)
    assert fwd > 0 and fwd % (4 * 1 * (128 + 4) * 4) == 0
    rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None)
    assert rc == sdpa.ERR_WORKSPACE
    rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE,
                         need - 4, None)
    assert rc == sdpa.ERR_WORKSPACE
    assert b"workspace" in lib.attn_last_error()
    # The partial records are written 16 bytes at a time.
    odd = ctypes.c_void_p(0x1008)
    rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, odd, need,
                         None)
    assert rc == sdpa.ERR_INVALID and b"aligned" in lib.attn_last_error()


def test_forward_one_row_runs_decode_kernels_with_their_workspace():
    """A forward call with one query row runs on the decode kernels, so its
    workspace covers theirs, and it is checked before anything runs."""
    lib = sdpa.load_library()
    p = _problem(q_len=1, k_len=4096, dtype=sdpa.DTYPE_F16, head_dim=128)
    for lay, H, L in (("q", 4, 1), ("k", 2, 4096), ("v", 2, 4096), ("o", 4, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * 128, 128, H * 128))
    fwd = sdpa.workspace_size(p, sdpa.OP_FORWARD)
    assert fwd == sdpa.workspace_size(p, sdpa.OP_DECODE) > 0
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0,
                          None)
    assert rc == sdpa.ERR_WORKSPACE and b"decode needs" in lib.attn_last_error()


def test_decode_workspace_covers_the_forward_fallback():
    """A decode shape the split decode path does not take (head dim 250, not
    whole 16-byte chunks) runs as a forward call, whose few query blocks split
    the keys and whose K/V are staged: the decode workspace covers that call."""
    lib = sdpa.load_library()
    p = _problem(batch=2, q_heads=12, kv_heads=3, q_len=1, k_len=681, head_dim=250,
                 dtype=sdpa.DTYPE_BF16, causal=1)
    for lay, H, L in (("q", 12, 1), ("k", 3, 681), ("v", 3, 681), ("o", 12, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * 250, 250, H * 250))
    fwd = sdpa.workspace_size(p, sdpa.OP_FORWARD)
    assert fwd > 0
    assert sdpa.workspace_size(p, sdpa.OP_DECODE) >= fwd
    rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None)
    assert rc == sdpa.ERR_WORKSPACE


def test_fp32_forward_split_needs_workspace():
    """The fp32 causal GQA shape (few row blocks) is cut into key ranges and
    needs a workspace; without it the call fails before launching."""
    lib = sdpa.load_library()
    p = _problem(batch=2, q_heads=12, kv_heads=4, q_len=512, k_len=512, head_dim=64,
                 dtype=sdpa.DTYPE_F32, causal=1)
    for lay, H, L in (("q", 12, 512), ("k", 4, 512), ("v", 4, 512), ("o", 12, 512)):
        setattr(p, lay, sdpa.Layout(0, L * H * 64, 64, H * 64))
    need = sdpa.workspace_size(p, sdpa.OP_FORWARD)
    assert need > 0
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None)
    assert rc == sdpa.ERR_WORKSPACE
    # The split writes 16-byte records: a misaligned workspace is refused too.
    odd = ctypes.c_void_p(0x1004)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, odd, need,
                          None)
    assert rc == sdpa.ERR_INVALID and b"aligned" in lib.attn_last_error()


def test_matrix_core_forward_split_workspace():
    """bf16/fp16 prefill with too few query blocks for the GPU cuts the keys
    into ranges (shape only) and needs a 16-byte aligned workspace, checked
    before anything is launched; the full-size prefill shape needs none."""
    lib = sdpa.load_library()
    p = _problem(batch=1, q_heads=8, kv_heads=2, q_len=100, k_len=8192, head_dim=128, causal=1)
    for lay, H, L in (("q", 8, 100), ("k", 2, 8192), ("v", 2, 8192), ("o", 8, 100)):
        setattr(p, lay, sdpa.Layout(0, L * H * 128, 128, H * 128))
    need = sdpa.workspace_size(p, sdpa.OP_FORWARD)
    per_range = 1 * 8 * 100 * (128 + 4) * 4
    assert need > 0 and need % per_range == 0 and 2 <= need // per_range <= 32
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, None)
    assert rc == sdpa.ERR_WORKSPACE
    odd = ctypes.c_void_p(0x1004)
    rc = lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, odd, need,
                          None)
    assert rc == sdpa.ERR_INVALID and b"aligned" in lib.attn_last_error()
    big = _problem(batch=4, q_heads=32, kv_heads=8, q_len=4096, k_len=4096, head_dim=128,
                   causal=1)
    for lay, H in (("q", 32), ("k", 8), ("v", 8), ("o", 32)):
        setattr(big, lay, sdpa.Layout(0, 4096 * H * 128, 128, H * 128))
    assert sdpa.workspace_size(big, sdpa.OP_FORWARD) == 0


def test_offset_sentinels_match_c(tmp_path):
    src = tmp_path / "sentinels.c"
    src.write_text('#include <stdio.h>\n#include <inttypes.h>\n#include "sdpa_flash.h"\n'
                   'int main(void){printf("%" PRId64 " %" PRId64 "\\n",'
                   '(int64_t)ATTN_CAUSAL_OFFSET_DEFAULT,(int64_t)ATTN_CAUSAL_OFFSET_KEY_END);'
                   'return 0;}\n')
    exe = tmp_path / "sentinels"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    d, e = map(int, subprocess.check_output([str(exe)]).split())
    assert (d, e) == (sdpa.CAUSAL_OFFSET_DEFAULT, sdpa.CAUSAL_OFFSET_KEY_END)


def test_int8_cache_is_decode_only_and_checked():
    lib = sdpa.load_library()
    p = _problem(kv_int8=1, k_quant=1, v_quant=2, k_scale=0x1000, v_scale=0x1000)
    assert lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0,
                            None) == sdpa.ERR_UNSUPPORTED
    for bad in (dict(kv_int8=1, k_quant=0, v_quant=1, k_scale=0x1000, v_scale=0x1000),
                dict(kv_int8=1, k_quant=1, v_quant=1, k_scale=0x1000, v_scale=None),
                dict(kv_int8=0, k_quant=1),
                dict(kv_int8=2)):
        p = _problem(**bad)
        assert lib.attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                                0, None) == sdpa.ERR_INVALID


@pytest.mark.parametrize("D,split", [(128, True), (64, True), (100, True), (4, True),
                                     (96, True), (130, False), (256, False), (50, False)])
def test_decode_f32_head_dims(D, split):
    """fp32 decode on the decode kernels: head dims that are whole 16-byte
    chunks (multiples of 4) up to 128, padded to 64 or 128, with the same
    records; others run as a forward call.  A forward call with one query row
    needs the same workspace."""
    B, Hq, Hkv, Lk = 3, 8, 2, 1000
    p = _problem(batch=B, q_heads=Hq, kv_heads=Hkv, q_len=1, k_len=Lk, head_dim=D,
                 dtype=sdpa.DTYPE_F32)
    for lay, H, L in (("q", Hq, 1), ("k", Hkv, Lk), ("v", Hkv, Lk), ("o", Hq, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * D, D, H * D))
    need = sdpa.workspace_size(p, sdpa.OP_DECODE)
    dp = 64 if D <= 64 else 128
    split_bytes = (B * Hkv + 2048) * (Hq // Hkv) * (dp + 4) * 4
    if split:
        assert need >= split_bytes
        assert sdpa.workspace_size(p, sdpa.OP_FORWARD) == need
    else:
        assert need != split_bytes


@pytest.mark.parametrize("D,int8,split", [(96, 0, True), (40, 0, True), (8, 0, True),
                                         (136, 0, True), (256, 0, True), (112, 1, True),
                                         (48, 1, True), (208, 1, True), (24, 1, False),
                                         (100, 0, False), (250, 0, False)])
def test_decode_split_head_dims(D, int8, split):
    """Head dims that are whole 16-byte chunks (16-value chunks for an int8
    cache) up to 256 take the split decode path, padded to 64, 128 or 256:
    its workspace holds padded records for up to 2048 waves.  Others fall
    back to the forward path, or are unsupported with an int8 cache."""
    lib = sdpa.load_library()
    B, Hq, Hkv, Lk = 3, 8, 2, 1000
    kw = dict(batch=B, q_heads=Hq, kv_heads=Hkv, q_len=1, k_len=Lk, head_dim=D,
              dtype=sdpa.DTYPE_F16)
    if int8:
        kw.update(kv_int8=1, k_quant=1, v_quant=1, k_scale=0x1000, v_scale=0x1000)
    p = _problem(**kw)
    for lay, H, L in (("q", Hq, 1), ("k", Hkv, Lk), ("v", Hkv, Lk), ("o", Hq, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * D, D, H * D))
    need = sdpa.workspace_size(p, sdpa.OP_DECODE)
    dp = 64 if D <= 64 else (128 if D <= 128 else 256)
    split_bytes = (B * Hkv + 2048) * (Hq // Hkv) * (dp + 4) * 4
    if split:
        assert need >= split_bytes
    elif int8:
        rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE,
                             1 << 30, None)
        assert rc == sdpa.ERR_UNSUPPORTED and b"multiple of 16" in lib.attn_last_error()
    else:
        assert need != split_bytes


def test_int8_cache_with_fp32_query_is_unsupported():
    """An int8 cache is read with fp16/bf16 queries only; an fp32 problem with
    kv_int8 = 1 is refused before anything runs (the fp32 decode kernels read
    fp32 rows)."""
    lib = sdpa.load_library()
    B, Hq, Hkv, Lk, D = 2, 8, 2, 256, 64
    p = _problem(batch=B, q_heads=Hq, kv_heads=Hkv, q_len=1, k_len=Lk, head_dim=D,
                 dtype=sdpa.DTYPE_F32, kv_int8=1, k_quant=1, v_quant=1, k_scale=0x1000,
                 v_scale=0x1000)
    for lay, H, L in (("q", Hq, 1), ("k", Hkv, Lk), ("v", Hkv, Lk), ("o", Hq, 1)):
        setattr(p, lay, sdpa.Layout(0, L * H * D, D, H * D))
    rc = lib.attn_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE,
                         1 << 30, None)
    assert rc == sdpa.ERR_UNSUPPORTED and b"fp16/bf16" in lib.attn_last_error()
