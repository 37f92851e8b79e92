"""bench.py's host logic on the CPU: the multi-GPU refusal, the counter
summaries it writes from rocprofv3 CSV output, and the checks that keep a
stale summary out of the roofline."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from scaled_dot_product_flash_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scales_and_sums_kernels(tmp_path):
    # Two kernels per launch (a split kernel and its merge), two dispatches each.
    run = str(tmp_path / "run")
    _write_counters(run, [("void sdpa::(anonymous namespace)::dec_split<1>", "FETCH_SIZE", 100.0),
                          ("void sdpa::(anonymous namespace)::dec_split<1>", "FETCH_SIZE", 300.0),
                          ("dec_merge", "FETCH_SIZE", 10.0), ("dec_merge", "FETCH_SIZE", 10.0),
                          ("void sdpa::(anonymous namespace)::dec_split<1>", "WRITE_SIZE", 8.0),
                          ("dec_merge", "WRITE_SIZE", 2.0),
                          ("unrelated", "FETCH_SIZE", 1e9)])
    cal = str(tmp_path / "cal")
    # A 1 MiB copy: FETCH_SIZE reads half the bytes, WRITE_SIZE all of them.
    _write_counters(cal, [("copy_kernel(x)", "FETCH_SIZE", 512.0),
                          ("copy_kernel(x)", "WRITE_SIZE", 1024.0)])
    out = str(tmp_path / "s.txt")
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize", out,
                    "--kind", "counters", "--kernel", "dec_", "--dirs", run, "--calib-dirs", cal,
                    "--calib-bytes", str(1 << 20), "--sources", "decode",
                    "--algorithmic-bytes", "1000", "--title", "t", "--command", "c"],
                   check=True, capture_output=True, timeout=120)
    vals = {}
    for line in open(out):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    assert float(vals["fetch_kib_per_launch"]) == 210.0       # mean 200 + mean 10
    assert float(vals["write_kib_per_launch"]) == 10.0
    assert float(vals["fetch_scale"]) == 2.0 and float(vals["write_scale"]) == 1.0
    assert int(vals["hbm_bytes_per_launch"]) == (210 * 2 + 10) * 1024
    # The stamp matches the current decode sources, so bench.py reads it back...
    src_hash = bench.kernel_source_hash(bench.DECODE_SOURCES)
    assert vals["kernel_source_hash"] == src_hash
    # (an absolute path is read as given)
    assert bench.read_traffic(out, src_hash) == (210 * 2 + 10) * 1024
    # ... and ignores it for any other source.
    assert bench.read_traffic(out, "0" * 16) is None


def test_utilisation_ratios(tmp_path):
    run = str(tmp_path / "u")
    k = "prefill_kernel<1>"
    _write_counters(run, [(k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 50.0),
                          (k, "GRBM_GUI_ACTIVE", 8 * 100.0),
                          (k, "SQ_WAVE_CYCLES", 1000.0), (k, "SQ_ACTIVE_INST_VALU", 250.0),
                          (k, "SQ_WAIT_INST_ANY", 400.0), (k, "SQ_LDS_BANK_CONFLICT", 5.0),
                          (k, "SQ_LDS_IDX_ACTIVE", 100.0),
                          (k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0)])
    out = str(tmp_path / "u.txt")
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize", out,
                    "--kernel", "prefill_kernel", "--dirs", run, "--sources", "none",
                    "--algorithmic-flops", "1024"], check=True, capture_output=True, timeout=120)
    text = open(out).read()
    assert "mfma_busy: 0.5\n" in text
    assert "valu_issue_per_wave: 0.25\n" in text
    assert "wait_any_per_wave: 0.4\n" in text
    assert "lds_bank_conflict_per_access: 0.05\n" in text
    assert "mfma_flop_per_kernel_flop: 1.0\n" in text


def test_live_kv_bytes_counts_live_keys_only():
    spec = synth.DECODE_F16.replace(batch=3, k_len=100, local_window=9)
    case = synth.generate(spec)
    case.key_lens[:] = [0, 5, 100]
    # window 9: at most 10 live keys per entry
    want = (0 + 5 + 10) * spec.kv_heads * spec.head_dim * 2 * 2
    assert bench.live_kv_bytes(case) == want


def test_visible_flops_causal_square():
    spec = synth.CAUSAL_GQA_F32.replace(batch=1, q_heads=2, kv_heads=1, q_len=8, k_len=8)
    case = synth.generate(spec)
    pairs = 8 * 9 // 2
    assert bench.visible_flops(case) == 4.0 * spec.head_dim * 2 * pairs


def test_source_hash_ignores_comments_only():
    """Counter summaries are keyed to the kernels' code: comment and layout
    edits keep the hash, a changed token or string literal does not."""
    a = 'int f(int x) { // add one\n  return x + 1; /* done */ }\nconst char* s = "a // b";\n'
    b = 'int f(int x) {\n    return x + 1;\n}\n// trailing note\nconst char* s = "a // b";'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("x + 1", "x + 2"))
    assert bench.code_text(a) != bench.code_text(a.replace('"a // b"', '"a / b"'))


def test_other_workload_filter_rejects_unknown_names():
    """--only others --workload NAME runs just that workload (for counter
    passes over one of them); a name that is not one of them is refused
    before anything runs."""
    import pytest
    with pytest.raises(SystemExit, match="unknown workload"):
        bench.other_workloads(None, synth, 1, 0, only=["no_such_workload"])
