"""Throughput of the fused-attention hot path on one MI355X.

A step is one attn_forward call over the bf16 causal GQA prefill workload
(B=4, Hq=32, Hkv=8, Lq=Lk=4096, D=128, positions-first, fp32 LSE output);
`value` is its attention TFLOP/s (4*B*Hq*Lq*Lk*D, halved under the causal
rule).  The fp16 decode workload (B=64, Hq=32, Hkv=8, cache 8192, per-batch
lengths uniform in [1, 8192]) is timed the same way after it, rotating over
three copies of the cache so that no call finds the previous call's K/V in
the last-level cache, and reported under "decode" as KV-read GB/s.  Inputs
are synthetic (seeded N(0,1)) and resident in HBM before timing starts.
Kernel durations come from HIP events recorded around each call on the
stream the kernels run on, after about a second of untimed work that brings
the GPU clock up (then the W warmup steps).  The graphics clock is sampled
(amdsmi, mean over the XCDs) while the headline step runs back to back, and
plain MFMA / streaming loops give this part's reachable ceilings as context.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

  --summarize OUT ...   turns rocprofv3 output into the short text summaries
                        kept under profiles/ (no GPU needed); see --help.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16_TFLOPS = 2516.6     # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
PEAK_SCLK_MHZ = 2400.0             # the clock the published peaks assume
METRIC = "attention TFLOP/s (prefill) + KV GB/s (decode), % of MI355X roofline"

# Sources whose text decides each kernel's code: a committed counter summary
# is used only while their hash matches the one stamped in it.
PREFILL_SOURCES = ["prefill_mfma.hip", "mfma_common.h", "device_common.h", "attn_internal.h"]
DECODE_SOURCES = ["decode.hip", "mfma_common.h", "device_common.h", "attn_internal.h"]
PREFILL_TAG = "prefill_mfma_bf16_causal_B4H32L4096D128"
DECODE_TAG = "decode_splitk_f16_B64H32_cache8192D128"


def code_text(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that comment and layout edits do not change a kernel's source hash."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                      # string or character literal, copied whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc", n)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def read_summary(summary: str, src_hash: str):
    """key: value fields of a committed profiles/ summary, or None when it is
    missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != src_hash:
        return None
    return vals


def read_traffic(summary: str, src_hash: str):
    """HBM bytes per launch from a FETCH_SIZE / WRITE_SIZE summary, or None."""
    vals = read_summary(summary, src_hash)
    try:
        return None if vals is None else float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_utilisation(summary: str, src_hash: str):
    """The derived ratios of a committed unit-utilisation counter summary."""
    vals = read_summary(summary, src_hash)
    if vals is None:
        return None
    out = {}
    for k in ("mfma_busy", "valu_issue_per_wave", "lds_issue_per_wave", "wait_any_per_wave",
              "wait_lds_per_wave", "lds_bank_conflict_per_access", "mfma_flop_per_kernel_flop"):
        try:
            out[k] = float(vals[k])
        except (KeyError, ValueError):
            out[k] = None
    return out


class ClockSampler:
    """Samples the graphics clock of the GPU torch runs on through amdsmi's
    gpu_metrics (current_gfxclks, one value per XCD).  Measurement context
    only: every failure leaves it disabled with the reason."""

    def __init__(self, torch):
        self.handle, self.reason = None, ""
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            props = torch.cuda.get_device_properties(0)
            bus = getattr(props, "pci_bus_id", None)
            if bus is not None:
                for h in handles:
                    bdf = str(amdsmi.amdsmi_get_gpu_device_bdf(h))
                    if int(bdf.split(":")[1], 16) == int(bus):
                        self.handle = h
                        break
            if self.handle is None and len(handles) == 1:
                self.handle = handles[0]
            if self.handle is None:
                self.reason = "could not match torch's device to an amdsmi handle"
            else:
                self.read()
        except Exception as e:                      # noqa: BLE001 - context only
            self.handle, self.reason = None, "amdsmi: %s" % (str(e)[:120],)

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        vals = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and c > 0]
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [m["current_gfxclk"]]
        return float(np.mean(vals)) if vals else None

    def during(self, fn, seconds: float = 0.6):
        """Mean / min / max MHz over samples taken while fn runs back to back."""
        if self.handle is None:
            return {"sclk_mhz": None, "reason": self.reason}
        import threading
        import torch
        samples, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    v = self.read()
                except Exception:                   # noqa: BLE001
                    v = None
                if v is not None:
                    samples.append(v)
                time.sleep(0.005)

        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = threading.Thread(target=loop, daemon=True)
        t0 = time.perf_counter()
        t.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
        stop.set()
        t.join(timeout=2.0)
        if not samples:
            return {"sclk_mhz": None, "reason": "no clock samples"}
        return {"sclk_mhz": round(float(np.mean(samples)), 1),
                "sclk_min_mhz": round(float(np.min(samples)), 1),
                "sclk_max_mhz": round(float(np.max(samples)), 1), "samples": len(samples),
                "source": "amdsmi gpu_metrics current_gfxclks, mean over XCDs, sampled while "
                          "the step runs back to back"}


def settle(fn, seconds: float = 1.0):
    """Run fn until the GPU has been busy for `seconds`: the MI355X clock ramps
    up over the first few hundred milliseconds of load, and kernels timed on a
    cold part read up to ~20% slow.  Not timed."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()


_SLEEP_CYCLES_PER_MS = []


def hold_gpu(ms: float) -> bool:
    """Queue a spin kernel of about `ms` on the current stream (torch's
    _sleep, calibrated once with events), so that calls enqueued behind it
    run back to back on the GPU however slowly the host issues them."""
    import torch
    try:
        if not _SLEEP_CYCLES_PER_MS:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(100000)
            a.record()
            torch.cuda._sleep(2000000)
            b.record()
            torch.cuda.synchronize()
            _SLEEP_CYCLES_PER_MS.append(2000000 / max(a.elapsed_time(b), 1e-3))
        torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS[0]))
        return True
    except Exception:                               # noqa: BLE001 - timing aid only
        return False


def time_calls(fn, steps: int, warmup: int, settle_s: float = 1.0, queue_ahead: bool = False):
    """Per-call HIP event durations (ms) on the current stream, plus wall time.
    With queue_ahead the timed calls are enqueued behind a spin kernel and
    timed as one span (two events around all of them, divided by the count):
    back-to-back GPU time per call, for calls shorter than their host-side
    launch cost; the wall time is then the host's enqueue time."""
    import torch
    if settle_s > 0:
        settle(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if queue_ahead and hold_gpu(1.0 + 0.1 * steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        t1 = time.perf_counter()
        b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / steps] * steps, (t1 - t0) * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    durs = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return durs, wall


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline_prefill(case, target_s: float = 12.0):
    """The float64 oracle, as it stands, on a bounded sample of query rows of the
    same workload, scaled to TFLOP/s with the same causal FLOP count per row."""
    import oracle
    s = case.spec
    rng = np.random.default_rng(7)
    threads = oracle.max_threads()

    def run(n):
        rows = np.stack([rng.integers(0, s.batch, n), rng.integers(0, s.q_heads, n),
                         rng.integers(0, s.q_len, n)], axis=1).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention(case.q, case.k, case.v, dtype=s.dtype, layout=s.q_layout,
                         kv_layout=s.kv_layout, causal=s.causal, causal_offset=s.causal_offset,
                         rows=rows)
        dt = time.perf_counter() - t0
        flops = float(np.sum(4.0 * s.head_dim * (rows[:, 2] + 1)))   # visible keys of row i: i+1
        return n, dt, flops

    n, dt = max(threads, 8), 0.0
    while True:                      # grow the sample until it runs >= 1 s
        n, dt, _ = run(n)
        if dt >= 1.0 or n >= 1 << 20:
            break
        n *= 4
    n2 = int(min(1 << 21, n * target_s / max(dt, 1e-3)))
    n2, dt2, flops2 = run(n2)
    return {"value": flops2 / dt2 / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d random query rows of the bf16 causal prefill workload (float64 "
                      "three-pass oracle, %.1f s)" % (n2, dt2)}


def visible_flops(case) -> float:
    """4*D flop per visible (query row, key) pair, summed over all rows and
    heads: key lengths, the causal rule, its offset and a local window
    applied (keys a mask hides are still counted; the kernels compute their
    scores)."""
    s = case.spec
    Lq, Lk = s.q_len, s.k_len
    lens = (np.full(s.batch, Lk) if case.key_lens is None
            else np.clip(case.key_lens.astype(np.int64), 0, Lk))
    i = np.arange(Lq, dtype=np.int64)
    pairs = 0
    for b in range(s.batch):
        L = int(lens[b])
        if s.causal:
            d = (L - Lq if s.causal_offset == "end"
                 else (Lk - Lq if s.causal_offset is None else int(s.causal_offset)))
            hi = np.clip(i + d + 1, 0, L)
            lo = (np.clip(i + d - s.local_window, 0, None) if s.local_window >= 0
                  else np.zeros_like(i))
        else:
            hi, lo = np.full(Lq, L, np.int64), np.zeros(Lq, np.int64)
        if case.doc_start is not None:
            lo = np.maximum(lo, case.doc_start[b].astype(np.int64))
        pairs += int(np.clip(hi - lo, 0, None).sum())
    return 4.0 * s.head_dim * s.q_heads * pairs


def workload_tensors(case):
    """Device copies of a synthetic case's inputs (int8 caches kept int8)."""
    import torch
    s = case.spec
    kv_dtype = None if s.kv_quant else s.dtype
    dev = (lambda a: torch.from_numpy(a).cuda()) if s.kv_quant else \
        (lambda a: to_dev(a, kv_dtype))
    opt = (lambda a: None if a is None else torch.from_numpy(a).cuda())
    return dict(q=to_dev(case.q, s.dtype), k=dev(case.k), v=dev(case.v), mask=opt(case.mask),
                lens=opt(case.key_lens), sink=opt(case.head_sink), docs=opt(case.doc_start),
                k_scale=opt(case.k_scale), v_scale=opt(case.v_scale))


def workload_call(sdpa, case, t, policy: str, out):
    """A no-argument callable running one forward / decode call of the case."""
    s = case.spec
    var = dict(local_window=s.local_window, softcap=s.softcap, sink=s.sink is not None,
               head_sink=t["sink"], doc_start=t["docs"], masked_rows=policy,
               return_lse=s.lse, out=out, mask=t["mask"])
    if s.decode:
        quant = {} if t["k_scale"] is None else dict(k_scale=t["k_scale"], v_scale=t["v_scale"])
        return lambda: sdpa.decode(t["q"], t["k"], t["v"], t["lens"], layout=s.q_layout,
                                   kv_layout=s.kv_layout, **var, **quant)
    return lambda: sdpa.forward(t["q"], t["k"], t["v"], layout=s.q_layout, kv_layout=s.kv_layout,
                                causal=s.causal, causal_offset=s.causal_offset,
                                key_lens=t["lens"], **var)


def live_kv_bytes(case) -> float:
    """K and V bytes a decode call must read: live keys per entry (capped by a
    local window) x kv heads x D x 2 tensors x element size."""
    s = case.spec
    lens = (np.full(s.batch, s.k_len, np.float64) if case.key_lens is None
            else case.key_lens.astype(np.float64))
    if s.local_window >= 0:
        lens = np.minimum(lens, s.local_window + 1)
    elem = 1 if s.kv_quant else {"f32": 4, "f16": 2, "bf16": 2}[s.dtype]
    return float(lens.sum()) * s.kv_heads * s.head_dim * 2 * elem


def other_workloads(sdpa, synth, steps: int, warmup: int, only=None):
    """The other workloads (report only): the smaller named workloads, the
    extensions' workloads and the pages' model shapes.  Calls under 100 us are
    re-timed back to back behind a short spin kernel, so us_per_call is GPU
    time even where the host's launch cost (host_us_per_call) is the longer;
    tflops counts visible (row, key) pairs only; decode lines add the GB/s of
    live K/V read.  only: workload keys (synth names) to run, else all."""
    import torch
    out = []
    specs = [(n, synth.WORKLOADS[n]) for n in ("tiny_f32", "causal_gqa_f32", "cross_mask_f16")]
    specs += [(n, synth.EXTRA_WORKLOADS[n])
              for n in ("chunk_f16", "long_chunk_bf16", "window_bf16", "softcap_sink_bf16",
                        "docs_bf16", "d96_bf16", "d256_bf16", "d100_bf16", "d96_f32",
                        "decode_window_f16", "decode_int8_f16", "decode_d96_f16",
                        "decode_f32")]
    specs += list(synth.PAGE_SHAPES.items())
    if only:
        unknown = set(only) - {n for n, _ in specs}
        if unknown:
            raise SystemExit("unknown workload(s): %s" % ", ".join(sorted(unknown)))
        specs = [(n, s) for n, s in specs if n in only]
    for _, spec in specs:
        case = synth.generate(spec)
        t = workload_tensors(case)
        o = torch.empty_like(t["q"])
        for policy in (("nan", "zero") if spec.mask else ("nan",)):
            f = workload_call(sdpa, case, t, policy, o)
            f()
            kern = sdpa.last_kernel()
            durs, host = time_calls(f, steps, warmup, settle_s=0.3)
            ms = float(np.mean(durs))
            queued = ms * 1e3 < 100.0      # short calls: time them back to back instead
            if queued:
                durs, host = time_calls(f, steps, 0, settle_s=0.0, queue_ahead=True)
                ms = float(np.mean(durs))
            line = {"workload": spec.name, "kernel": kern, "us_per_call": round(ms * 1e3, 2),
                    "timing": "back-to-back span" if queued else "per-call events",
                    "host_us_per_call": round(host * 1e3 / steps, 2),
                    "tflops": round(visible_flops(case) / (ms * 1e-3) / 1e12, 3),
                    "dtype": spec.dtype if not spec.kv_quant else spec.dtype + "/i8"}
            if spec.mask:
                line["masked_rows"] = policy
            if spec.decode:
                gb = live_kv_bytes(case)
                line["gbs"] = round(gb / (ms * 1e-3) / 1e9, 1)
                if spec.kv_quant:
                    line["fp16_equiv_gbs"] = round(2 * gb / (ms * 1e-3) / 1e9, 1)
            out.append(line)
        del t, o
    return out


def ceilings(torch, sampler=None):
    """Plain MFMA and streaming loops (libsdpa_ceilings.so): what this part
    reaches without attention's dependencies, as context for the fractions."""
    import ctypes
    path = os.path.join(ROOT, "scaled_dot_product_flash_amd", "libsdpa_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError("%s is missing: run python -m scaled_dot_product_flash_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.sdpa_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.sdpa_ceiling_read.argtypes = [vp, sz, vp, ctypes.c_int, vp]
    lib.sdpa_ceiling_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError("%s launch failed (%d)" % (what, rc))

    res = {}
    n_wg, iters = 256 * 8, 1000                 # 8 workgroups of 4 waves per CU
    acc = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    f = lambda: check(lib.sdpa_ceiling_mfma_bf16(n_wg, iters, vp(acc.data_ptr()), stream),  # noqa
                      "mfma loop")
    durs, _ = time_calls(f, 10, 2, 0.5)
    ms = float(np.mean(durs))
    flops = float(n_wg) * 4 * iters * 32 * 32768
    res["mfma_bf16_loop"] = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                             "ms_per_call": round(ms, 4),
                             "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 /
                                                   PEAK_MFMA_BF16_TFLOPS, 4)}
    if sampler is not None:
        res["mfma_bf16_loop"]["clock"] = sampler.during(f, 0.4)
    del acc
    nbytes = 1 << 32                            # 4 GiB streaming read
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    r_wg = 256 * 32
    sink = torch.empty(r_wg * 256, dtype=torch.int32, device="cuda")
    g = lambda: check(lib.sdpa_ceiling_read(vp(buf.data_ptr()), nbytes, vp(sink.data_ptr()),  # noqa
                                            r_wg, stream), "read")
    durs, _ = time_calls(g, 10, 2, 0.3)
    ms = float(np.mean(durs))
    res["stream_read"] = {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
                          "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del buf, sink
    half = 1 << 31                              # 2 GiB -> 2 GiB copy
    src = torch.ones(half // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    h = lambda: check(lib.sdpa_ceiling_copy(vp(src.data_ptr()), vp(dst.data_ptr()), half,  # noqa
                                            r_wg, stream), "copy")
    durs, _ = time_calls(h, 10, 2, 0.3)
    ms = float(np.mean(durs))
    res["stream_copy"] = {"gbs": round(2 * half / (ms * 1e-3) / 1e9, 1),
                          "bytes_read_plus_written": 2 * half,
                          "frac_of_peak": round(2 * half / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if not torch.equal(dst[:1024], src[:1024]):
        raise RuntimeError("ceiling copy did not copy")
    del src, dst
    return res


# ---------------------------------------------------------------------------
# rocprofv3 output -> the short summaries kept under profiles/ (no GPU).

def _csv_rows(dirs, suffix):
    import csv
    import glob
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
            with open(f, newline="") as fh:
                yield from csv.DictReader(fh)


def _short(name: str) -> str:
    for junk in ("void sdpa::(anonymous namespace)::", "(anonymous namespace)::", "sdpa::"):
        name = name.replace(junk, "")
    return name[:100]


def _counter_means(dirs, match: str):
    """{counter: (sum over the matching kernels of their per-dispatch mean,
    min, max, dispatches)} -- one launch runs each matching kernel once (a
    split kernel and its merge, say) -- and the per-kernel means."""
    acc = {}
    for r in _csv_rows(dirs, "counter_collection.csv"):
        if match in r["Kernel_Name"]:
            acc.setdefault((r["Counter_Name"], _short(r["Kernel_Name"])), []).append(
                float(r["Counter_Value"]))
    per = {key: (float(np.mean(v)), float(np.min(v)), float(np.max(v)), len(v))
           for key, v in acc.items()}
    tot = {}
    for (ctr, _), (m, lo, hi, n) in per.items():
        t = tot.get(ctr, (0.0, 0.0, 0.0, 0))
        tot[ctr] = (t[0] + m, t[1] + lo, t[2] + hi, t[3] + n)
    return tot, per


def summarize(args):
    """Write a profiles/ summary from rocprofv3 CSV output directories."""
    all_srcs = sorted(f for f in os.listdir(os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc"))
                      if f.endswith((".hip", ".h", ".cpp")))
    srcs = {"prefill": PREFILL_SOURCES, "decode": DECODE_SOURCES, "all": all_srcs}.get(args.sources)
    lines = ["# " + t for t in args.title]
    lines += ["#", "# Commands (from the repository root, TMPDIR=/tmp):"]
    lines += ["#   " + c for c in args.command]
    fields = {}
    if srcs:
        fields["kernel_source_hash"] = kernel_source_hash(srcs)
    fields["kernel_match"] = args.kernel
    if args.kind == "stats":
        rows = list(_csv_rows(args.dirs, "kernel_stats.csv"))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        lines += ["#", "# %-96s %7s %12s %7s" % ("kernel", "calls", "avg us", "% time")]
        for r in rows[:40]:
            lines.append("# %-96s %7s %12.2f %7.2f" % (
                r["Name"].replace("void sdpa::(anonymous namespace)::", "")[:96], r["Calls"],
                float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
        hit = [r for r in rows if args.kernel in r["Name"]]
        if not hit:
            raise SystemExit("no kernel matching %r in the stats" % args.kernel)
        calls = sum(int(r["Calls"]) for r in hit)
        tot = sum(float(r["TotalDurationNs"]) for r in hit)
        fields["calls"] = calls
        fields["avg_us"] = round(tot / calls / 1e3, 3)
    else:
        c, per = _counter_means(args.dirs, args.kernel)
        if not c:
            raise SystemExit("no counters for a kernel matching %r" % args.kernel)
        lines += ["#", "# per dispatch, mean over the run's dispatches of each kernel:"]
        for (k, kn) in sorted(per):
            m, lo, hi, n = per[(k, kn)]
            lines.append("#   %-28s %14.6g  (n=%d, min %.6g, max %.6g)  %s" % (
                k, m, n, lo, hi, kn[:60]))
        g = {k: v[0] for k, v in c.items()}
        if "FETCH_SIZE" in g or "WRITE_SIZE" in g:
            cal = _counter_means(args.calib_dirs, "copy_kernel")[0] if args.calib_dirs else {}
            cb = args.calib_bytes / 1024.0
            fs = cb / cal["FETCH_SIZE"][0] if "FETCH_SIZE" in cal else 1.0
            ws = cb / cal["WRITE_SIZE"][0] if "WRITE_SIZE" in cal else 1.0
            if cal:
                lines += ["#", "# calibration: a %d-byte copy (copy_kernel of the ceilings "
                          "library) reads FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB" % (
                              args.calib_bytes, cal.get("FETCH_SIZE", (0,))[0],
                              cal.get("WRITE_SIZE", (0,))[0])]
            fk, wk = g.get("FETCH_SIZE"), g.get("WRITE_SIZE")
            if fk is not None:
                fields["fetch_kib_per_launch"] = round(fk, 1)
                fields["fetch_scale"] = round(fs, 5)
            if wk is not None:
                fields["write_kib_per_launch"] = round(wk, 1)
                fields["write_scale"] = round(ws, 5)
            if fk is not None and wk is not None:
                fields["hbm_bytes_per_launch"] = int(round((fk * fs + wk * ws) * 1024))
            if args.algorithmic_bytes:
                fields["algorithmic_bytes_per_launch"] = int(args.algorithmic_bytes)
                if "hbm_bytes_per_launch" in fields:
                    fields["traffic_over_algorithmic"] = round(
                        fields["hbm_bytes_per_launch"] / args.algorithmic_bytes, 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in g and "GRBM_GUI_ACTIVE" in g:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; MFMA busy cycles over
            # the 1024 SIMDs.
            fields["mfma_busy"] = round(g["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                        (1024.0 * g["GRBM_GUI_ACTIVE"] / 8.0), 4)
        wc = g.get("SQ_WAVE_CYCLES")
        for key, ctr in (("valu_issue_per_wave", "SQ_ACTIVE_INST_VALU"),
                         ("lds_issue_per_wave", "SQ_ACTIVE_INST_LDS"),
                         ("wait_any_per_wave", "SQ_WAIT_INST_ANY"),
                         ("wait_lds_per_wave", "SQ_WAIT_INST_LDS")):
            if wc and ctr in g:
                fields[key] = round(g[ctr] / wc, 4)
        if "SQ_LDS_BANK_CONFLICT" in g and g.get("SQ_LDS_IDX_ACTIVE"):
            fields["lds_bank_conflict_per_access"] = round(
                g["SQ_LDS_BANK_CONFLICT"] / g["SQ_LDS_IDX_ACTIVE"], 5)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in g and args.algorithmic_flops:
            # one MOPS unit is 512 flop
            fields["mfma_flop_per_kernel_flop"] = round(
                g["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 / args.algorithmic_flops, 4)
    lines += ["#"] + ["# " + n for n in args.note]
    lines += ["%s: %s" % (k, v) for k, v in fields.items()]
    with open(args.summarize, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads' lines")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the MFMA-loop / streaming ceilings")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed calls before each workload's warmup (clock ramp)")
    ap.add_argument("--workload", action="append", default=[],
                    help="with --only others: run just this workload (repeatable)")
    ap.add_argument("--only", choices=["prefill", "decode", "ceilings", "others",
                                       "calibrate-copy"],
                    help="run one part only (for profiling runs)")
    g = ap.add_argument_group("summaries of rocprofv3 output (no GPU)")
    g.add_argument("--summarize", metavar="OUT", help="write a profiles/ summary to OUT")
    g.add_argument("--kind", choices=["counters", "stats"], default="counters")
    g.add_argument("--kernel", default="prefill_mfma_kernel", help="kernel name substring")
    g.add_argument("--dirs", nargs="*", default=[], help="rocprofv3 -d output directories")
    g.add_argument("--calib-dirs", nargs="*", default=[],
                   help="FETCH_SIZE / WRITE_SIZE runs of --only calibrate-copy")
    g.add_argument("--calib-bytes", type=int, default=1 << 28)
    g.add_argument("--algorithmic-bytes", type=float, default=0.0)
    g.add_argument("--algorithmic-flops", type=float, default=0.0)
    g.add_argument("--sources", choices=["prefill", "decode", "all", "none"], default="prefill")
    g.add_argument("--title", action="append", default=[])
    g.add_argument("--command", action="append", default=[])
    g.add_argument("--note", action="append", default=[])
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the hot path here is a single-GPU kernel and no "
              "multi-GPU run is part of this build (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_flash_amd as sdpa
    from scaled_dot_product_flash_amd import synth

    torch.cuda.set_device(0)
    if args.only == "calibrate-copy":
        # A copy of known size through the ceilings library's copy kernel:
        # its FETCH_SIZE / WRITE_SIZE readings scale the attention kernels'.
        import ctypes
        lib = ctypes.CDLL(os.path.join(ROOT, "scaled_dot_product_flash_amd",
                                       "libsdpa_ceilings.so"))
        vp = ctypes.c_void_p
        lib.sdpa_ceiling_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
        src = torch.ones(1 << 26, dtype=torch.int32, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            rc = lib.sdpa_ceiling_copy(vp(src.data_ptr()), vp(dst.data_ptr()), 1 << 28, 8192,
                                       vp(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError("copy launch failed (%d)" % rc)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 28, "dispatches": 3}))
        return
    if args.only == "ceilings":
        print(json.dumps({"ceilings": ceilings(torch)}), flush=True)
        return
    if args.only == "others":
        print(json.dumps({"other_workloads": other_workloads(sdpa, synth, args.steps,
                                                             args.warmup, args.workload)}),
              flush=True)
        return
    result = {}
    case = None
    if args.only in (None, "prefill"):
        spec = synth.CAUSAL_GQA_BF16
        case = synth.generate(spec)
        q, k, v = (to_dev(x, spec.dtype) for x in (case.q, case.k, case.v))
        out = torch.empty_like(q)

        def step():
            sdpa.forward(q, k, v, causal=True, causal_offset=0, return_lse=True, out=out)

        step()
        kernel = sdpa.last_kernel()
        durs, wall = time_calls(step, args.steps, args.warmup, args.settle)
        ms = float(np.mean(durs))
        tflops = spec.flops / (ms * 1e-3) / 1e12
        src_hash = kernel_source_hash(PREFILL_SOURCES)
        traffic = read_traffic(PREFILL_TAG + "_pmc.txt", src_hash)
        sampler = ClockSampler(torch)
        clock = sampler.during(step, 0.6) if args.only is None else {"sclk_mhz": None}
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel_ms": round(ms, 4), "kernel_source_hash": src_hash,
                "clock": clock,
                "unit_utilisation": read_utilisation(PREFILL_TAG + "_mfma_pmc.txt", src_hash)}
        if clock.get("sclk_mhz"):
            roof["frac_at_measured_clock"] = round(
                tflops / (PEAK_MFMA_BF16_TFLOPS * clock["sclk_mhz"] / PEAK_SCLK_MHZ), 4)
        result.update({
            "metric": METRIC,
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(wall / args.steps, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "bf16 causal GQA prefill B=4 Hq=32 Hkv=8 Lq=Lk=4096 D=128, "
                                   "positions-first, fp32 LSE", "batch": 4, "q_heads": 32,
                       "kv_heads": 8, "seq_len": 4096, "head_dim": 128, "causal": True,
                       "kernel": kernel, "parallelism": "single GPU"},
            "roofline": roof,
        })
        del q, k, v, out

    if args.only in (None, "decode") and not args.no_decode:
        dspec = synth.DECODE_F16
        dcase = synth.generate(dspec)
        dq = to_dev(dcase.q, dspec.dtype)
        caches = [(to_dev(dcase.k, dspec.dtype), to_dev(dcase.v, dspec.dtype))]
        for _ in range(2):       # three copies of the 2 GiB cache, used in turn
            caches.append((caches[0][0].clone(), caches[0][1].clone()))
        lens = torch.from_numpy(dcase.key_lens).cuda()
        dout = torch.empty_like(dq)
        turn = [0]

        def dstep():
            dk, dv = caches[turn[0] % len(caches)]
            turn[0] += 1
            sdpa.decode(dq, dk, dv, lens, kv_layout="bhsd", out=dout)

        dstep()
        dkernel = sdpa.last_kernel()
        ddurs, _ = time_calls(dstep, args.steps, args.warmup, args.settle)
        dms = float(np.mean(ddurs))
        kv_bytes = live_kv_bytes(dcase)
        gbs = kv_bytes / (dms * 1e-3) / 1e9
        dhash = kernel_source_hash(DECODE_SOURCES)
        result["decode"] = {
            "workload": "fp16 decode B=64 Hq=32 Hkv=8 D=128, head-first cache of 8192, "
                        "lengths uniform in [1, 8192] (seed 4), three cache copies in turn",
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(dms, 4),
            "kv_bytes": kv_bytes, "kernel": dkernel,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic(DECODE_TAG + "_pmc.txt", dhash),
                         "kernel_source_hash": dhash},
        }
        del dq, caches, dout

    if args.only is None and not args.no_ceilings:
        result["ceilings"] = ceilings(torch, ClockSampler(torch))

    if args.only is None and not args.no_others:
        result["other_workloads"] = other_workloads(sdpa, synth, args.steps, args.warmup)

    if args.only is None and not args.no_cpu_baseline and case is not None:
        result["cpu_baseline"] = cpu_baseline_prefill(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
