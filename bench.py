"""Throughput of the fused-attention hot path on one MI355X.

A step is one attn_forward call over the bf16 causal GQA prefill workload
(B=4, Hq=32, Hkv=8, Lq=Lk=4096, D=128, positions-first, fp32 LSE output);
`value` is its attention TFLOP/s (4*B*Hq*Lq*Lk*D, halved under the causal
rule).  The fp16 decode workload (B=64, Hq=32, Hkv=8, cache 8192, per-batch
lengths uniform in [1, 8192]) is timed the same way after it and reported
under "decode" as KV-read GB/s.  Inputs are synthetic (seeded N(0,1)) and
resident in HBM before timing starts.  Kernel durations come from HIP events
recorded around each call on the stream the kernels run on, after about a
second of untimed work that brings the GPU clock up (then the W warmup steps).

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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
METRIC = "attention TFLOP/s (prefill) + KV GB/s (decode), % of MI355X roofline"


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when the summary is missing or was taken on a different kernel source."""
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
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


def time_calls(fn, steps: int, warmup: int, settle_s: float = 1.0):
    """Per-call HIP event durations (ms) on the current stream, plus wall time."""
    import torch
    if settle_s > 0:
        settle(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
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


def other_workloads(sdpa, synth, steps: int, warmup: int):
    """The smaller workloads and the chunked-prefill extension, timed like the
    headline (report only).  tflops counts visible (row, key) pairs only."""
    import torch
    out = []
    specs = [synth.WORKLOADS[n] for n in ("tiny_f32", "causal_gqa_f32", "cross_mask_f16")]
    specs += [synth.EXTRA_WORKLOADS[n]
              for n in ("chunk_f16", "long_chunk_bf16", "window_bf16", "softcap_sink_bf16",
                        "docs_bf16", "d96_bf16",
                        "d256_bf16")]
    for spec in specs:
        case = synth.generate(spec)
        q, k, v = (to_dev(x, spec.dtype) for x in (case.q, case.k, case.v))
        mask = None if case.mask is None else torch.from_numpy(case.mask).cuda()
        lens = None if case.key_lens is None else torch.from_numpy(case.key_lens).cuda()
        sink = None if case.head_sink is None else torch.from_numpy(case.head_sink).cuda()
        docs = None if case.doc_start is None else torch.from_numpy(case.doc_start).cuda()
        o = torch.empty_like(q)
        for policy in (("nan", "zero") if spec.mask else ("nan",)):
            def f():
                sdpa.forward(q, k, v, layout=spec.q_layout, kv_layout=spec.kv_layout,
                             causal=spec.causal, causal_offset=spec.causal_offset, mask=mask,
                             key_lens=lens, masked_rows=policy, return_lse=spec.lse,
                             local_window=spec.local_window, softcap=spec.softcap,
                             sink=spec.sink is not None, head_sink=sink, doc_start=docs, out=o)
            f()
            kern = sdpa.last_kernel()
            durs, _ = time_calls(f, steps, warmup, settle_s=0.3)
            ms = float(np.mean(durs))
            out.append({"workload": spec.name, "masked_rows": policy, "kernel": kern,
                        "ms_per_call": round(ms, 5),
                        "tflops": round(visible_flops(case) / (ms * 1e-3) / 1e12, 3),
                        "dtype": spec.dtype})
    # Decode with a local window and head sinks: KV GB/s over the live ranges.
    spec = synth.EXTRA_WORKLOADS["decode_window_f16"]
    case = synth.generate(spec)
    q, k, v = (to_dev(x, spec.dtype) for x in (case.q, case.k, case.v))
    lens = torch.from_numpy(case.key_lens).cuda()
    sink = torch.from_numpy(case.head_sink).cuda()
    o = torch.empty_like(q)

    def g():
        sdpa.decode(q, k, v, lens, kv_layout=spec.kv_layout, local_window=spec.local_window,
                    softcap=spec.softcap, sink=True, head_sink=sink, out=o)
    g()
    kern = sdpa.last_kernel()
    durs, _ = time_calls(g, steps, warmup, settle_s=0.3)
    ms = float(np.mean(durs))
    live = np.minimum(case.key_lens.astype(np.float64), spec.local_window + 1)
    kv_bytes = float(live.sum()) * spec.kv_heads * spec.head_dim * 2 * 2
    out.append({"workload": spec.name, "kernel": kern, "ms_per_call": round(ms, 5),
                "gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "dtype": spec.dtype})
    # Decode against an int8 cache: GB/s of int8 K/V bytes read (1 byte each).
    spec = synth.EXTRA_WORKLOADS["decode_int8_f16"]
    case = synth.generate(spec)
    q = to_dev(case.q, spec.dtype)
    k = torch.from_numpy(case.k).cuda()
    v = torch.from_numpy(case.v).cuda()
    lens = torch.from_numpy(case.key_lens).cuda()
    ks = torch.from_numpy(case.k_scale).cuda()
    vs = torch.from_numpy(case.v_scale).cuda()
    o = torch.empty_like(q)

    def h():
        sdpa.decode(q, k, v, lens, kv_layout=spec.kv_layout, k_scale=ks, v_scale=vs, out=o)
    h()
    kern = sdpa.last_kernel()
    durs, _ = time_calls(h, steps, warmup, settle_s=0.3)
    ms = float(np.mean(durs))
    kv_bytes = float(case.key_lens.astype(np.float64).sum()) * spec.kv_heads * spec.head_dim * 2
    out.append({"workload": spec.name, "kernel": kern, "ms_per_call": round(ms, 5),
                "gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
                "fp16_equiv_gbs": round(2 * kv_bytes / (ms * 1e-3) / 1e9, 1), "dtype": "f16/i8"})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the tiny fp32, fp32 causal GQA and fp16 cross-attention lines")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed calls before each workload's warmup (clock ramp)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the hot path here is a single-GPU kernel and no "
              "multi-GPU run is part of this build (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_flash_amd as sdpa
    from scaled_dot_product_flash_amd import synth

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # A copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale the
        # counters taken on the attention kernels.
        src = torch.ones(1 << 27, dtype=torch.float16, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 28, "dispatches": 3}))
        return
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
    src_hash = kernel_source_hash(["prefill_mfma.hip"])
    traffic = read_traffic("prefill_mfma_bf16_causal_B4H32L4096D128_pmc.txt", src_hash)
    result = {
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
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel_ms": round(ms, 4), "kernel_source_hash": src_hash},
    }
    del q, k, v, out

    if not args.no_decode:
        dspec = synth.DECODE_F16
        dcase = synth.generate(dspec)
        dq, dk, dv = (to_dev(x, dspec.dtype) for x in (dcase.q, dcase.k, dcase.v))
        lens = torch.from_numpy(dcase.key_lens).cuda()
        dout = torch.empty_like(dq)

        def dstep():
            sdpa.decode(dq, dk, dv, lens, kv_layout="bhsd", out=dout)

        dstep()
        dkernel = sdpa.last_kernel()
        ddurs, _ = time_calls(dstep, args.steps, args.warmup, args.settle)
        dms = float(np.mean(ddurs))
        kv_bytes = float(np.sum(dcase.key_lens.astype(np.float64))) * dspec.kv_heads * \
            dspec.head_dim * 2 * 2
        gbs = kv_bytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "workload": "fp16 decode B=64 Hq=32 Hkv=8 D=128, head-first cache of 8192, "
                        "lengths uniform in [1, 8192] (seed 4)",
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(dms, 4),
            "kv_bytes": kv_bytes, "kernel": dkernel,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic("decode_splitk_f16_B64H32_cache8192D128_pmc.txt",
                                                 kernel_source_hash(["decode.hip"])),
                         "kernel_source_hash": kernel_source_hash(["decode.hip"])},
        }
        del dq, dk, dv, dout

    if not args.no_others:
        result["other_workloads"] = other_workloads(sdpa, synth, args.steps, args.warmup)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
