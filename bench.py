"""Benchmark: paged decode latency and achieved HBM bandwidth on KV bytes.

One step is one pkv_decode call (attention kernel plus, when the planner
splits the KV range, the log-sum-exp reducer) over the headline workload:
bf16 paged GQA decode, B=32, one query row, Hq=32 / Hkv=8, D=128, HND pages of
32 tokens, 4096 keys per request, pages shuffled across the pool.  Inputs are
seeded synthetic draws already resident in HBM when timing starts.

Prints ONE JSON line.  `value` is KV GB/s (algorithmic KV bytes of the call /
wall time per call).  `roofline` reports the dominant kernel against the
MI355X HBM peak (8 TB/s); `cpu_baseline` is the fp64 CPU oracle timed on a
bounded sample of the same workload on the host.  `secondary` holds the same
measurements for the other four workloads (FP8 ragged split decode, MLA decode
q=1 / q=2, causal context) unless --no-secondary is given.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "paged decode µs/call + achieved HBM GB/s (KV bytes) as % of MI355X peak"


# Sources the headline kernel (register-staged bf16 GQA decode) is built from;
# a stored HBM-counter reading is used only while these are unchanged.
HEADLINE_SOURCES = ("pkv_attn_mfma.hip", "pkv_device.h", "pkv_internal.h")


def _src_hash() -> str:
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_15_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str, num_splits: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    they are missing, were taken on other kernel sources or on another plan."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_hash") != _src_hash() or rec.get("plan") != [kernel, num_splits]:
        return None
    return rec.get("bytes_per_launch")


def time_calls(dp, steps: int, warmup: int):
    """Time `steps` back-to-back calls after `warmup` untimed ones.

    Returns (wall seconds per call from the host clock between two device
    synchronizations, device seconds per call from one pair of HIP events
    recorded on the launch stream around the same calls)."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dp.run(stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        dp.run(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, e0.elapsed_time(e1) / 1e3 / steps


def time_graph(dp, steps: int, warmup: int):
    """Per-call time of exactly `steps` calls, captured 10 (or 1, when `steps`
    is not a multiple of 10) back to back per HIP graph and replayed (the launch
    protocol of the pages' own benchmark tables): returns (wall seconds per
    call, device seconds per call from one HIP event pair)."""
    import torch

    per_graph = 10 if steps % 10 == 0 else 1

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup)):
            dp.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            dp.run()
    reps = max(1, steps // per_graph)
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    n = reps * per_graph
    wall = (time.perf_counter() - t0) / n
    return wall, e0.elapsed_time(e1) / 1e3 / n


def single_call_stats(dp, kv_bytes: int, samples: int = 30):
    """Single calls replayed from a one-call HIP graph, one HIP event pair around
    each: warm (back to back) and cold (a 1 GiB buffer read before every call,
    outside the timed span, so L2 and the Infinity Cache hold none of the
    inputs).  The eviction pass reads rather than writes: dirty lines left by a
    write pass would be written back during the timed call and be counted as
    part of it.  Median, p10 and p90 in microseconds."""
    import numpy as np
    import torch

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dp.run()
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    torch.sum(scratch, dim=0, out=sink[0])  # the initial writes reach memory before the samples
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = {}
    for mode in ("warm", "cold"):
        ts = []
        for i in range(samples):
            if mode == "cold":
                torch.sum(scratch, dim=0, out=sink[0])
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = np.array(ts)
        med = float(np.median(ts))
        out[mode] = {"us_median": round(med, 2), "us_p10": round(float(np.percentile(ts, 10)), 2),
                     "us_p90": round(float(np.percentile(ts, 90)), 2), "gbs_median": round(kv_bytes / med / 1e3, 1)}
    del scratch, sink
    return out


def gpu_clocks():
    """Current and highest shader (sclk) and memory (mclk) clock levels of
    device 0 from its sysfs DPM tables (the entry marked '*' is the current
    one), read before the timed region (ClockSampler follows sclk during it);
    absent keys where the files are missing."""
    import glob
    import re

    import torch

    props = torch.cuda.get_device_properties(0)
    bdf = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    paths = [f"/sys/bus/pci/devices/{bdf}"]
    cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not os.path.exists(os.path.join(paths[0], "pp_dpm_sclk")) and len(cards) == 1:
        paths.append(os.path.dirname(cards[0]))  # the only card visible: it is device 0
    out = {"pci": bdf}
    for name in ("sclk", "mclk"):
        for base in paths:
            try:
                lines = open(os.path.join(base, f"pp_dpm_{name}")).read().splitlines()
            except OSError:
                continue
            levels = [(int(m.group(1)), line.strip().endswith("*"))
                      for line in lines for m in [re.search(r"(\d+)\s*[Mm]hz", line)] if m]
            if levels:
                out[f"{name}_mhz"] = next((v for v, cur in levels if cur), None)
                out[f"{name}_max_mhz"] = max(v for v, _ in levels)
                out[f"{name}_source"] = base
                break
    if out.get("sclk_mhz") and out.get("sclk_max_mhz"):
        out["sclk_below_70pct_of_max"] = out["sclk_mhz"] < 0.7 * out["sclk_max_mhz"]
    return out


class ClockSampler:
    """Reads device 0's current sclk level from sysfs every millisecond on a
    host thread while a timed region runs (the level read after the region
    shows the idle clock, not the clock the kernels ran at)."""

    def __init__(self, source):
        import threading

        self.path = os.path.join(source, "pp_dpm_sclk") if source else None
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re

        while not self._stop.is_set():
            try:
                for line in open(self.path).read().splitlines():
                    m = re.search(r"(\d+)\s*[Mm]hz", line)
                    if m and line.strip().endswith("*"):
                        self.samples.append(int(m.group(1)))
            except OSError:
                return
            self._stop.wait(0.001)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"samples": len(v), "sclk_mhz_median": v[len(v) // 2], "sclk_mhz_min": v[0], "sclk_mhz_max": v[-1]}


# MI355X's shader clock climbs from about 1 GHz to 2.2-2.4 GHz over the first
# 100-200 ms of sustained load (measured with ClockSampler: bf16 decode calls
# took 87.0 us at a median 1.1 GHz, 83.8 us from 1.5 GHz on), so every workload
# first runs untimed for this long before its W warm-up calls
CLOCK_SETTLE_S = 0.3


def settle_clocks(dp, seconds: Optional[float] = None):
    """Untimed calls for `seconds` of wall time (synchronizing every 20 calls)."""
    import torch

    seconds = CLOCK_SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            dp.run()
        torch.cuda.synchronize()


def measure(prob, steps: int, warmup: int, num_splits=None):
    from paged_kv_attention_15_amd import pkv

    # the separate reducer kernel: measured faster than the in-kernel reducer
    # (merge_counters) on the ragged e4m3 workload
    dp = pkv.upload(prob, "cuda", with_lse=False, with_err=False, num_splits=num_splits)
    info = pkv.pkv_plan(dp.args, dp.is_context)
    settle_clocks(dp)
    wall, ev_mean = time_calls(dp, steps, warmup)
    return dp, info, wall, ev_mean


def cpu_baseline(prob, max_pairs: int):
    import numpy as np

    import oracle

    pairs = oracle.all_pairs(prob)
    if len(pairs) > max_pairs:
        idx = np.linspace(0, len(pairs) - 1, max_pairs).astype(np.int64)
        pairs = pairs[idx]
    t0 = time.perf_counter()
    oracle.attention(prob, pairs)
    dt = time.perf_counter() - t0
    frac = len(pairs) / (prob.total_q * prob.num_qo_heads)
    kv_bytes = prob.kv_bytes() * frac  # bytes the sample's rows read, counted like the GPU metric
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(pairs)} of {prob.total_q * prob.num_qo_heads} (query row, head) pairs of the "
                      f"same workload, single-threaded fp64 C oracle, {dt:.1f} s"}


def secondary_results(steps: int, warmup: int, single_call: bool = True, clock_source=None, only=None):
    import torch

    from paged_kv_attention_15_amd import pkv, workloads as W

    out = {}
    cases = [
        ("fp8-gqa-b16-ragged", lambda: W.gqa_fp8_b16_ragged(), "hbm"),
        ("mla-b512-kv4096-q1", lambda: W.mla_b512_kv4096(q_len=1), "hbm"),
        ("mla-b512-kv4096-q2", lambda: W.mla_b512_kv4096(q_len=2), "mfma"),
        ("ctx-b4-q511-kv2047", lambda: W.context_b4_q511_kv2047(), "mfma"),
        ("ctx-b4-q257-kv1024-p1024-sepkv", lambda: W.context_b4_q257_kv1024_p1024(separate=True), "mfma"),
    ]
    for name, make, bound in cases:
        if only and name != only:
            continue
        prob = make()
        dp, info, wall, ev_mean = measure(prob, steps, warmup)
        with ClockSampler(clock_source) as sampler:
            try:
                wall, ev_mean = time_graph(dp, steps, warmup)
            except Exception:  # capture unavailable: keep the eager figures
                pass
        gbs = prob.kv_bytes() / ev_mean / 1e9
        tflops = prob.flops() / ev_mean / 1e12
        sc = None
        if single_call:
            try:
                sc = single_call_stats(dp, prob.kv_bytes())
            except Exception as exc:
                sc = {"error": str(exc)[:200]}
        rec = {"us_per_call": round(ev_mean * 1e6, 3), "single_call": sc,
               "kernel": pkv.KERNEL_NAMES[info.kernel], "num_splits": info.num_splits,
               "fused_merge": int(info.fused_merge),
               "kv_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
               "tflops": round(tflops, 2), "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
               "bound": bound, "kv_bytes": prob.kv_bytes(), "flops": prob.flops(),
               "sclk_during": sampler.summary()}
        out[name] = rec
        del dp
        torch.cuda.empty_cache()
    return out


def append_result(steps: int, warmup: int, fp8: bool = False):
    """The paged-KV append producer on the pages' H1 row (Hq=64 / Hkv=8, 32
    requests appending one row each, norm then RoPE, caches of 64-token pages;
    bf16 throughout, or with `fp8` e4m3 caches and e4m3 queries with a dynamic
    scale per (row, head)): per-call time as HIP-graph replays, and bytes moved
    per call."""
    import torch

    from paged_kv_attention_15_amd import pkv, workloads as W

    prob = (W.append_h64x8_b32_decode(norm_policy=2, kv_dtype=W.E4M3, q_quant=1) if fp8
            else W.append_h64x8_b32_decode(norm_policy=2))
    da = pkv.upload_append(prob, "cuda", with_err=False)
    settle_clocks(da)
    for _ in range(warmup):
        da.run()
    torch.cuda.synchronize()
    try:
        _, ev = time_graph(da, steps, warmup)
        timing = "graph"
    except Exception:
        _, ev = time_calls(da, steps, warmup)
        timing = "eager"
    nbytes = prob.bytes_moved()
    rec = {"us_per_call": round(ev * 1e6, 3), "bytes_per_call": nbytes, "gbs": round(nbytes / ev / 1e9, 1),
           "hbm_frac": round(nbytes / ev / 1e9 / HBM_PEAK_GBS, 4), "timing": timing,
           "bound": "latency (1.3 MB per call: one dependent load-compute-store chain per wave)"}
    del da
    torch.cuda.empty_cache()
    return rec


def main():
    global CLOCK_SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single-call", action="store_true",
                    help="skip the warm/cold single-call samples (profiling runs: only the timed calls)")
    ap.add_argument("--cpu-pairs", type=int, default=1024)
    ap.add_argument("--only", default=None,
                    help="run only this secondary workload after the headline (profiling runs)")
    ap.add_argument("--settle", type=float, default=CLOCK_SETTLE_S,
                    help="seconds of untimed calls before each workload's warm-up (0: none, as in profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (known bytes) to scale HBM counters")
    args = ap.parse_args()
    CLOCK_SETTLE_S = max(0.0, args.settle)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              f"Decode shards over requests or KV heads with no exchange; see the sharding note of the design.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_attention_15_amd import pkv, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkv.load_library()
    prob = W.gqa_bf16_b32_kv4096()
    dp, info, wall, ev_mean = measure(prob, args.steps, args.warmup, args.num_splits)
    kv = prob.kv_bytes()
    eager = {"us_per_call": round(ev_mean * 1e6, 3), "gbs": round(kv / ev_mean / 1e9, 1),
             "wall_gbs": round(kv / wall / 1e9, 1), "note": "back-to-back calls from the host, no graph"}
    # The pages time their kernels as CUDA-graph replays; the calls here are
    # capturable (kernels only: no allocation, memset or host sync), so the
    # headline is the same K calls replayed from HIP graphs, eager kept beside it.
    timing = "HIP graphs of 10 back-to-back calls, replayed; one HIP event pair on the launch stream"
    try:
        clocks = gpu_clocks()
    except Exception as exc:  # no sysfs view of the device: report why
        clocks = {"error": str(exc)[:120]}
    with ClockSampler(clocks.get("sclk_source")) as sampler:
        try:
            wall, ev_mean = time_graph(dp, args.steps, args.warmup)
        except Exception as exc:  # capture unavailable: the eager figures are the headline
            timing = f"back-to-back eager calls (graph capture failed: {str(exc)[:120]}); one HIP event pair"
    value = kv / wall / 1e9
    achieved = kv / ev_mean / 1e9
    during = sampler.summary()
    if during is not None:
        clocks["during_timed_calls"] = during
        if clocks.get("sclk_max_mhz"):
            clocks["sclk_below_70pct_of_max"] = during["sclk_mhz_median"] < 0.7 * clocks["sclk_max_mhz"]
    single_kernel = info.num_splits == 1
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "us_per_call": round(ev_mean * 1e6, 3),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16-gqa-b32-kv4096", "batch": 32, "q_len": 1, "num_qo_heads": 32,
                   "num_kv_heads": 8, "head_dim": 128, "page_size": 32, "kv_len": 4096, "layout": "HND",
                   "kv_dtype": "bf16", "kernel": pkv.KERNEL_NAMES[info.kernel], "num_splits": info.num_splits,
                   "kv_bytes_per_call": kv},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic("bf16-gqa-b32-kv4096", pkv.KERNEL_NAMES[info.kernel], info.num_splits),
                     "kernel": f"{pkv.KERNEL_NAMES[info.kernel]} attention kernel" + ("" if single_kernel else " + lse_merge_kernel"),
                     "timing": timing},
        "eager": eager,
        "clocks": clocks,
        "clock_settle_s": CLOCK_SETTLE_S,
    }
    if not args.no_single_call:
        try:
            line["single_call"] = single_call_stats(dp, kv)
        except Exception as exc:
            line["single_call"] = {"error": str(exc)[:200]}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(prob, args.cpu_pairs)
    del dp
    torch.cuda.empty_cache()
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = src.numel() * 4
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_secondary:
        line["secondary"] = secondary_results(max(20, args.steps // 4), max(5, args.warmup // 2),
                                              not args.no_single_call, clocks.get("sclk_source"), args.only)
        if not args.only or args.only == "append-h64x8-b32-decode":
            line["secondary"]["append-h64x8-b32-decode"] = append_result(max(20, args.steps // 4),
                                                                         max(5, args.warmup // 2))
        if not args.only or args.only == "append-h64x8-b32-decode-e4m3-dynq":
            line["secondary"]["append-h64x8-b32-decode-e4m3-dynq"] = append_result(
                max(20, args.steps // 4), max(5, args.warmup // 2), fp8=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
