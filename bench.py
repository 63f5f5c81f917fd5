"""Benchmark: paged decode latency and achieved HBM bandwidth on KV bytes.

One step is one pkv_decode call (attention kernel plus, when the planner
splits the KV range, the log-sum-exp reducer) over the headline workload, the
largest of the five on one GPU: MLA decode, B=512, one query row, Hq=128 on
one shared latent head (D_qk = 576 = 512 latent + 64 rope, D_v = 512, V = the
latent rows), pages of 64 tokens, 4096 keys per request (2.42 GB of KV per
call), pages shuffled across the pool.  Inputs are seeded synthetic draws
already resident in HBM when timing starts.

Prints ONE JSON line.  `value` is KV GB/s (algorithmic KV bytes of the call /
wall time per call).  `roofline` reports the dominant kernel against the
MI355X HBM peak (8 TB/s); `cpu_baseline` is the fp64 CPU oracle timed on a
bounded sample of the same workload on the host.  `secondary` holds the same
measurements, each with its own roofline, for the other workloads (bf16 GQA
decode, FP8 ragged split decode, MLA decode q=2, causal context, the append
producer) unless --no-secondary is given; --only NAME measures one workload.
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


# The kernel sources each family is built from: a stored HBM-counter reading
# is used only while these are unchanged.
COMMON_SOURCES = ("pkv_device.h", "pkv_internal.h")
FAMILY_SOURCES = {
    "mla32": ("pkv_attn_mla.hip", "pkv_ring.h"),
    "m32": ("pkv_attn_m32.hip", "pkv_ring.h"),
    "dma": ("pkv_attn_dma.hip", "pkv_ring.h"),
    "generic": ("pkv_attn_generic.hip",),
    "mfma": ("pkv_attn_mfma.hip",),
}


def kernel_sources(kernel: str):
    fam = ("mla32" if kernel.startswith("mla32") else "m32" if kernel.startswith("m32_") else
           "dma" if kernel.startswith("dma_") else "generic" if kernel == "generic" else "mfma")
    return FAMILY_SOURCES[fam] + COMMON_SOURCES


def _src_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in kernel_sources(kernel):
        with open(os.path.join(ROOT, "paged_kv_attention_15_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str, num_splits: int):
    """HBM bytes per launch of the attention kernel from committed rocprofv3
    counter runs, or None when they are missing, were taken on other kernel
    sources or on another plan."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_hash") != _src_hash(kernel) or rec.get("plan") != [kernel, num_splits]:
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
    """Reads device 0's current sclk level (and, where the driver exposes it,
    its socket power) from sysfs every millisecond on a host thread while a
    timed region runs (the level read after the region shows the idle clock,
    not the clock the kernels ran at)."""

    def __init__(self, source):
        import glob
        import threading

        self.path = os.path.join(source, "pp_dpm_sclk") if source else None
        self.power_path, self.power_cap_w = None, None
        if source:
            for name in ("power1_average", "power1_input"):
                hits = sorted(glob.glob(os.path.join(source, "hwmon", "hwmon*", name)))
                if hits:
                    self.power_path = hits[0]
                    try:
                        cap = os.path.join(os.path.dirname(hits[0]), "power1_cap")
                        self.power_cap_w = int(open(cap).read().strip()) / 1e6
                    except (OSError, ValueError):
                        pass
                    break
        self.samples = []
        self.power_w = []
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
            if self.power_path:
                try:
                    self.power_w.append(int(open(self.power_path).read().strip()) / 1e6)
                except (OSError, ValueError):
                    self.power_path = None
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
        out = {"samples": len(v), "sclk_mhz_median": v[len(v) // 2], "sclk_mhz_min": v[0], "sclk_mhz_max": v[-1]}
        if self.power_w:
            pw = sorted(self.power_w)
            out["power_w_median"] = round(pw[len(pw) // 2], 1)
            out["power_w_max"] = round(pw[-1], 1)
            if self.power_cap_w:
                out["power_cap_w"] = round(self.power_cap_w, 1)
        return out


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


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cpu():
    """The host's CPU model (lscpu, else /proc/cpuinfo) and the cores this
    process may run on."""
    import subprocess

    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        model = next((ln.split(":", 1)[1].strip() for ln in out.splitlines() if ln.startswith("Model name")), None)
    except Exception:
        pass
    if model is None:
        try:
            model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                          if ln.startswith("model name")), None)
        except OSError:
            pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count()}


def cpu_baseline(prob, target_s: float):
    """The single-threaded fp64 C oracle on an evenly spaced sample of the
    workload's (query row, head) pairs, sized from a 16-pair probe to take
    about `target_s` seconds; reported in the metric's unit (KV GB/s, the
    sample's share of the KV bytes over its time)."""
    import numpy as np

    import oracle

    pairs = oracle.all_pairs(prob)
    t0 = time.perf_counter()
    oracle.attention(prob, pairs[np.linspace(0, len(pairs) - 1, 16).astype(np.int64)])
    per_pair = (time.perf_counter() - t0) / 16
    n = int(min(len(pairs), max(16, target_s / max(per_pair, 1e-9))))
    sample = pairs[np.linspace(0, len(pairs) - 1, n).astype(np.int64)]
    t0 = time.perf_counter()
    oracle.attention(prob, sample)
    dt = time.perf_counter() - t0
    frac = n / (prob.total_q * prob.num_qo_heads)
    kv_bytes = prob.kv_bytes() * frac  # bytes the sample's rows read, counted like the GPU metric
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {prob.total_q * prob.num_qo_heads} evenly spaced (query row, head) pairs of the "
                      f"same workload ({prob.name}), single-threaded fp64 C oracle, {dt:.1f} s",
            **host_cpu()}


# name -> (builder, the roofline that bounds it)
WORKLOADS = {
    "mla-b512-kv4096-q1": (lambda W: W.mla_b512_kv4096(q_len=1), "hbm"),
    "bf16-gqa-b32-kv4096": (lambda W: W.gqa_bf16_b32_kv4096(), "hbm"),
    "fp8-gqa-b16-ragged": (lambda W: W.gqa_fp8_b16_ragged(), "hbm"),
    "mla-b512-kv4096-q2": (lambda W: W.mla_b512_kv4096(q_len=2), "mfma"),
    "ctx-b4-q511-kv2047": (lambda W: W.context_b4_q511_kv2047(), "mfma"),
    "ctx-b4-q257-kv1024-p1024-sepkv": (lambda W: W.context_b4_q257_kv1024_p1024(separate=True), "mfma"),
}
HEADLINE = "mla-b512-kv4096-q1"


def roofline(name, prob, info, sec_per_call, bound, timing):
    """Roofline object of one workload: algorithmic KV bytes (hbm) or flops
    (mfma) per call over the measured device time per call."""
    from paged_kv_attention_15_amd import pkv

    kernel = pkv.KERNEL_NAMES[info.kernel]
    merged = info.num_splits > 1 and not info.fused_merge
    rec = {"bound": bound}
    if bound == "hbm":
        ach = prob.kv_bytes() / sec_per_call / 1e9
        rec.update(achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4))
    else:
        ach = prob.flops() / sec_per_call / 1e12
        rec.update(achieved=round(ach, 1), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                   frac=round(ach / BF16_MFMA_PEAK_TFLOPS, 4))
    rec.update(traffic=_traffic(name, kernel, info.num_splits),
               kernel=f"{kernel} attention kernel" + (" + lse_merge_kernel" if merged else ""), timing=timing)
    return rec


def config_of(name, prob, info):
    from paged_kv_attention_15_amd import pkv

    q_lens = sorted(set(int(x) for x in (prob.q_indptr[1:] - prob.q_indptr[:-1])))
    lens = prob.seq_lens
    return {"workload": name, "batch": prob.batch, "q_len": q_lens[0] if len(q_lens) == 1 else q_lens,
            "num_qo_heads": prob.num_qo_heads, "num_kv_heads": prob.num_kv_heads, "head_dim_qk": prob.head_dim_qk,
            "head_dim_v": prob.head_dim_v, "page_size": prob.page_size, "layout": prob.layout,
            "kv_len": int(lens[0]) if (lens == lens[0]).all() else [int(lens.min()), int(lens.max())],
            "kv_dtype": prob.kv_dtype, "causal": bool(prob.causal), "mla": bool(prob.mla),
            "kernel": pkv.KERNEL_NAMES[info.kernel], "num_splits": info.num_splits,
            "kv_bytes_per_call": prob.kv_bytes(), "flops_per_call": prob.flops()}


def run_workload(name, steps: int, warmup: int, single_call: bool = True, clock_source=None, num_splits=None):
    """Measure one workload: eager back-to-back calls, then the same number of
    calls replayed from HIP graphs (the reported figure), optional warm/cold
    single calls.  Returns (record, problem, wall seconds per graph-replayed call)."""
    import torch

    from paged_kv_attention_15_amd import pkv, workloads as W

    make, bound = WORKLOADS[name]
    progress(f"{name}: drawing inputs")
    prob = make(W)
    progress(f"{name}: timing")
    dp, info, wall_e, ev_e = measure(prob, steps, warmup, num_splits)
    timing = "HIP graphs of 10 back-to-back calls, replayed; one HIP event pair on the launch stream"
    with ClockSampler(clock_source) as sampler:
        try:
            wall, ev = time_graph(dp, steps, warmup)
        except Exception as exc:  # capture unavailable: the eager figures stand
            wall, ev = wall_e, ev_e
            timing = f"back-to-back eager calls (graph capture failed: {str(exc)[:120]}); one HIP event pair"
    kv = prob.kv_bytes()
    rec = {"us_per_call": round(ev * 1e6, 3), "config": config_of(name, prob, info),
           "kv_gbs": round(kv / ev / 1e9, 1), "hbm_frac": round(kv / ev / 1e9 / HBM_PEAK_GBS, 4),
           "tflops": round(prob.flops() / ev / 1e12, 2),
           "mfma_frac": round(prob.flops() / ev / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
           "fused_merge": int(info.fused_merge),
           "roofline": roofline(name, prob, info, ev, bound, timing),
           "eager": {"us_per_call": round(ev_e * 1e6, 3), "wall_us_per_call": round(wall_e * 1e6, 3),
                     "note": "back-to-back calls from the host, no graph"},
           "sclk_during": sampler.summary()}
    if single_call:
        try:
            rec["single_call"] = single_call_stats(dp, kv)
        except Exception as exc:
            rec["single_call"] = {"error": str(exc)[:200]}
    del dp
    torch.cuda.empty_cache()
    progress(f"{name}: {rec['us_per_call']} us per call ({rec['config']['kernel']})")
    return rec, prob, wall


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
    gbs = nbytes / ev / 1e9
    rec = {"us_per_call": round(ev * 1e6, 3), "bytes_per_call": nbytes, "gbs": round(gbs, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "timing": timing,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "append_kernel",
                        "note": "latency-bound, not bandwidth-bound: about 1 MB per call, one dependent "
                                "load-compute-store chain per wave plus the launch"}}
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle's bounded sample")
    ap.add_argument("--only", default=None,
                    help="measure only this workload (profiling runs): " + ", ".join(
                        list(WORKLOADS) + ["append-h64x8-b32-decode", "append-h64x8-b32-decode-e4m3-dynq"]))
    ap.add_argument("--settle", type=float, default=CLOCK_SETTLE_S,
                    help="seconds of untimed calls before each workload's warm-up (0: none)")
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

    from paged_kv_attention_15_amd import pkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkv.load_library()
    try:
        clocks = gpu_clocks()
    except Exception as exc:  # no sysfs view of the device: report why
        clocks = {"error": str(exc)[:120]}
    src = clocks.get("sclk_source")
    sec_steps, sec_warm = max(20, args.steps // 4), max(5, args.warmup // 2)
    line = {"metric": METRIC, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "data": "synthetic"}
    if args.only is None or args.only == HEADLINE:
        rec, prob, wall = run_workload(HEADLINE, args.steps, args.warmup, not args.no_single_call, src,
                                       args.num_splits)
        kv = prob.kv_bytes()
        value = kv / wall / 1e9
        if rec["sclk_during"] is not None:
            clocks["during_timed_calls"] = rec["sclk_during"]
            if clocks.get("sclk_max_mhz"):
                clocks["sclk_below_70pct_of_max"] = rec["sclk_during"]["sclk_mhz_median"] < 0.7 * clocks["sclk_max_mhz"]
        line.update({
            "value": round(value, 1),
            "unit": "GB/s",
            "ms_per_step": round(wall * 1e3, 5),
            "us_per_call": rec["us_per_call"],
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "dtype": "bf16",
            "config": rec["config"],
            "roofline": rec["roofline"],
            "tflops": rec["tflops"],
            "mfma_frac": rec["mfma_frac"],
            "eager": rec["eager"],
        })
        if "single_call" in rec:
            line["single_call"] = rec["single_call"]
        if not args.no_cpu_baseline:
            progress("CPU oracle baseline")
            line["cpu_baseline"] = cpu_baseline(prob, args.cpu_seconds)
        del prob
    line["clocks"] = clocks
    line["clock_settle_s"] = CLOCK_SETTLE_S
    if args.calibrate_copy:
        src_t = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = src_t.numel() * 4
        del src_t, dst_t
        torch.cuda.empty_cache()
    if not args.no_secondary:
        sec = {}
        for name in WORKLOADS:
            if name == HEADLINE or (args.only and name != args.only):
                continue
            sec[name], _, _ = run_workload(name, sec_steps, sec_warm, not args.no_single_call, src)
        for name, fp8 in (("append-h64x8-b32-decode", False), ("append-h64x8-b32-decode-e4m3-dynq", True)):
            if not args.only or args.only == name:
                sec[name] = append_result(sec_steps, sec_warm, fp8=fp8)
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
