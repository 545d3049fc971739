"""Benchmark of the attention hot path on one MI355X.

One step = one pass over both halves of the path, with inputs resident in
HBM before timing starts:
  * prefill: fa_fwd on the Llama-2-7B-shaped causal workload
    (B=4, Hq=Hkv=32, L=4096, D=128, bf16);
  * decode: fa_decode (split kernel + logsumexp combine) on 128 sequences,
    Hq=32, Hkv=8, D=128, bf16, cache lengths uniform on [512, 8192], 8 splits.

``value`` is the prefill throughput in algorithmic TFLOP/s (4*D per allowed
query-key pair per query head) from HIP events around every prefill launch
on the stream the kernel runs on; the decode half is reported in the same
line as algorithmic HBM GB/s (K/V rows of each cache read once, q read, o and
lse written).  ``ms_per_step`` is wall time per step over the K timed steps.

Before the W warm-up steps the step is repeated untimed for ``--settle``
seconds (``settle_s`` in the line): the GPU clocks take ~100 ms of load to
ramp up after an idle spell, and a few warm-up steps do not cover that.  The
graphics clock under the step's load is read from amd-smi after the timed
region (``sclk``).

The other prefill workloads are timed after the step loop, each launch with
its own HIP event pair, and reported under ``configs``: the long-context GQA
prefill, the D=256 prefill, the bidirectional encoder (cold: a 512 MiB buffer
is written between launches, outside the timed region, so that its inputs
are not served from the 256 MiB last-level cache) and the tiny case (µs:
HIP events around each call, host time to the launch included, and per launch
of 200 calls replayed from one HIP graph, the GPU's own time).
The paged / int8 decode, FP8 forward, backward and structured-mask workloads
follow under their own keys.  None of them is part of ``value``.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--settle SECONDS]
                    [--no-cpu-baseline] [--probe] [--only ...]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (causal prefill) + decode HBM GB/s, % roofline"
PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X published dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X published HBM3E bandwidth
PEAK_MFMA_FP8_TFLOPS = 5000.0   # MI355X published dense fp8 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "exact_tiled_attention_fa_amd", "csrc")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle", type=float, default=2.0,
                   help="seconds of untimed steps before the warm-up (clock ramp)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU oracle sample")
    p.add_argument("--with-copy", type=int, default=0, metavar="MIB",
                   help="after timing, run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--only", choices=["prefill", "decode", "masks", "paged", "bwd", "fp8",
                                      "config"],
                   default=None,
                   help="time only this part (one JSON line); config: one prefill workload "
                        "named by --config")
    p.add_argument("--config", default=None, help="with --only config: the prefill workload")
    p.add_argument("--reps", type=int, default=None,
                   help="launches per side measurement (default: per workload)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other prefill workloads (long-context, D=256, encoder, tiny)")
    p.add_argument("--no-bwd", action="store_true", help="skip the backward workload")
    p.add_argument("--bwd-workload", choices=["llama7b", "varlen16"], default=None,
                   help="with --only bwd: time only this backward workload")
    p.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward workload")
    p.add_argument("--probe", action="store_true",
                   help="also time the matrix-core probe (libfa_probe.so) on the prefill's Q "
                        "and on constant operands")
    p.add_argument("--no-sclk", action="store_true", help="do not read the clock from amd-smi")
    p.add_argument("--rates", action="store_true",
                   help="only run the instruction-rate probes (libfa_probe.so): SIMD cycles of "
                        "MFMA, FMA and exp mixes at 1 and 2 waves per SIMD")
    p.add_argument("--paged-format", choices=["native", "k8", "kv8"], default=None,
                   help="time only this paged-cache format")
    p.add_argument("--no-paged", action="store_true",
                   help="skip the paged-cache decode workloads")
    p.add_argument("--mask", default=None, help="time only this structured-mask workload")
    p.add_argument("--no-masks", action="store_true",
                   help="skip the structured-mask prefill workloads (sliding window, packed)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs of this script with "
                        "--with-copy (FETCH_SIZE, then WRITE_SIZE) into profiles/traffic.json")
    p.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                   help="no GPU work: from a rocprofv3 --kernel-trace --stats run of the default "
                        "bench and the JSON line it printed, print the per-kernel statistics and "
                        "the step prefill's average over the timed steps")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="no GPU work: per-dispatch medians of every counter in rocprofv3 --pmc "
                        "runs, for the kernels named by --kernel-match")
    p.add_argument("--kernel-match", default="fwd_kernel<fa::bf16_t, 128, true>",
                   help="substring of the kernel name for --summarize-counters")
    p.add_argument("--pmc-key", default=None,
                   help="with --summarize-pmc on a run of --only masks --mask NAME: record the "
                        "forward kernel's traffic under this key (e.g. masks:NAME)")
    return p.parse_args()


# headers every kernel includes (helpers, work map, LDS layouts): part of every digest
SHARED_HEADERS = ["fa_common.hpp", "fa_sched.hpp", "fa_lds.hpp"]


def source_digest(names) -> str:
    """Hash of a kernel's sources (the named files plus the shared headers),
    tying a counter record to the code it was taken on."""
    h = hashlib.sha256()
    for n in list(names) + [x for x in SHARED_HEADERS if x not in names]:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, digest: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        e = t.get(kernel)
        if e and e.get("source_digest") == digest:
            return e.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def summarize_pmc(fetch_dir: str, write_dir: str, copy_mib: int, key=None) -> dict:
    """HBM bytes per launch of the prefill and decode kernels from rocprofv3
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the same
    counter reads for a plain device copy of copy_mib MiB (reads and writes
    exactly copy_mib MiB)."""
    import csv
    import glob
    import statistics

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    def med(rows, pred):
        v = [x for _, n, x in rows if pred(n)]
        return statistics.median(v) if v else None

    is_copy = lambda n: "copybuffer" in n.lower()  # the runtime's device-to-device copy kernel
    if key == "fp8":
        is_fwd = lambda n: "fwd_fp8_kernel<128, fa::bf16_t, true>" in n
    else:
        is_fwd = lambda n: "fwd_kernel<fa::bf16_t, 128, true>" in n
    is_split = lambda n: "decode_split_kernel<fa::bf16_t, 128," in n  # one cache format per run
    is_comb = lambda n: "decode_combine_kernel<fa::bf16_t, 128>" in n
    fr, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    kib = copy_mib * 1024.0
    # only the calibration copies (the run also holds small input uploads)
    fr = [r for r in fr if not is_copy(r[1]) or r[2] > kib / 16]
    wr = [r for r in wr if not is_copy(r[1]) or r[2] > kib / 16]
    ff = kib / med(fr, is_copy)
    fw = kib / med(wr, is_copy)
    out = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                     "dispatch, median over dispatches), each scaled by the factor that makes a "
                     f"plain {copy_mib} MiB device copy read and write exactly {copy_mib} MiB.",
           "copy_mib": copy_mib, "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)}
    if key == "bwd":  # the three backward kernels of one fa_bwd call, summed
        parts = [(med(fr, pr), med(wr, pr)) for pr in (
            lambda n: "bwd_prep_kernel<fa::bf16_t, 128>" in n,
            lambda n: "bwd_dq_kernel<fa::bf16_t, 128, true>" in n,
            lambda n: "bwd_dkdv_kernel<fa::bf16_t, 128, true>" in n)]
        if all(a is not None and b is not None for a, b in parts):
            out["bwd"] = {"source_digest": source_digest(["fa_bwd.hip", "fa_common.hpp"]),
                          "fetch_kib": sum(a for a, _ in parts),
                          "write_kib": sum(b for _, b in parts),
                          "bytes_per_launch": int(sum(a * ff + b * fw for a, b in parts) * 1024)}
        return out
    f_k, w_k = med(fr, is_fwd), med(wr, is_fwd)
    if f_k is not None and w_k is not None and not (key or "").startswith("paged:"):
        src = ["fa_fwd_fp8.hip" if key == "fp8" else "fa_fwd.hip", "fa_common.hpp"]
        out[key or "fwd_kernel"] = {"source_digest": source_digest(src),
                             "fetch_kib": f_k, "write_kib": w_k,
                             "bytes_per_launch": int((f_k * ff + w_k * fw) * 1024)}
    parts = [(med(fr, p), med(wr, p)) for p in (is_split, is_comb)]
    if all(a is not None and b is not None for a, b in parts) and (key is None or
                                                                  key.startswith("paged:")):
        out[key or "decode"] = {"source_digest": source_digest(["fa_decode.hip", "fa_common.hpp"]),
                         "fetch_kib": sum(a for a, _ in parts), "write_kib": sum(b for _, b in parts),
                         "bytes_per_launch": int(sum(a * ff + b * fw for a, b in parts) * 1024)}
    return out


def _csv_rows(d, suffix):
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_trace(trace_dir: str, bench_json: str) -> dict:
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run of the
    default bench, and the average duration of the step's prefill launches
    over the timed steps only (the dispatches after the settle and warm-up
    steps the bench's JSON line reports), to set against its HIP-event
    figure."""
    import statistics

    with open(bench_json) as f:
        line = [ln for ln in f.read().splitlines() if ln.startswith("{")][-1]
    b = json.loads(line)
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    fwd = [r for r in trace if "fwd_kernel<fa::bf16_t, 128, true>" in r["Kernel_Name"]]
    first = b["settle_steps"] + b["warmup"]
    timed = fwd[first:first + b["steps"]]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    out = {"bench_prefill_ms_mean": b["prefill_ms"]["mean"], "bench_value": b["value"],
           "bench_frac": b["roofline"]["frac"],
           "trace_timed_prefill_us_mean": round(statistics.mean(dur), 2) if dur else None,
           "trace_timed_prefill_us_median": round(statistics.median(dur), 2) if dur else None,
           "timed_dispatches": len(dur), "first_timed_dispatch": first,
           "stats": [{k: r[k] for k in ("Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage")
                      if k in r} for r in stats]}
    if dur:
        tf = b["roofline"]["alg_flops_per_launch"] / (statistics.mean(dur) * 1e-6) / 1e12
        out["trace_timed_prefill_tflops"] = round(tf, 1)
        out["trace_timed_prefill_frac"] = round(tf / PEAK_MFMA_BF16_TFLOPS, 4)
    return out


def summarize_counters(dirs, match: str) -> dict:
    """Median over dispatches of each counter of the kernels whose name holds
    ``match``, from one or more rocprofv3 --pmc runs (one pass each)."""
    import statistics

    vals = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if match in r["Kernel_Name"]:
                key = (d, r["Dispatch_Id"])  # dispatch ids restart in every run
                vals.setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
                vals[r["Counter_Name"]][key] += float(r["Counter_Value"])
    return {k: {"median": statistics.median(v.values()), "dispatches": len(v)}
            for k, v in sorted(vals.items())}


def cpu_baseline_prefill(cfg, q, k, v, scale, target_s):
    """Time the fp64 oracle on a bounded sample of whole (batch, head) slices
    (all of them when they fit in about target_s seconds)."""
    import oracle
    from oracle.attention import _default_workers

    workers = _default_workers()
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    per_head_flops = cfg.flops() // len(pairs)
    t0 = time.perf_counter()
    oracle.attention_ref(q, k, v, scale, cfg.causal, heads=pairs[:1], workers=1)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(len(pairs), round(target_s / max(t1, 1e-3) * workers))))
    n = max(workers, n - n % workers) if n >= workers else n
    n = min(n, len(pairs))
    t0 = time.perf_counter()
    oracle.attention_ref(q, k, v, scale, cfg.causal, heads=pairs[:n], workers=workers)
    dt = time.perf_counter() - t0
    return {"value": round(per_head_flops * n / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": workers, "kind": "oracle", "host": host_cpu(),
            "sample": f"{n} of {len(pairs)} (batch, head) slices of the same workload, "
                      f"fp64 numpy, {dt:.2f} s wall"}


def cpu_baseline_decode(cfg, q, kc, vc, lens, scale):
    """The fp64 oracle's decode on the whole decode workload (every sequence
    and head), one thread per sequence over the host's cores."""
    import oracle
    from oracle.attention import _default_workers

    workers = _default_workers()
    t0 = time.perf_counter()
    oracle.decode_ref(q, kc, vc, lens, scale, workers=workers)
    dt = time.perf_counter() - t0
    from exact_tiled_attention_fa_amd import workloads as W
    byts = W.decode_bytes(cfg, lens)
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "host": host_cpu(),
            "sample": f"all {cfg.B} sequences x {cfg.Hq} heads of the same workload, fp64 numpy, "
                      f"{dt:.2f} s wall"}


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return f"{line.split(':', 1)[1].strip()} ({os.cpu_count()} logical CPUs)"
    except OSError:
        pass
    return f"{os.cpu_count()} logical CPUs"


def copy_calibration(mib, dev):
    """A plain device copy of `mib` MiB, three times: the reference the HBM
    counters are scaled by."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


PAGED_FORMATS = {"native": (False, False), "k8": (True, False), "kv8": (True, True)}
PAGE_SIZE = 16


def settle(run, seconds=0.25):
    """Untimed: repeat run() for `seconds` of wall time so that the GPU clocks
    have ramped up before a measurement (a few calls are not enough; the first
    ~100 ms of work after idle run 10-20 % slow).  Returns the number of
    calls."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            run()
        n += 4
        torch.cuda.synchronize()
    return n


def ms_stats(ms):
    import numpy as np

    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "min": round(float(a.min()), 5), "p90": round(float(np.percentile(a, 90)), 5),
            "n": int(a.size)}


def time_launches(run, reps, between=None):
    """Per-launch times (ms) of run(), each bracketed by its own HIP event
    pair on the current stream (the stream the library launches on).
    between(), if given, runs before each launch outside its event pair."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        if between is not None:
            between()
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def sclk_under_load(run, timeout_s=20.0):
    """The graphics clock (MHz) amd-smi reports while run() keeps the GPU busy:
    amd-smi runs as a child process and the step is repeated until it ends."""
    import subprocess

    import torch

    cmds = [["amd-smi", "metric", "-g", "0", "-c", "--json"],
            ["rocm-smi", "-d", "0", "--showclocks", "--json"]]
    for cmd in cmds:
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                                    text=True)
        except OSError:
            continue
        t0 = time.perf_counter()
        while proc.poll() is None and time.perf_counter() - t0 < timeout_s:
            for _ in range(4):
                run()
            torch.cuda.synchronize()
        try:
            out, _ = proc.communicate(timeout=max(1.0, timeout_s - (time.perf_counter() - t0)))
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.communicate()
            continue
        mhz = _parse_sclk(out)
        if mhz:
            return {"mhz_mean": round(sum(mhz) / len(mhz), 1), "mhz_min": min(mhz),
                    "mhz_max": max(mhz), "readings": len(mhz), "tool": cmd[0]}
    return None


def _parse_sclk(text):
    """Graphics-clock readings (MHz) in amd-smi / rocm-smi JSON output (amd-smi
    gives one per XCD)."""
    import re

    try:
        data = json.loads(text)
    except ValueError:
        return None
    found = []

    def walk(x, path):
        if isinstance(x, dict):
            for k, v in x.items():
                walk(v, path + [str(k).lower()])
        elif isinstance(x, list):
            for v in x:
                walk(v, path)
        else:
            p = "/".join(path)
            gfx = re.search(r"gfx_\d+/clk(/value)?$", p) or re.search(r"sclk clock speed", p)
            if gfx:
                m = re.search(r"(\d+(\.\d+)?)", str(x))
                if m:
                    found.append(float(m.group(1)))

    walk(data, [])
    return found or None


def time_prefill_cfg(name, dev, reps=50, cold=False):
    """One prefill workload: per-launch HIP-event times and algorithmic
    TFLOP/s against the bf16/fp16 MFMA peak (and, for the HBM-side encoder,
    against min(MFMA, arithmetic intensity x HBM bandwidth))."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd

    cfg = W.PREFILL[name]
    q, k, v = (t.to(dev) for t in W.prefill_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.L), dtype=torch.float32, device=dev)
    sc = float(np.float32(cfg.scale))
    run = lambda: flash_attn_fwd(q, k, v, softmax_scale=sc, causal=cfg.causal, out=o, lse=lse)
    between = None
    if cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        between = lambda: flush.fill_(1)
    settle(run)
    st = ms_stats(time_launches(run, reps, between))
    ms = st["mean"]
    tf = cfg.flops() / (ms * 1e-3) / 1e12
    ai = cfg.flops() / cfg.hbm_bytes()
    roof = min(PEAK_MFMA_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
    res = {"workload": f"{name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} L={cfg.L} D={cfg.D} "
                       f"{str(cfg.dtype)[6:]} {'causal' if cfg.causal else 'bidirectional'}"
                       + (" (cold: last-level cache flushed between launches)" if cold else ""),
           "ms": st, "alg_flops_per_launch": cfg.flops(), "alg_bytes_per_launch": cfg.hbm_bytes(),
           "value": round(tf, 3), "unit": "TFLOP/s",
           "roofline": {"bound": "mfma" if roof >= PEAK_MFMA_BF16_TFLOPS else "hbm",
                        "achieved": round(tf, 3), "peak": round(roof, 1), "unit": "TFLOP/s",
                        "frac": round(tf / roof, 4),
                        "frac_of_mfma_peak": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)},
           "kernel": f"fwd_kernel<{str(cfg.dtype)[6:].replace('float16', 'f16')}, {cfg.D}, "
                     f"{str(cfg.causal).lower()}>"}
    if name == "tiny":
        # "us": HIP events around each call from Python, so the host's time to
        # reach the launch is inside; "us_graph": the same call captured
        # GRAPH_LAUNCHES times in one HIP graph and replayed, per launch (the
        # GPU's own time with back-to-back launches)
        res["us"] = {k_: round(v_ * 1e3, 2) for k_, v_ in st.items() if k_ != "n"}
        res["us_graph"] = {k_: round(v_ * 1e3 / GRAPH_LAUNCHES, 2)
                           for k_, v_ in graph_replay_ms(run, GRAPH_LAUNCHES, 20).items()
                           if k_ != "n"}
        res["graph_launches"] = GRAPH_LAUNCHES
    del q, k, v, o, lse
    return res


GRAPH_LAUNCHES = 200


def graph_replay_ms(run, launches, reps):
    """ms_stats of `reps` replays of one HIP graph holding `launches` calls of
    run() (captured on a side stream of default priority, after one eager
    warm-up call there)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            run()
    torch.cuda.synchronize()
    graph.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    st = ms_stats(time_launches(graph.replay, reps))
    del graph
    return st


def _timed_block(run, reps):
    settle(run)
    return ms_stats(time_launches(run, reps))


def time_paged(fmt, dev, reps=20):
    """The decode workload in a paged cache of 16-slot pages (native, int8
    keys, or int8 keys and values): time of fa_decode_paged (split + combine,
    HIP events on the launch stream) and algorithmic GB/s."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import decode_workspace, flash_attn_decode_paged

    cfg = W.DECODE["decode"]
    k8, v8 = PAGED_FORMATS[fmt]
    q, kp, vp, ks, vs, table, lens = W.paged_decode_inputs(cfg, PAGE_SIZE, k_int8=k8, v_int8=v8)
    to = lambda t: None if t is None else t.to(dev)
    q, kp, vp, ks, vs, table, lens_d = (to(t) for t in (q, kp, vp, ks, vs, table, lens))
    ws = decode_workspace(cfg.B, cfg.Hq, cfg.D, cfg.num_splits, dev)
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device=dev)
    sc = float(np.float32(cfg.scale))
    run = lambda: flash_attn_decode_paged(q, kp, vp, table, lens_d, k_scales=ks, v_scales=vs,
                                          softmax_scale=sc, num_splits=cfg.num_splits,
                                          workspace=ws, out=o, lse=lse)
    st = _timed_block(run, reps)
    byts = W.paged_decode_bytes(cfg, lens, PAGE_SIZE, k_int8=k8, v_int8=v8)
    gbs = byts / (st["mean"] * 1e-3) / 1e9
    traffic = traffic_for(f"paged:{fmt}", source_digest(["fa_decode.hip", "fa_common.hpp"]))
    return {"workload": f"decode workload in {PAGE_SIZE}-slot pages, keys "
                        f"{'int8' if k8 else 'bf16'}, values {'int8' if v8 else 'bf16'}",
            "ms": st, "alg_bytes_per_step": byts, "value": round(gbs, 2), "unit": "GB/s",
            "tokens_per_s": round(cfg.B / (st["mean"] * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic}}


def time_bwd(dev, reps=10):
    """fa_bwd (prep + dQ + dK/dV kernels) on the Llama-2-7B-shaped causal
    workload, fed by one untimed fa_fwd: time (HIP events on the launch
    stream) and algorithmic TFLOP/s (10*D per allowed pair per query head:
    the S, dP, dV, dQ and dK products)."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import _abi
    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_bwd, flash_attn_fwd

    cfg = W.PREFILL["llama7b"]
    q, k, v = (t.to(dev) for t in W.prefill_inputs(cfg))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 100)).to(
        cfg.dtype).to(dev)
    sc = float(np.float32(cfg.scale))
    o, lse = flash_attn_fwd(q, k, v, softmax_scale=sc, causal=cfg.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((_abi.fa_bwd_workspace_size(cfg.B, cfg.Hq, cfg.L),), dtype=torch.uint8,
                     device=dev)
    run = lambda: flash_attn_bwd(q, k, v, o, lse, do, softmax_scale=sc, causal=cfg.causal, dq=dq,
                                 dk=dk, dv=dv, workspace=ws)
    st = _timed_block(run, reps)
    flops = cfg.flops() // 4 * 10
    tf = flops / (st["mean"] * 1e-3) / 1e12
    # Q, O, dO read and dQ written (query side), K, V read and dK, dV written,
    # lse read: each once
    nq, nk = cfg.B * cfg.L * cfg.Hq * cfg.D * 2, cfg.B * cfg.L * cfg.Hkv * cfg.D * 2
    alg_bytes = 4 * nq + 4 * nk + cfg.B * cfg.Hq * cfg.L * 4
    return {"workload": "llama7b causal backward B=4 Hq=Hkv=32 L=4096 D=128 bf16 (dQ, dK, dV)",
            "ms": st, "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes,
            "value": round(tf, 3), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": traffic_for("bwd", source_digest(["fa_bwd.hip",
                                                                      "fa_common.hpp"]))}}


def time_bwd_varlen(dev, reps=10):
    """fa_bwd_ex on the varlen16 workload (16 causal sequences packed back to
    back, lengths U[256, 4096], Hq=32, Hkv=8, D=128, bf16), fed by one untimed
    packed forward: time (HIP events) and algorithmic TFLOP/s (10*D per
    allowed pair per query head)."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import _abi
    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_varlen, flash_attn_varlen_bwd

    cfg = W.MASKED["varlen16"]
    q, k, v, cu = W.masked_inputs(cfg)
    lens = cfg.lengths()
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 2)).to(cfg.dtype)
    q, k, v, cu, do = (t.to(dev) for t in (q, k, v, cu, do))
    L = max(lens)
    sc = float(np.float32(cfg.scale))
    o, lse = flash_attn_varlen(q, k, v, cu, cu, L, L, softmax_scale=sc, causal=cfg.causal,
                               window=cfg.window)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((_abi.fa_bwd_workspace_size(cfg.nseq, cfg.Hq, L),), dtype=torch.uint8,
                     device=dev)
    run = lambda: flash_attn_varlen_bwd(q, k, v, o, lse, do, cu, cu, L, L, softmax_scale=sc,
                                        causal=cfg.causal, window=cfg.window, dq=dq, dk=dk, dv=dv,
                                        workspace=ws)
    st = _timed_block(run, reps)
    flops = cfg.flops() // 4 * 10
    tf = flops / (st["mean"] * 1e-3) / 1e12
    return {"workload": "varlen16 causal backward: 16 packed sequences U[256,4096], Hq=32 Hkv=8 "
                        "D=128 bf16 (dQ, dK, dV)",
            "ms": st, "alg_flops_per_launch": flops, "value": round(tf, 3), "unit": "TFLOP/s",
            "frac_mfma": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)}


def time_fp8_d256(dev, reps=20):
    """fa_fwd_fp8 at D = 256 on the d256 workload's shape (B=2, Hq=Hkv=16,
    L=4096, causal, e4m3, fp16 O): algorithmic TFLOP/s against the fp8 peak.
    (Two workgroups share each query tile there, so the MFMAs executed are
    1.5x the algorithmic ones.)"""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd_fp8

    cfg = W.PREFILL["d256"]
    q8, k8, vt8, ds = W.fp8_inputs(cfg.B, cfg.L, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.seed)
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    o = torch.empty((cfg.B, cfg.L, cfg.Hq, cfg.D), dtype=torch.float16, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.L), dtype=torch.float32, device=dev)
    sc = float(np.float32(cfg.scale))
    run = lambda: flash_attn_fwd_fp8(q8, k8, vt8, q_descale=ds, k_descale=ds, v_descale=ds,
                                     softmax_scale=sc, causal=True, out_dtype=torch.float16,
                                     out=o, lse=lse)
    st = _timed_block(run, reps)
    tf = cfg.flops() / (st["mean"] * 1e-3) / 1e12
    return {"workload": "d256 shape B=2 Hq=Hkv=16 L=4096 D=256 causal, e4m3 Q/K/V, fp16 O",
            "ms": st, "alg_flops_per_launch": cfg.flops(), "value": round(tf, 3),
            "unit": "TFLOP/s", "frac_fp8": round(tf / PEAK_MFMA_FP8_TFLOPS, 4)}


def time_fp8(dev, reps=20):
    """fa_fwd_fp8 on the Llama-2-7B-shaped causal workload with e4m3 Q, K, V:
    time (HIP events on the launch stream) and algorithmic TFLOP/s (4*D per
    allowed pair per query head) against the fp8 MFMA peak."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd_fp8

    cfg = W.PREFILL["llama7b"]
    q8, k8, vt8, ds = W.fp8_inputs(cfg.B, cfg.L, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.seed)
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    o = torch.empty((cfg.B, cfg.L, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.L), dtype=torch.float32, device=dev)
    sc = float(np.float32(cfg.scale))
    run = lambda: flash_attn_fwd_fp8(q8, k8, vt8, q_descale=ds, k_descale=ds, v_descale=ds,
                                     softmax_scale=sc, causal=True, out=o, lse=lse)
    st = _timed_block(run, reps)
    tf = cfg.flops() / (st["mean"] * 1e-3) / 1e12
    return {"workload": "llama7b causal prefill B=4 Hq=Hkv=32 L=4096 D=128, e4m3 Q/K/V "
                        "(per-tensor descale), bf16 O",
            "ms": st, "alg_flops_per_launch": cfg.flops(), "value": round(tf, 3),
            "unit": "TFLOP/s",
            # Q, K, V one byte per element read once, O (bf16) and lse written once
            "alg_bytes_per_launch": cfg.B * cfg.L * (3 * cfg.Hq * cfg.D + 2 * cfg.Hkv * cfg.D)
            + cfg.B * cfg.Hq * cfg.L * 4,
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_FP8_TFLOPS, 4),
                         "traffic": traffic_for("fp8", source_digest(["fa_fwd_fp8.hip",
                                                                      "fa_common.hpp"]))},
            "kernel": "fwd_fp8_kernel<128, bf16_t, true>"}


def time_mfma_probe(q, dev, reps=10, iters=2048):
    """The matrix cores' rate on the prefill's own data: the benchmark's MFMA
    probe (libfa_probe.so: bf16 32x32x16 MFMAs only, in the forward step's
    chain pattern, two waves per SIMD on every CU) timed with HIP events,
    once with its operands taken from the prefill's Q and once with every
    operand 1.0.  The MFMA rate depends on the operand values, so the first
    figure, not the published peak, is what the forward's MFMA work can reach
    on this data."""
    import torch

    from exact_tiled_attention_fa_amd.probe import mfma_probe

    ones = torch.ones(1 << 24, dtype=torch.bfloat16, device=dev)
    res = {"about": "MFMA-only probe, bf16 32x32x16, 2 waves/SIMD, every CU; operands read "
                    "once from the given buffer"}
    for name, ops in (("prefill_q", q), ("constant_1", ones)):
        out, flops = mfma_probe(ops, iters)
        st = _timed_block(lambda: mfma_probe(ops, iters, out), reps)
        res[name] = {"TFLOP/s": round(flops / (st["mean"] * 1e-3) / 1e12, 1), "ms": st}
    return res


def time_masked(cfg, dev, reps=20):
    """One structured-mask workload: launch times (HIP events on the launch
    stream) and algorithmic TFLOP/s."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd, flash_attn_varlen

    q, k, v, cu = (None if t is None else t.to(dev) for t in W.masked_inputs(cfg))
    sc = float(np.float32(cfg.scale))
    lmax = max(cfg.lengths())
    o = torch.empty_like(q)
    if cfg.packed:
        lse = torch.empty((cfg.Hq, q.shape[0]), dtype=torch.float32, device=dev)
        run = lambda: flash_attn_varlen(q, k, v, cu, cu, lmax, lmax, softmax_scale=sc,
                                        causal=cfg.causal, window=cfg.window, out=o, lse=lse)
    else:
        lse = torch.empty((cfg.nseq, cfg.Hq, lmax), dtype=torch.float32, device=dev)
        run = lambda: flash_attn_fwd(q, k, v, softmax_scale=sc, causal=cfg.causal,
                                     window=cfg.window, out=o, lse=lse)
    st = _timed_block(run, reps)
    tf = cfg.flops() / (st["mean"] * 1e-3) / 1e12
    lens = cfg.lengths()
    traffic = traffic_for(f"masks:{cfg.name}", source_digest(["fa_fwd.hip", "fa_common.hpp"]))
    return {"workload": f"{cfg.nseq} x L={'%d' % lens[0] if cfg.len_lo == cfg.len_hi else 'U[%d,%d]' % (cfg.len_lo, cfg.len_hi)}"
                        f" Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} {str(cfg.dtype)[6:]}"
                        f" causal={cfg.causal} window={tuple(cfg.window)}"
                        f" {'packed' if cfg.packed else 'dense'}",
            "ms": st, "alg_flops_per_launch": cfg.flops(), "value": round(tf, 3),
            "unit": "TFLOP/s", "alg_bytes_per_launch": cfg.hbm_bytes(),
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": traffic},
            "kernel": "fwd_kernel<bf16_t, 128, true>"}


CONFIG_LEGS = [("gqa16k", 20, False), ("d256", 50, False), ("encoder", 50, True),
               ("tiny", 1000, False)]


def main():
    args = parse()
    if args.summarize_pmc:
        t = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.with_copy or 1024,
                          args.pmc_key)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        try:
            with open(TRAFFIC_FILE) as f:
                merged = json.load(f)
        except (OSError, ValueError):
            merged = {}
        merged.update(t)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(merged, f, indent=1)
        print(json.dumps(t))
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(*args.summarize_trace), indent=1))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, args.kernel_match), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.exit("bench.py measures one GPU only: the library has no multi-GPU path "
                 "(run with --gpus 1).")
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import _abi
    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import (decode_workspace, flash_attn_decode,
                                                        flash_attn_fwd)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    info = _abi.fa_info()
    if args.rates:
        from exact_tiled_attention_fa_amd import probe

        g = torch.Generator().manual_seed(5)
        ops = torch.randn((1 << 22,), generator=g).to(torch.bfloat16).to(dev)
        ones = torch.ones((1 << 22,), dtype=torch.bfloat16, device=dev)
        res = {}
        for data, t in (("random_bf16", ops), ("constant_1", ones)):
            for n in (1, 2):
                for vg in (False, True):
                    key = f"{data}/{n}_waves_per_simd/{'archvgpr' if vg else 'accvgpr'}_acc"
                    print(f"# rates: {key}", file=sys.stderr, flush=True)
                    res[key] = probe.rates(t, n, vgpr_acc=vg)
        print(json.dumps({"rates": res, "lib": info}), flush=True)
        return
    do_pf = args.only in (None, "prefill")
    do_dec = args.only in (None, "decode")
    masks = {n: c for n, c in W.MASKED.items() if args.mask in (None, n)}
    paged_fmts = [f for f in PAGED_FORMATS if args.paged_format in (None, f)]

    def finish(res):
        if args.with_copy:
            copy_calibration(args.with_copy, dev)
        res["lib"] = info
        print(json.dumps(res), flush=True)

    if args.only == "config":
        legs = {n: (r, c) for n, r, c in CONFIG_LEGS}
        legs["llama7b"] = (50, False)
        if args.config not in legs:
            sys.exit(f"--only config needs --config in {sorted(legs)}")
        reps, cold = legs[args.config]
        print(f"# prefill workload {args.config}", file=sys.stderr, flush=True)
        return finish({"configs": {args.config: time_prefill_cfg(
            args.config, dev, args.reps or reps, cold)}})
    if args.only == "fp8":
        print("# fp8 forward workload", file=sys.stderr, flush=True)
        res = time_fp8(dev, args.reps or 20)
        res["d256"] = time_fp8_d256(dev, args.reps or 20)
        return finish({"fp8": res})
    if args.only == "bwd":
        print("# backward workload", file=sys.stderr, flush=True)
        res = time_bwd(dev, args.reps or 10) if args.bwd_workload in (None, "llama7b") else {}
        if args.bwd_workload in (None, "varlen16"):
            res["varlen16"] = time_bwd_varlen(dev, args.reps or 10)
        return finish({"backward": res})
    if args.only == "paged":
        print("# paged decode workloads", file=sys.stderr, flush=True)
        return finish({"paged": {f: time_paged(f, dev, args.reps or 20) for f in paged_fmts}})
    if args.only == "masks":
        print("# structured-mask workloads", file=sys.stderr, flush=True)
        return finish({"masks": {n: time_masked(c, dev, args.reps or 20)
                                 for n, c in masks.items()}})

    pcfg = W.PREFILL["llama7b"]
    dcfg = W.DECODE["decode"]
    pscale = float(np.float32(pcfg.scale))
    dscale = float(np.float32(dcfg.scale))
    print(f"# generating inputs ({pcfg.name}, {dcfg.name})", file=sys.stderr, flush=True)
    if do_pf:
        q_c, k_c, v_c = W.prefill_inputs(pcfg)
        q, k, v = q_c.to(dev), k_c.to(dev), v_c.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((pcfg.B, pcfg.Hq, pcfg.L), dtype=torch.float32, device=dev)
    if do_dec:
        dq_c, kc_c, vc_c, lens_c = W.decode_inputs(dcfg)
        dq, kc, vc, lens = dq_c.to(dev), kc_c.to(dev), vc_c.to(dev), lens_c.to(dev)
        do_ = torch.empty_like(dq)
        dlse = torch.empty((dcfg.B, dcfg.Hq), dtype=torch.float32, device=dev)
        ws = decode_workspace(dcfg.B, dcfg.Hq, dcfg.D, dcfg.num_splits, dev)
    torch.cuda.synchronize()

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        if do_pf:
            flash_attn_fwd(q, k, v, softmax_scale=pscale, causal=True, out=o, lse=lse)
        if evs is not None:
            evs[1].record()
        if do_dec:
            flash_attn_decode(dq, kc, vc, lens, softmax_scale=dscale, num_splits=dcfg.num_splits,
                              workspace=ws, out=do_, lse=dlse)
        if evs is not None:
            evs[2].record()

    print(f"# settle {args.settle} s", file=sys.stderr, flush=True)
    settle_steps = settle(step, args.settle) if args.settle > 0 else 0
    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    sclk = None
    if not args.no_sclk:
        print("# graphics clock under the step's load (amd-smi)", file=sys.stderr, flush=True)
        sclk = sclk_under_load(step)

    out = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V; no model weights)",
           "config": {"workload": "llama7b causal prefill B=4 Hq=Hkv=32 L=4096 D=128 bf16 + "
                                  "split-KV decode B=128 Hq=32 Hkv=8 D=128 bf16 len~U[512,8192] "
                                  "8 splits",
                      "prefill": {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "L": pcfg.L,
                                  "D": pcfg.D, "causal": True},
                      "decode": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "D": dcfg.D,
                                 "num_splits": dcfg.num_splits},
                      "lib": info},
           "settle_s": args.settle, "settle_steps": settle_steps, "sclk": sclk}
    if do_pf:
        st = ms_stats(pf_ms)
        tf = pcfg.flops() / (st["mean"] * 1e-3) / 1e12
        out["value"] = round(tf, 3)
        out["prefill_ms"] = st
        out["roofline"] = {"bound": "mfma", "achieved": round(tf, 3),
                           "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                           "traffic": traffic_for("fwd_kernel", source_digest(
                               ["fa_fwd.hip", "fa_common.hpp"])),
                           "kernel": "fwd_kernel<bf16_t, 128, true>",
                           "alg_flops_per_launch": pcfg.flops(),
                           "alg_bytes_per_launch": pcfg.hbm_bytes()}
    if do_dec:
        st = ms_stats(dec_ms)
        byts = W.decode_bytes(dcfg, lens_c)
        gbs = byts / (st["mean"] * 1e-3) / 1e9
        out["decode"] = {"value": round(gbs, 2), "unit": "GB/s", "ms": st,
                         "alg_bytes_per_step": byts,
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 2),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": traffic_for("decode", source_digest(
                                          ["fa_decode.hip", "fa_common.hpp"]))}}
        if out["value"] is None:
            out["value"], out["unit"] = round(gbs, 2), "GB/s"
    if do_pf and not args.no_configs:
        out["configs"] = {}
        for name, reps, cold in CONFIG_LEGS:
            print(f"# prefill workload {name}", file=sys.stderr, flush=True)
            out["configs"][name] = time_prefill_cfg(name, dev, reps, cold)
    if do_dec and not args.no_paged:
        print("# paged decode workloads", file=sys.stderr, flush=True)
        out["decode"]["paged"] = {f: time_paged(f, dev) for f in paged_fmts}
    if do_pf and not args.no_fp8:
        print("# fp8 forward workload", file=sys.stderr, flush=True)
        out["fp8"] = time_fp8(dev)
        out["fp8"]["d256"] = time_fp8_d256(dev)
    if do_pf and not args.no_bwd:
        print("# backward workload", file=sys.stderr, flush=True)
        out["backward"] = time_bwd(dev)
        out["backward"]["varlen16"] = time_bwd_varlen(dev)
    if do_pf and not args.no_masks:
        print("# structured-mask workloads", file=sys.stderr, flush=True)
        out["masks"] = {name: time_masked(cfg, dev) for name, cfg in masks.items()}
    if do_pf and args.probe:
        print("# matrix-core probe", file=sys.stderr, flush=True)
        out["mfma_probe"] = time_mfma_probe(q, dev)
        out["mfma_probe"]["prefill_frac_of_prefill_q_rate"] = round(
            out["value"] / out["mfma_probe"]["prefill_q"]["TFLOP/s"], 4)
    if args.with_copy:
        copy_calibration(args.with_copy, dev)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        if do_pf:
            out["cpu_baseline"] = cpu_baseline_prefill(pcfg, q_c, k_c, v_c, pscale, args.cpu_seconds)
        if do_dec:
            out.setdefault("decode", {})["cpu_baseline"] = cpu_baseline_decode(
                dcfg, dq_c, kc_c, vc_c, lens_c, dscale)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
