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

The structured-mask prefill workloads (sliding window ``swa16k``, packed
sequences ``varlen16``) are timed after the step loop, with HIP events around
each launch, and reported under ``masks`` in the same line; they are not part
of ``value``.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--with-copy MIB] [--only prefill|decode] [--no-masks]
                    [--all-configs]
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
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU oracle sample")
    p.add_argument("--with-copy", type=int, default=0, metavar="MIB",
                   help="after timing, run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--only", choices=["prefill", "decode", "masks", "paged", "bwd", "fp8"],
                   default=None,
                   help="masks / paged / bwd: time only the structured-mask prefill, the paged "
                        "decode or the backward workloads (one JSON line)")
    p.add_argument("--no-bwd", action="store_true", help="skip the backward workload")
    p.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward workload")
    p.add_argument("--no-probe", action="store_true",
                   help="skip the matrix-core ceiling probe on the prefill's operands")
    p.add_argument("--paged-format", choices=["native", "k8", "kv8"], default=None,
                   help="time only this paged-cache format")
    p.add_argument("--no-paged", action="store_true",
                   help="skip the paged-cache decode workloads")
    p.add_argument("--mask", default=None, help="time only this structured-mask workload")
    p.add_argument("--no-masks", action="store_true",
                   help="skip the structured-mask prefill workloads (sliding window, packed)")
    p.add_argument("--all-configs", action="store_true",
                   help="also print one extra JSON line per prefill workload")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs of this script with "
                        "--with-copy (FETCH_SIZE, then WRITE_SIZE) into profiles/traffic.json")
    p.add_argument("--pmc-key", default=None,
                   help="with --summarize-pmc on a run of --only masks --mask NAME: record the "
                        "forward kernel's traffic under this key (e.g. masks:NAME)")
    return p.parse_args()


def source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
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


def cpu_baseline_prefill(cfg, q, k, v, scale, target_s):
    """Time the fp64 oracle on a bounded sample of whole (batch, head) slices."""
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
            "cores": workers, "kind": "oracle",
            "sample": f"{n} of {len(pairs)} (batch, head) slices of the same workload, "
                      f"fp64 numpy, {dt:.2f} s wall"}


def cpu_baseline_decode(cfg, q, kc, vc, lens, scale, nseq=16):
    import oracle
    from exact_tiled_attention_fa_amd import workloads as W

    from threadpoolctl import threadpool_limits

    heads = [(b, h) for b in range(nseq) for h in range(cfg.Hq)]
    with threadpool_limits(limits=1):  # the oracle's decode is one thread; so is its BLAS
        t0 = time.perf_counter()
        oracle.decode_ref(q, kc, vc, lens, scale, heads=heads)
        dt = time.perf_counter() - t0
    sub = lens[:nseq]
    byts = int(sum(int(x) for x in sub)) * cfg.Hkv * cfg.D * 2 * 2 + nseq * cfg.Hq * (2 * cfg.D * 2 + 4)
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nseq} of {cfg.B} sequences, all heads, fp64 numpy, {dt:.2f} s wall"}


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
    ~100 ms of work after idle run 10-20 % slow)."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            run()
        torch.cuda.synchronize()


def time_paged(fmt, dev, reps=10):
    """The decode workload in a paged cache of 16-slot pages (native, int8
    keys, or int8 keys and values): mean time of fa_decode_paged (split +
    combine, HIP events on the launch stream) and algorithmic GB/s."""
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
    settle(run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    mean = float(np.mean(ms))
    byts = W.paged_decode_bytes(cfg, lens, PAGE_SIZE, k_int8=k8, v_int8=v8)
    gbs = byts / (mean * 1e-3) / 1e9
    traffic = traffic_for(f"paged:{fmt}", source_digest(["fa_decode.hip", "fa_common.hpp"]))
    return {"workload": f"decode workload in {PAGE_SIZE}-slot pages, keys "
                        f"{'int8' if k8 else 'bf16'}, values {'int8' if v8 else 'bf16'}",
            "ms": {"mean": round(mean, 5), "median": round(float(np.median(ms)), 5),
                   "min": round(float(np.min(ms)), 5)},
            "alg_bytes_per_step": byts, "value": round(gbs, 2), "unit": "GB/s",
            "tokens_per_s": round(cfg.B / (mean * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic}}


def time_bwd(dev, reps=10):
    """fa_bwd (prep + dQ + dK/dV kernels) on the Llama-2-7B-shaped causal
    workload, fed by one untimed fa_fwd: mean time (HIP events on the launch
    stream) and algorithmic TFLOP/s (10*D per allowed pair per query head:
    the S, dP, dV, dQ and dK products)."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd import workloads as W
    from exact_tiled_attention_fa_amd.attention import flash_attn_bwd, flash_attn_fwd

    cfg = W.PREFILL["llama7b"]
    q, k, v = (t.to(dev) for t in W.prefill_inputs(cfg))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 100)).to(
        cfg.dtype).to(dev)
    sc = float(np.float32(cfg.scale))
    o, lse = flash_attn_fwd(q, k, v, softmax_scale=sc, causal=cfg.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    from exact_tiled_attention_fa_amd import _abi
    ws = torch.empty((_abi.fa_bwd_workspace_size(cfg.B, cfg.Hq, cfg.L),), dtype=torch.uint8,
                     device=dev)
    run = lambda: flash_attn_bwd(q, k, v, o, lse, do, softmax_scale=sc, causal=cfg.causal, dq=dq,
                                 dk=dk, dv=dv, workspace=ws)
    settle(run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    mean = float(np.mean(ms))
    flops = cfg.flops() // 4 * 10
    tf = flops / (mean * 1e-3) / 1e12
    # Q, O, dO read and dQ written (query side), K, V read and dK, dV written,
    # lse read: each once
    nq, nk = cfg.B * cfg.L * cfg.Hq * cfg.D * 2, cfg.B * cfg.L * cfg.Hkv * cfg.D * 2
    alg_bytes = 4 * nq + 4 * nk + cfg.B * cfg.Hq * cfg.L * 4
    return {"workload": "llama7b causal backward B=4 Hq=Hkv=32 L=4096 D=128 bf16 (dQ, dK, dV)",
            "ms": {"mean": round(mean, 5), "median": round(float(np.median(ms)), 5),
                   "min": round(float(np.min(ms)), 5)},
            "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes,
            "value": round(tf, 3), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": traffic_for("bwd", source_digest(["fa_bwd.hip",
                                                                      "fa_common.hpp"]))}}


def time_bwd_varlen(dev, reps=10):
    """fa_bwd_ex on the varlen16 workload (16 causal sequences packed back to
    back, lengths U[256, 4096], Hq=32, Hkv=8, D=128, bf16), fed by one untimed
    packed forward: mean time (HIP events) and algorithmic TFLOP/s (10*D per
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
    settle(run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    mean = float(np.mean(ms))
    flops = cfg.flops() // 4 * 10
    tf = flops / (mean * 1e-3) / 1e12
    return {"workload": "varlen16 causal backward: 16 packed sequences U[256,4096], Hq=32 Hkv=8 "
                        "D=128 bf16 (dQ, dK, dV)",
            "ms": {"mean": round(mean, 5), "median": round(float(np.median(ms)), 5),
                   "min": round(float(np.min(ms)), 5)},
            "alg_flops_per_launch": flops, "value": round(tf, 3), "unit": "TFLOP/s",
            "frac_mfma": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)}


def time_fp8(dev, reps=10):
    """fa_fwd_fp8 on the Llama-2-7B-shaped causal workload with e4m3 Q, K, V:
    mean time (HIP events on the launch stream) and algorithmic TFLOP/s
    (4*D per allowed pair per query head) against the fp8 MFMA peak."""
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
    settle(run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    mean = float(np.mean(ms))
    tf = cfg.flops() / (mean * 1e-3) / 1e12
    return {"workload": "llama7b causal prefill B=4 Hq=Hkv=32 L=4096 D=128, e4m3 Q/K/V "
                        "(per-tensor descale), bf16 O",
            "ms": {"mean": round(mean, 5), "median": round(float(np.median(ms)), 5),
                   "min": round(float(np.min(ms)), 5)},
            "alg_flops_per_launch": cfg.flops(), "value": round(tf, 3), "unit": "TFLOP/s",
            # Q, K, V one byte per element read once, O (bf16) and lse written once
            "alg_bytes_per_launch": cfg.B * cfg.L * (3 * cfg.Hq * cfg.D + 2 * cfg.Hkv * cfg.D)
            + cfg.B * cfg.Hq * cfg.L * 4,
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_FP8_TFLOPS, 4),
                         "traffic": traffic_for("fp8", source_digest(["fa_fwd_fp8.hip",
                                                                      "fa_common.hpp"]))},
            "kernel": "fwd_fp8_kernel<128, bf16_t, true>"}


def time_mfma_probe(q, dev, reps=10, iters=2048):
    """The matrix cores' ceiling on the prefill's own data: the library's MFMA
    probe (bf16 32x32x16 MFMAs only, in the forward step's chain pattern, two
    waves per SIMD on every CU) timed with HIP events on the launch stream,
    once with its operands taken from the prefill's Q and once with every
    operand 1.0.  The MFMA rate depends on the operand values, so the first
    figure, not the published peak, is what the forward's MFMA work can reach
    on this data."""
    import numpy as np
    import torch

    from exact_tiled_attention_fa_amd.attention import mfma_probe

    ones = torch.ones(1 << 24, dtype=torch.bfloat16, device=dev)
    res = {"about": "MFMA-only probe, bf16 32x32x16, 2 waves/SIMD, every CU; operands read "
                    "once from the given buffer"}
    for name, ops in (("prefill_q", q), ("constant_1", ones)):
        out, flops = mfma_probe(ops, iters)
        settle(lambda: mfma_probe(ops, iters, out))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            mfma_probe(ops, iters, out)
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        res[name] = {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4)}
    return res


def time_masked(cfg, dev, reps=10):
    """Mean launch time (ms, HIP events on the launch stream) of one
    structured-mask workload, and its algorithmic TFLOP/s."""
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
    settle(run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    mean = float(np.mean(ms))
    tf = cfg.flops() / (mean * 1e-3) / 1e12
    lens = cfg.lengths()
    traffic = traffic_for(f"masks:{cfg.name}", source_digest(["fa_fwd.hip", "fa_common.hpp"]))
    return {"workload": f"{cfg.nseq} x L={'%d' % lens[0] if cfg.len_lo == cfg.len_hi else 'U[%d,%d]' % (cfg.len_lo, cfg.len_hi)}"
                        f" Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} {str(cfg.dtype)[6:]}"
                        f" causal={cfg.causal} window={tuple(cfg.window)}"
                        f" {'packed' if cfg.packed else 'dense'}",
            "ms": {"mean": round(mean, 5), "median": round(float(np.median(ms)), 5),
                   "min": round(float(np.min(ms)), 5)},
            "alg_flops_per_launch": cfg.flops(), "value": round(tf, 3), "unit": "TFLOP/s",
            "alg_bytes_per_launch": cfg.hbm_bytes(),
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": traffic},
            "kernel": "fwd_kernel<bf16_t, 128, true>"}


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
    do_pf = args.only in (None, "prefill")
    do_dec = args.only in (None, "decode")
    masks = {n: c for n, c in W.MASKED.items() if args.mask in (None, n)}
    paged_fmts = [f for f in PAGED_FORMATS if args.paged_format in (None, f)]
    if args.only == "fp8":
        print("# fp8 forward workload", file=sys.stderr, flush=True)
        res = time_fp8(dev)
        if args.with_copy:
            copy_calibration(args.with_copy, dev)
        print(json.dumps({"fp8": res, "lib": info}), flush=True)
        return
    if args.only == "bwd":
        print("# backward workload", file=sys.stderr, flush=True)
        res = time_bwd(dev)
        if args.with_copy:
            copy_calibration(args.with_copy, dev)
        print(json.dumps({"backward": res, "lib": info}), flush=True)
        return
    if args.only == "paged":
        print("# paged decode workloads", file=sys.stderr, flush=True)
        res = {f: time_paged(f, dev) for f in paged_fmts}
        if args.with_copy:
            copy_calibration(args.with_copy, dev)
        print(json.dumps({"paged": res, "lib": info}), flush=True)
        return
    if args.only == "masks":
        print("# structured-mask workloads", file=sys.stderr, flush=True)
        res = {n: time_masked(c, dev) for n, c in masks.items()}
        if args.with_copy:
            copy_calibration(args.with_copy, dev)
        print(json.dumps({"masks": res, "lib": info}), flush=True)
        return

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

    if args.with_copy:
        copy_calibration(args.with_copy, dev)

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
                      "lib": info}}
    if do_pf:
        ms = float(np.mean(pf_ms))
        tf = pcfg.flops() / (ms * 1e-3) / 1e12
        out["value"] = round(tf, 3)
        out["prefill_ms"] = {"mean": round(ms, 5), "median": round(float(np.median(pf_ms)), 5),
                             "min": round(float(np.min(pf_ms)), 5)}
        out["roofline"] = {"bound": "mfma", "achieved": round(tf, 3),
                           "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                           "traffic": traffic_for("fwd_kernel", source_digest(
                               ["fa_fwd.hip", "fa_common.hpp"])),
                           "kernel": "fwd_kernel<bf16_t, 128, true>",
                           "alg_flops_per_launch": pcfg.flops()}
    if do_dec:
        dms = float(np.mean(dec_ms))
        byts = W.decode_bytes(dcfg, lens_c)
        gbs = byts / (dms * 1e-3) / 1e9
        out["decode"] = {"value": round(gbs, 2), "unit": "GB/s",
                         "ms": {"mean": round(dms, 5), "median": round(float(np.median(dec_ms)), 5),
                                "min": round(float(np.min(dec_ms)), 5)},
                         "alg_bytes_per_step": byts,
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 2),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": traffic_for("decode", source_digest(
                                          ["fa_decode.hip", "fa_common.hpp"]))}}
        if out["value"] is None:
            out["value"], out["unit"] = round(gbs, 2), "GB/s"
    if do_dec and not args.no_paged:
        print("# paged decode workloads", file=sys.stderr, flush=True)
        out["decode"]["paged"] = {f: time_paged(f, dev) for f in paged_fmts}
    if do_pf and not args.no_fp8:
        print("# fp8 forward workload", file=sys.stderr, flush=True)
        out["fp8"] = time_fp8(dev)
    if do_pf and not args.no_bwd:
        print("# backward workload", file=sys.stderr, flush=True)
        out["backward"] = time_bwd(dev)
        out["backward"]["varlen16"] = time_bwd_varlen(dev)
    if do_pf and not args.no_masks:
        print("# structured-mask workloads", file=sys.stderr, flush=True)
        out["masks"] = {name: time_masked(cfg, dev) for name, cfg in masks.items()}
    if do_pf and not args.no_probe:
        print("# matrix-core ceiling probe", file=sys.stderr, flush=True)
        out["mfma_probe"] = time_mfma_probe(q, dev)
        out["mfma_probe"]["prefill_frac_of_prefill_q_ceiling"] = round(
            out["value"] / out["mfma_probe"]["prefill_q"]["TFLOP/s"], 4)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        if do_pf:
            out["cpu_baseline"] = cpu_baseline_prefill(pcfg, q_c, k_c, v_c, pscale, args.cpu_seconds)
        if do_dec:
            out.setdefault("decode", {})["cpu_baseline"] = cpu_baseline_decode(
                dcfg, dq_c, kc_c, vc_c, lens_c, dscale)
    print(json.dumps(out), flush=True)

    if args.all_configs:
        for name, cfg in W.PREFILL.items():
            qq, kk, vv = (t.to(dev) for t in W.prefill_inputs(cfg))
            sc = float(np.float32(cfg.scale))
            settle(lambda: flash_attn_fwd(qq, kk, vv, softmax_scale=sc, causal=cfg.causal))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 20
            e0.record()
            for _ in range(reps):
                flash_attn_fwd(qq, kk, vv, softmax_scale=sc, causal=cfg.causal)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = cfg.flops() / (ms * 1e-3) / 1e12
            print(json.dumps({"workload": name, "ms": round(ms, 5), "TFLOP/s": round(tf, 2),
                              "frac_mfma": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                              "GB/s": round(cfg.hbm_bytes() / (ms * 1e-3) / 1e9, 1)}), flush=True)
            del qq, kk, vv


if __name__ == "__main__":
    main()
