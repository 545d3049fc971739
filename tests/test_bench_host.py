"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the timing
statistics, the counter calibration (FETCH_SIZE / WRITE_SIZE scaled by what
they read for a device copy of known size), the trace summary's choice of
the timed dispatches, and the tie of counter records to the kernel sources."""

from __future__ import annotations

import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr, r.stderr


def test_ms_stats(bench):
    st = bench.ms_stats([1.0, 2.0, 3.0, 4.0, 10.0])
    assert st["mean"] == 4.0 and st["median"] == 3.0 and st["min"] == 1.0 and st["n"] == 5
    assert st["p90"] == pytest.approx(7.6)  # linear interpolation between 4 and 10


def _counter_run(d, counter, per_kernel):
    rows = []
    disp = 0
    for name, values in per_kernel:
        for v in values:
            disp += 1
            rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": v})
    _write_csv(os.path.join(d, "run_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_summarize_pmc_calibration(bench, tmp_path):
    """A 1024 MiB copy whose FETCH_SIZE reads half its bytes gives a fetch
    factor of 2 and a write factor of 1; the kernel's bytes per launch are
    then 1024 * (2 * fetch + write) from the medians over its dispatches (a
    small upload copy is ignored)."""
    copy = "__amd_rocclr_copyBuffer"
    fwd = "void fa::fwd_kernel<fa::bf16_t, 128, true>(FwdParams)"
    dec_s = "void fa::decode_split_kernel<fa::bf16_t, 128, false, false, false>(SplitParams)"
    dec_c = "void fa::decode_combine_kernel<fa::bf16_t, 128>(float const*)"
    fdir, wdir = str(tmp_path / "f"), str(tmp_path / "w")
    _counter_run(fdir, "FETCH_SIZE", [(copy, [3.0]), (fwd, [100.0, 110.0, 90.0]),
                                      (dec_s, [50.0, 50.0]), (dec_c, [5.0, 5.0]),
                                      (copy, [524288.0])])
    _counter_run(wdir, "WRITE_SIZE", [(copy, [3.0]), (fwd, [40.0, 40.0, 40.0]),
                                      (dec_s, [10.0, 10.0]), (dec_c, [1.0, 1.0]),
                                      (copy, [1048576.0])])
    out = bench.summarize_pmc(fdir, wdir, 1024)
    assert out["fetch_factor"] == 2.0 and out["write_factor"] == 1.0
    assert out["fwd_kernel"]["bytes_per_launch"] == int((100.0 * 2 + 40.0) * 1024)
    assert out["decode"]["bytes_per_launch"] == int(((50 + 5) * 2 + (10 + 1)) * 1024)
    assert out["fwd_kernel"]["source_digest"] == bench.source_digest(["fa_fwd.hip"])


def test_traffic_record_follows_the_sources(bench, tmp_path, monkeypatch):
    digest = bench.source_digest(["fa_fwd.hip", "fa_common.hpp"])
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"fwd_kernel": {"source_digest": digest, "bytes_per_launch": 7}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_for("fwd_kernel", digest) == 7
    assert bench.traffic_for("fwd_kernel", "0" * 16) is None  # taken on other sources
    assert bench.traffic_for("decode", digest) is None


def test_digest_covers_the_shared_headers(bench, tmp_path, monkeypatch):
    """A change to a header every kernel includes (here the LDS layouts)
    changes every kernel's digest, so old counter records go stale."""
    import shutil
    src = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, src, ignore=shutil.ignore_patterns("probe"))
    monkeypatch.setattr(bench, "CSRC", str(src))
    before = {k: bench.source_digest([k]) for k in ("fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip")}
    with open(src / "fa_lds.hpp", "a") as f:
        f.write("\n// changed\n")
    after = {k: bench.source_digest([k]) for k in before}
    assert all(before[k] != after[k] for k in before)


def test_summarize_trace_takes_the_timed_steps(bench, tmp_path):
    """The step's prefill dispatches are settle_steps + warmup untimed ones,
    then the timed ones; other kernels in between do not shift the count."""
    fwd = "void fa::fwd_kernel<fa::bf16_t, 128, true>(FwdParams)"
    other = "void fa::decode_split_kernel<fa::bf16_t, 128, false, false, false>(SplitParams)"
    settle, warmup, steps = 3, 2, 4
    rows, t = [], 0
    for i in range(settle + warmup + steps + 3):  # 3 more after the timed ones
        dur = 500_000 if settle + warmup <= i < settle + warmup + steps else 900_000
        rows.append({"Kernel_Name": fwd, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 10
        rows.append({"Kernel_Name": other, "Start_Timestamp": t, "End_Timestamp": t + 300_000})
        t += 300_010
    d = tmp_path / "trace"
    _write_csv(str(d / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               rows)
    _write_csv(str(d / "run_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [{"Name": fwd, "Calls": 12, "AverageNs": 1, "MinNs": 1, "MaxNs": 1, "Percentage": 1}])
    line = {"settle_steps": settle, "warmup": warmup, "steps": steps, "value": 1.0,
            "prefill_ms": {"mean": 0.5}, "roofline": {"frac": 0.1, "alg_flops_per_launch": 5e11}}
    bj = tmp_path / "bench.json"
    bj.write_text("# a progress line\n" + json.dumps(line) + "\n")
    out = bench.summarize_trace(str(d), str(bj))
    assert out["timed_dispatches"] == steps and out["first_timed_dispatch"] == settle + warmup
    assert out["trace_timed_prefill_us_mean"] == 500.0
    assert out["trace_timed_prefill_tflops"] == pytest.approx(5e11 / 500e-6 / 1e12, rel=1e-3)
