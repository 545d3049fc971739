"""The kernels' integer scheduling, checked on the host: tests/sched_check.cpp
compiles the same header the kernels use (csrc/fa_sched.hpp) with g++ and
checks that every workgroup grid maps one-to-one onto its work items and that
the prefill kernel's tile walk copies only whole in-range tiles without
clamping and forms each visible tile exactly once per wave, and that the
split waves' score exchange (D = 256) always completes a tile's scores from
the partial stored for that tile in the step before."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "exact_tiled_attention_fa_amd", "csrc")


def _build(tmp_path, src, extra=()):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "sched_check"
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", *extra, f"-I{CSRC}",
                    os.path.join(HERE, src), "-o", str(exe)], check=True)
    return exe


def test_scheduling(tmp_path):
    exe = _build(tmp_path, "sched_check.cpp")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr


def test_walk_check_catches_the_unclamped_overrun(tmp_path):
    """The walk replay fails on the main-phase condition without the key-range
    term (the last step of a group would copy a K tile past the keys, e.g.
    non-causal Lk = 96), so it does check what it claims."""
    src = open(os.path.join(CSRC, "fa_sched.hpp")).read()
    cond = "t >= m_lo && t + NS < m_hi && (t_first + t + 2 * NS) * BN <= Lk"
    assert cond in src
    bad_dir = tmp_path / "bad"
    bad_dir.mkdir()
    (bad_dir / "fa_sched.hpp").write_text(src.replace(cond, "t >= m_lo && t + NS < m_hi"))
    exe = _build(tmp_path, "sched_check.cpp", extra=(f"-I{bad_dir}",))
    # the mutated header shadows the real one (first -I wins for "fa_sched.hpp")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode != 0 and "main step" in res.stdout, res.stdout
