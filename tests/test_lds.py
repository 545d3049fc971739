"""The kernels' LDS layouts, checked on the host: tests/lds_check.cpp compiles
the header the kernels take their tile XORs from (csrc/fa_lds.hpp) with g++,
replays every tile access of the decode, backward and FP8 kernels lane by
lane, and checks them free of bank conflicts in the header's bank model and
each XOR one-to-one on its row's chunks."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "exact_tiled_attention_fa_amd", "csrc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    out = tmp_path_factory.mktemp("lds") / "lds_check"
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", f"-I{CSRC}",
                    os.path.join(HERE, "lds_check.cpp"), "-o", str(out)], check=True)
    return out


def test_lds_layouts(exe):
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr


def test_lds_check_catches_the_old_layouts(exe):
    """The XORs the kernels used before (row index masks) met 2- to 16-way
    conflicts in this model; the replay must report them."""
    res = subprocess.run([str(exe), "old"], capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and "conflicts" in res.stdout, res.stdout
    for where in ("decode D=128 K8 V8: K read", "decode D=128 K8 V8: V store",
                  "merge store", "bwd D=128: transpose read", "fp8 D=128: K read",
                  "fp8 D=128: V read"):
        assert where in res.stdout, where
