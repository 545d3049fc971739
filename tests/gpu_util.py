"""Shared pieces of the GPU parity tests: tolerances, comparison, printing."""

from __future__ import annotations

import sys

import numpy as np
import torch

# Acceptance bounds for 16-bit inputs/outputs with fp32 accumulation.
O_TOL = 2e-2
LSE_TOL = 1e-3


def f32(x: float) -> float:
    """The float32 value that crosses the C ABI as `float scale`."""
    return float(np.float32(x))


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what, *, o_tol=O_TOL, lse_tol=LSE_TOL, mask=None):
    """Element-wise comparison; returns (max|dO|, max|dlse|).  ``mask`` selects
    which entries of o_ref/lse_ref were computed (the rest are NaN)."""
    og = to64(o_gpu)
    lg = to64(lse_gpu)
    o_ref = np.asarray(o_ref)
    lse_ref = np.asarray(lse_ref)
    osel = ~np.isnan(o_ref)
    lsel = ~np.isnan(lse_ref)
    assert osel.any() and lsel.any(), f"{what}: nothing to compare"
    assert np.all(np.isfinite(og[osel])), f"{what}: non-finite GPU output"
    # rows with no visible key: exact zeros and -inf
    linf = lsel & np.isinf(lse_ref)
    assert np.array_equal(lg[linf], lse_ref[linf]), f"{what}: empty-row lse differs"
    lfin = lsel & ~np.isinf(lse_ref)
    do = float(np.max(np.abs(og[osel] - o_ref[osel])))
    dl = float(np.max(np.abs(lg[lfin] - lse_ref[lfin]))) if lfin.any() else 0.0
    mean_o = float(np.mean(np.abs(og[osel] - o_ref[osel])))
    dtype = o_gpu.dtype
    floor = float(np.max(np.abs(
        torch.from_numpy(o_ref[osel]).to(dtype).to(torch.float64).numpy() - o_ref[osel])))
    say(f"  {what}: max|dO|={do:.3e} (floor {floor:.3e}, mean {mean_o:.2e})  max|dlse|={dl:.3e}")
    assert do <= o_tol, f"{what}: max|dO| {do:.3e} > {o_tol}"
    assert dl <= lse_tol, f"{what}: max|dlse| {dl:.3e} > {lse_tol}"
    return do, dl
