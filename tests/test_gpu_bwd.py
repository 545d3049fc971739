"""Backward parity: libfa's fa_bwd (through the C ABI), fed by libfa's forward,
against the exact gradients of the fp64 oracle.

Error bound (per element, derived from the arithmetic): the kernel's P comes
from the forward's lse (|error| <= 1e-3, the forward's parity bound) and is
rounded to the 16-bit type for the MFMA; dS is rounded likewise; D_i = dO_i.O_i
uses the forward's 16-bit O (relative error ~2u); outputs are rounded once.
With u the unit roundoff of the type (bf16 2^-8, fp16 2^-11) each gradient is
off by at most about (4u + 2e-3) times the oracle's per-element magnitude sum
(sum of |terms|, plus the sensitivity of dS to D) plus u times its own size.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import f32, say, to64

pytestmark = pytest.mark.gpu

UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def compare_grad(got, ref, mag, dtype, what):
    g = to64(got)
    ref = np.asarray(ref)
    sel = ~np.isnan(ref)
    assert sel.any(), f"{what}: nothing to compare"
    assert np.all(np.isfinite(g[sel])), f"{what}: non-finite GPU gradient"
    u = UNIT[dtype]
    tol = (4 * u + 2e-3) * np.asarray(mag)[sel] + u * np.abs(ref[sel]) + 1e-6
    err = np.abs(g[sel] - ref[sel])
    ratio = float(np.max(err / tol))
    say(f"  {what}: max|d|={err.max():.3e} max|ref|={np.abs(ref[sel]).max():.3e} "
        f"worst err/bound={ratio:.3f}")
    assert ratio <= 1.0, f"{what}: error exceeds the bound by {ratio:.2f}x"


def run_bwd(q, k, v, do, scale, causal, window, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_bwd, flash_attn_fwd

    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = flash_attn_fwd(q, k, v, softmax_scale=scale, causal=causal, window=window)
    dq, dk, dv = flash_attn_bwd(q, k, v, o, lse, do, softmax_scale=scale, causal=causal,
                                window=window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(B, Lq, Lk, Hq, Hkv, D, dtype, causal, seed, gpu, scale=None, window=(-1, -1),
          q_scale=1.0, kv_heads=None):
    scale = f32(scale if scale is not None else D ** -0.5)
    q, k, v = W.randn_qkv(B, Lq, Lk, Hq, Hkv, D, dtype, seed, q_scale=q_scale)
    gen = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=gen).to(dtype)
    tag = (f"bwd B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} D={D} {str(dtype)[6:]} "
           f"causal={causal} window={window} s={scale:.4g}")
    say(tag)
    dq, dk, dv = run_bwd(q, k, v, do, scale, causal, window, gpu)
    r = oracle.attention_bwd_ref(q, k, v, do, scale, causal, window=window, bounds=True,
                                 kv_heads=kv_heads)
    compare_grad(dq, r[0], r[3], dtype, "dq")
    compare_grad(dk, r[1], r[4], dtype, "dk")
    compare_grad(dv, r[2], r[5], dtype, "dv")


RAGGED = [(1, 1), (17, 17), (64, 64), (65, 65), (129, 129), (300, 300), (65, 200), (200, 65),
          (129, 400)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lq,Lk", RAGGED, ids=[f"{a}x{b}" for a, b in RAGGED])
def test_bwd_ragged(Lq, Lk, D, dtype, causal, gpu):
    check(1, Lq, Lk, 4, 2, D, dtype, causal, seed=Lq * 31 + Lk + D, gpu=gpu)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_bwd_gqa_groups(g, gpu):
    check(2, 257, 257, 8, 8 // g, 128, torch.bfloat16, True, seed=41 * g, gpu=gpu)


WINDOWS = [(0, 0), (5, 3), (64, -1), (-1, 40)]


@pytest.mark.parametrize("window", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_windows(window, causal, gpu):
    check(1, 300, 300, 4, 2, 64, torch.bfloat16, causal, seed=7 + window[0], gpu=gpu,
          window=window)


def test_bwd_d256_gqa_window(gpu):
    check(2, 200, 333, 8, 2, 256, torch.float16, True, seed=81, gpu=gpu)
    check(1, 300, 300, 4, 1, 256, torch.bfloat16, False, seed=82, gpu=gpu, window=(40, 9))


def test_bwd_d256_full_size(gpu):
    """The d256 workload (B=2, H=16, L=4096, D=256, fp16, causal); the oracle
    computes every head's gradients."""
    cfg = W.PREFILL["d256"]
    q, k, v = W.prefill_inputs(cfg)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 100)).to(cfg.dtype)
    scale = f32(cfg.scale)
    say("bwd full-size d256")
    dq, dk, dv = run_bwd(q, k, v, do, scale, True, (-1, -1), gpu)
    r = oracle.attention_bwd_ref(q, k, v, do, scale, True, bounds=True, workers=16)
    compare_grad(dq, r[0], r[3], cfg.dtype, "dq all heads")
    compare_grad(dk, r[1], r[4], cfg.dtype, "dk all heads")
    compare_grad(dv, r[2], r[5], cfg.dtype, "dv all heads")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_bwd_scales(scale, gpu):
    check(1, 130, 130, 2, 1, 128, torch.bfloat16, True, seed=13, gpu=gpu, scale=scale)


def test_bwd_large_logits(gpu):
    check(1, 300, 300, 2, 2, 64, torch.float16, False, seed=14, gpu=gpu, q_scale=4.0)
    check(1, 300, 300, 2, 2, 128, torch.bfloat16, True, seed=15, gpu=gpu, q_scale=4.0)


def test_bwd_deterministic(gpu):
    q, k, v = W.randn_qkv(2, 1000, 1000, 8, 2, 128, torch.bfloat16, 16)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(17)).to(torch.bfloat16)
    r1 = run_bwd(q, k, v, do, f32(128 ** -0.5), True, (-1, -1), gpu)
    r2 = run_bwd(q, k, v, do, f32(128 ** -0.5), True, (-1, -1), gpu)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("packed", [False, True], ids=["dense", "packed"])
def test_bwd_ignores_workspace_contents(packed, gpu):
    """The gradients do not depend on what the workspace held before the
    call: a workspace filled with NaN gives bit-identical results to a zeroed
    one (the padding rows past each sequence's end included)."""
    from exact_tiled_attention_fa_amd import _abi
    from exact_tiled_attention_fa_amd.attention import (flash_attn_bwd, flash_attn_fwd,
                                                        flash_attn_varlen, flash_attn_varlen_bwd)

    D, Hq, Hkv = 128, 4, 2
    q, k, v = W.randn_qkv(1, 277, 277, Hq, Hkv, D, torch.bfloat16, 18)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(19)).to(torch.bfloat16)
    q, k, v, do = (t.to(gpu) for t in (q, k, v, do))
    scale = f32(D ** -0.5)
    outs = []
    for fill in (0.0, float("nan")):
        if packed:
            cu = torch.tensor([0, 45, 45, 200, 277], dtype=torch.int32, device=gpu)
            args = (q[0], k[0], v[0])
            n = _abi.fa_bwd_workspace_size(4, Hq, 155)
            ws = torch.full((n // 4,), fill, dtype=torch.float32, device=gpu)
            o, lse = flash_attn_varlen(*args, cu, cu, 155, 155, softmax_scale=scale,
                                       causal=True)
            g = flash_attn_varlen_bwd(*args, o, lse, do[0], cu, cu, 155, 155,
                                      softmax_scale=scale, causal=True, workspace=ws)
        else:
            n = _abi.fa_bwd_workspace_size(1, Hq, 277)
            ws = torch.full((n // 4,), fill, dtype=torch.float32, device=gpu)
            o, lse = flash_attn_fwd(q, k, v, softmax_scale=scale, causal=True)
            g = flash_attn_bwd(q, k, v, o, lse, do, softmax_scale=scale, causal=True,
                               workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in g])
    for a, b in zip(*outs):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a, b)


def test_bwd_offsets_past_2_31(gpu):
    """136 batches made of 17 copies of 8 random ones (L = 512, 128 heads,
    D = 256: 2.3e9 elements per tensor, so element offsets run past 2^31).
    With no atomics every block's arithmetic is fixed, so the last copy's
    gradients, at the far end of memory, are bit-identical to the first
    copy's; the first copy matches the oracle on two (batch, head) slices."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_bwd, flash_attn_fwd

    Bs, R, L, H, D = 8, 17, 512, 128, 256
    q, k, v = W.randn_qkv(Bs, L, L, H, H, D, torch.bfloat16, 380)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(381)).to(torch.bfloat16)
    Q, K, V, DO = (t.repeat(R, 1, 1, 1).to(gpu) for t in (q, k, v, do))
    assert Q.numel() > 2 ** 31
    scale = f32(D ** -0.5)
    say(f"bwd past 2^31: B={Bs * R} L={L} H={H} D={D}")
    o, lse = flash_attn_fwd(Q, K, V, softmax_scale=scale, causal=False)
    dq, dk, dv = flash_attn_bwd(Q, K, V, o, lse, DO, softmax_scale=scale, causal=False)
    torch.cuda.synchronize()
    first = [t[:Bs].cpu() for t in (dq, dk, dv)]
    last = [t[-Bs:].cpu() for t in (dq, dk, dv)]
    del Q, K, V, DO, o, lse, dq, dk, dv
    for a, b in zip(first, last):
        assert torch.equal(a, b)
    heads = [(0, 0), (Bs - 1, H - 1)]
    r = oracle.attention_bwd_ref(q, k, v, do, scale, False, bounds=True, kv_heads=heads)
    compare_grad(first[0], r[0], r[3], torch.bfloat16, f"dq {heads}")
    compare_grad(first[1], r[1], r[4], torch.bfloat16, f"dk {heads}")
    compare_grad(first[2], r[2], r[5], torch.bfloat16, f"dv {heads}")


def test_bwd_full_size(gpu):
    """The Llama-2-7B-shaped causal workload (B=4, H=32, L=4096, D=128, bf16)
    in the launch the benchmark times; the oracle computes the gradients of
    every head of the first and of the last batch entry."""
    cfg = W.PREFILL["llama7b"]
    q, k, v = W.prefill_inputs(cfg)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 100)).to(cfg.dtype)
    scale = f32(cfg.scale)
    say("bwd full-size llama7b")
    dq, dk, dv = run_bwd(q, k, v, do, scale, True, (-1, -1), gpu)
    heads = [(b, c) for b in (0, cfg.B - 1) for c in range(cfg.Hkv)]
    r = oracle.attention_bwd_ref(q, k, v, do, scale, True, bounds=True, kv_heads=heads,
                                 workers=16)
    compare_grad(dq, r[0], r[3], cfg.dtype, "dq batch entries 0 and 3")
    compare_grad(dk, r[1], r[4], cfg.dtype, "dk batch entries 0 and 3")
    compare_grad(dv, r[2], r[5], cfg.dtype, "dv batch entries 0 and 3")


def test_bwd_errors(gpu):
    from exact_tiled_attention_fa_amd.attention import FAError, flash_attn_bwd

    q = torch.zeros((1, 8, 2, 96), dtype=torch.bfloat16, device=gpu)
    lse = torch.zeros((1, 2, 8), dtype=torch.float32, device=gpu)
    with pytest.raises(FAError, match="FA_ERR_UNSUPPORTED"):
        flash_attn_bwd(q, q, q, q, lse, q)
