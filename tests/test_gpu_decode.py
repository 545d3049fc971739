"""Split-KV decode parity: libfa's fa_decode (through the C ABI) against the
fp64 oracle's decode_ref."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import compare, f32, say

pytestmark = pytest.mark.gpu


def make_cache(B, Hq, Hkv, D, lens, lmax, dtype, seed, pad=float("nan")):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g).to(dtype)
    kc = torch.full((B, lmax, Hkv, D), pad, dtype=dtype)
    vc = torch.full((B, lmax, Hkv, D), pad, dtype=dtype)
    for b, n in enumerate(lens):
        n = max(0, min(n, lmax))
        kc[b, :n] = torch.randn((n, Hkv, D), generator=g).to(dtype)
        vc[b, :n] = torch.randn((n, Hkv, D), generator=g).to(dtype)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32)


def run(q, kc, vc, lens, scale, splits, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_decode

    o, lse = flash_attn_decode(q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev), softmax_scale=scale,
                               num_splits=splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


LENS = [0, 1, 31, 32, 33, 100, 511, 777]


@pytest.mark.parametrize("splits", [1, 2, 8, 16, 64])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_decode_small(D, dtype, splits, gpu):
    B, Hq, Hkv, lmax = len(LENS), 8, 2, 800
    scale = f32(D ** -0.5)
    q, kc, vc, lens = make_cache(B, Hq, Hkv, D, LENS, lmax, dtype, seed=D + splits)
    tag = f"decode D={D} {str(dtype)[6:]} splits={splits}"
    say(tag)
    o, lse = run(q, kc, vc, lens, scale, splits, gpu)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens, scale)
    compare(o, lse, o_ref, l_ref, tag)
    assert torch.all(o[0] == 0) and torch.all(lse[0] == float("-inf"))  # empty cache


@pytest.mark.parametrize("splits", [8, 64])
def test_decode_long_cache(splits, gpu):
    """A cache of 3 x 800000 rows x 8 K/V heads x 128 dims (2.5e9 elements):
    the last sequence's 600000 rows lie past element 2^31 of the tensor.
    Unused rows hold NaN, so a stray read shows."""
    B, Hq, Hkv, D, lmax = 3, 32, 8, 128, 800000
    lens = [5, 100, 600000]
    q, kc, vc, lens_t = make_cache(B, Hq, Hkv, D, lens, lmax, torch.bfloat16, seed=96)
    assert kc.numel() > 2 ** 31
    scale = f32(D ** -0.5)
    say(f"decode long cache {lens} splits={splits}")
    o, lse = run(q, kc, vc, lens_t, scale, splits, gpu)
    heads = [(b, h) for b in range(B) for h in (0, 13, 31)]
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens, scale, heads=heads)
    compare(o, lse, o_ref, l_ref, f"long cache splits={splits}")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2), (64, 2), (40, 8)])
def test_decode_head_groups(Hq, Hkv, gpu):
    """Group sizes 1, 8, 32 (two 16-head groups) and 5 (ragged group)."""
    lens = [5, 300, 1024]
    q, kc, vc, lens_t = make_cache(3, Hq, Hkv, 128, lens, 1024, torch.bfloat16, seed=Hq * Hkv)
    o, lse = run(q, kc, vc, lens_t, f32(128 ** -0.5), 8, gpu)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens_t, f32(128 ** -0.5))
    compare(o, lse, o_ref, l_ref, f"decode Hq={Hq} Hkv={Hkv}")


def test_decode_lengths_clamped(gpu):
    """Lengths outside [0, Lk_max] are clamped on the device."""
    q, kc, vc, _ = make_cache(3, 4, 1, 64, [64, 64, 0], 64, torch.float16, seed=5, pad=0.0)
    lens = torch.tensor([-5, 1000, 64], dtype=torch.int32)
    o, lse = run(q, kc, vc, lens, 0.125, 4, gpu)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, [0, 64, 64], f32(0.125))
    compare(o, lse, o_ref, l_ref, "clamped lengths")


def test_decode_equals_last_prefill_row(gpu):
    from exact_tiled_attention_fa_amd.attention import flash_attn_decode, flash_attn_fwd

    L, Hq, Hkv, D = 700, 8, 2, 128
    g = torch.Generator().manual_seed(9)
    qf = torch.randn((1, L, Hq, D), generator=g).to(torch.bfloat16).to(gpu)
    kf = torch.randn((1, L, Hkv, D), generator=g).to(torch.bfloat16).to(gpu)
    vf = torch.randn((1, L, Hkv, D), generator=g).to(torch.bfloat16).to(gpu)
    o_p, l_p = flash_attn_fwd(qf, kf, vf, causal=True)
    o_d, l_d = flash_attn_decode(qf[:, -1].contiguous(), kf, vf,
                                 torch.tensor([L], dtype=torch.int32, device=gpu), num_splits=5)
    torch.cuda.synchronize()
    assert (o_p[0, -1].float() - o_d[0].float()).abs().max().item() < 2e-2
    assert (l_p[0, :, -1] - l_d[0]).abs().max().item() < 1e-3


def test_decode_splits_agree_and_deterministic(gpu):
    lens = [4000, 123, 2048, 999]
    q, kc, vc, lens_t = make_cache(4, 32, 8, 128, lens, 4096, torch.bfloat16, seed=11)
    res = {s: run(q, kc, vc, lens_t, f32(128 ** -0.5), s, gpu) for s in (1, 2, 8, 16)}
    for s in (2, 8, 16):
        assert (res[s][0].float() - res[1][0].float()).abs().max().item() < 2e-2
        assert (res[s][1] - res[1][1]).abs().max().item() < 1e-3
    again = run(q, kc, vc, lens_t, f32(128 ** -0.5), 8, gpu)
    assert torch.equal(again[0], res[8][0]) and torch.equal(again[1], res[8][1])


def test_decode_config_full_size(gpu):
    """The full decode workload (128 sequences, lengths U[512, 8192], NaN
    padding, 8 splits); the oracle computes every sequence and head."""
    cfg = W.DECODE["decode"]
    say(f"config decode: {cfg}")
    q, kc, vc, lens = W.decode_inputs(cfg)
    o, lse = run(q, kc, vc, lens, f32(cfg.scale), cfg.num_splits, gpu)
    assert torch.all(torch.isfinite(o.float())), "padding leaked into the output"
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens, f32(cfg.scale), workers=16)
    compare(o, lse, o_ref, l_ref, f"decode full (all {cfg.B} sequences x {cfg.Hq} heads)")
