"""FP8 forward parity: libfa's fa_fwd_fp8 (through the C ABI) against the fp64
oracle on the decoded e4m3 inputs.

Error bound (derived from the arithmetic): the scores of e4m3 codes are exact
products summed in fp32, so the only rounding beyond the 16-bit output is P's
rounding to e4m3 for the PV product (relative error <= 2^-4 for the normal
range; 64 * P keeps P >= 2^-12 of the running reference normal).  Hence per element
|dO| <= 2^-4 * sum_j P_ij |v_j| (the oracle's `mag`) + u_out |O| + 1e-4, and lse
(from unrounded probabilities) keeps the 16-bit path's 1e-3 bound.
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


def compare_fp8(o, lse, o_ref, l_ref, mag, out_dtype, what):
    og, lg = to64(o), to64(lse)
    o_ref, l_ref, mag = np.asarray(o_ref), np.asarray(l_ref), np.asarray(mag)
    sel, lsel = ~np.isnan(o_ref), ~np.isnan(l_ref)
    assert sel.any() and np.all(np.isfinite(og[sel])), f"{what}: non-finite output"
    linf = lsel & np.isinf(l_ref)
    assert np.array_equal(lg[linf], l_ref[linf]), f"{what}: empty-row lse differs"
    lfin = lsel & ~np.isinf(l_ref)
    tol = 2.0 ** -4 * mag[sel] + UNIT[out_dtype] * np.abs(o_ref[sel]) + 1e-4
    err = np.abs(og[sel] - o_ref[sel])
    ratio = float(np.max(err / tol))
    dl = float(np.max(np.abs(lg[lfin] - l_ref[lfin]))) if lfin.any() else 0.0
    rms = float(np.sqrt(np.mean(err ** 2)))
    say(f"  {what}: max|dO|={err.max():.3e} rms {rms:.2e} worst err/bound={ratio:.3f} "
        f"max|dlse|={dl:.2e}")
    assert ratio <= 1.0, f"{what}: O error exceeds the bound by {ratio:.2f}x"
    assert dl <= 1e-3, f"{what}: max|dlse| {dl:.3e} > 1e-3"


def run_fp8(q8, k8, vt8, ds, scale, causal, window, out_dtype, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd_fp8

    o, lse = flash_attn_fwd_fp8(q8.to(dev), k8.to(dev), vt8.to(dev), q_descale=ds, k_descale=ds,
                                v_descale=ds, softmax_scale=scale, causal=causal, window=window,
                                out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(B, Lq, Lk, Hq, Hkv, D, causal, seed, gpu, *, window=(-1, -1), scale=None,
          out_dtype=torch.bfloat16, q_scale=1.0, heads=None):
    scale = f32(scale if scale is not None else D ** -0.5)
    q8, k8, vt8, ds = W.fp8_inputs(B, Lq, Lk, Hq, Hkv, D, seed, q_scale=q_scale)
    tag = f"fp8 B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} D={D} causal={causal} window={window}"
    say(tag)
    o, lse = run_fp8(q8, k8, vt8, ds, scale, causal, window, out_dtype, gpu)
    o_ref, l_ref, mag = oracle.attention_fp8_ref(q8, k8, vt8, Lk, scale, ds, ds, ds, causal,
                                                 heads=heads)
    if window != (-1, -1):  # the fp8 oracle has no window argument: rebuild it from the definition
        q = oracle.e4m3_decode(q8) * ds
        k = oracle.e4m3_decode(k8) * ds
        v = np.ascontiguousarray(oracle.e4m3_decode(vt8)[..., :Lk].transpose(0, 3, 1, 2)) * ds
        o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal, window=window)
        mag, _ = oracle.attention_ref(q, k, np.abs(v), scale, causal, window=window)
    compare_fp8(o, lse, o_ref, l_ref, mag, out_dtype, tag)


RAGGED = [(1, 1), (17, 17), (63, 63), (64, 64), (65, 65), (128, 128), (129, 129), (300, 300),
          (1000, 1000), (1, 129), (65, 200), (200, 65), (129, 4097)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lq,Lk", RAGGED, ids=[f"{a}x{b}" for a, b in RAGGED])
def test_fp8_ragged(Lq, Lk, D, causal, gpu):
    check(1, Lq, Lk, 4, 2, D, causal, seed=Lq * 13 + Lk + D, gpu=gpu)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_fp8_gqa(g, gpu):
    check(2, 257, 257, 8, 8 // g, 128, True, seed=50 + g, gpu=gpu)


@pytest.mark.parametrize("window", [(0, 0), (5, 3), (64, -1), (-1, 40)],
                         ids=["w0_0", "w5_3", "w64_", "w_40"])
def test_fp8_windows(window, gpu):
    check(1, 300, 300, 4, 2, 128, True, seed=60 + window[0], gpu=gpu, window=window)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_fp8_scales(scale, gpu):
    check(1, 130, 130, 2, 1, 128, True, seed=70, gpu=gpu, scale=scale)


def test_fp8_f16_output_and_large_logits(gpu):
    check(1, 700, 700, 2, 2, 64, False, seed=71, gpu=gpu, out_dtype=torch.float16)
    check(1, 700, 700, 2, 2, 128, True, seed=72, gpu=gpu, q_scale=4.0)


def test_fp8_full_size(gpu):
    """The Llama-2-7B-shaped causal workload (B=4, H=32, L=4096, D=128) in fp8,
    in the launch the benchmark times; the oracle computes every (batch, head)
    slice."""
    cfg = W.PREFILL["llama7b"]
    check(cfg.B, cfg.L, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, True, seed=cfg.seed, gpu=gpu)


def test_fp8_d256_full_size(gpu):
    """The D = 256 workload's shape (B=2, H=16, L=4096, causal) in fp8; at
    D = 256 two workgroups share each query tile, 128 output dimensions each.
    The oracle computes every (batch, head) slice."""
    cfg = W.PREFILL["d256"]
    check(cfg.B, cfg.L, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, True, seed=cfg.seed, gpu=gpu,
          out_dtype=torch.float16)


@pytest.mark.parametrize("window", [(0, 0), (64, -1)], ids=["w0_0", "w64_"])
def test_fp8_d256_gqa_window(window, gpu):
    check(2, 300, 333, 8, 2, 256, True, seed=66 + window[0], gpu=gpu, window=window)


def test_fp8_deterministic(gpu):
    q8, k8, vt8, ds = W.fp8_inputs(2, 1000, 1000, 8, 2, 128, 73)
    a = run_fp8(q8, k8, vt8, ds, 0.088, True, (-1, -1), torch.bfloat16, gpu)
    b = run_fp8(q8, k8, vt8, ds, 0.088, True, (-1, -1), torch.bfloat16, gpu)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# Packed sequences (fa_fwd_fp8_ex): query / key length mixes with an empty
# query sequence, an empty key sequence, starts off the 16-key grid and on it,
# and Lk != Lq within one batch.
VARLEN_MIXES = [
    ([5, 0, 37, 64, 1, 130], [5, 20, 37, 64, 1, 130]),
    ([40, 17, 200], [40, 17, 200]),
    ([16, 48, 64], [16, 48, 64]),
    ([33, 1, 90], [70, 129, 0]),
]


def check_varlen(lens_q, lens_k, Hq, Hkv, D, causal, seed, gpu, *, window=(-1, -1), scale=None,
                 out_dtype=torch.bfloat16):
    from exact_tiled_attention_fa_amd.attention import flash_attn_varlen_fp8

    scale = f32(scale if scale is not None else D ** -0.5)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q8, k8, vt8, ds = W.fp8_varlen_inputs(total_q, total_k, Hq, Hkv, D, seed)
    tag = (f"fp8 varlen q={lens_q} k={lens_k} Hq={Hq} Hkv={Hkv} D={D} causal={causal} "
           f"window={window}")
    say(tag)
    o, lse = flash_attn_varlen_fp8(q8.to(gpu), k8.to(gpu), vt8.to(gpu),
                                   torch.from_numpy(cu_q).to(gpu), torch.from_numpy(cu_k).to(gpu),
                                   max(lens_q), max(lens_k), q_descale=ds, k_descale=ds,
                                   v_descale=ds, softmax_scale=scale, causal=causal, window=window,
                                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    q = oracle.e4m3_decode(q8) * ds
    k = oracle.e4m3_decode(k8) * ds
    v = np.ascontiguousarray(oracle.e4m3_decode(vt8)[..., :total_k].transpose(2, 0, 1)) * ds
    o_ref, l_ref = oracle.varlen_ref(q, k, v, cu_q, cu_k, scale, causal, window=window)
    mag, _ = oracle.varlen_ref(q, k, np.abs(v), cu_q, cu_k, scale, causal, window=window)
    compare_fp8(o.cpu(), lse.cpu(), o_ref, l_ref, mag, out_dtype, tag)


@pytest.mark.parametrize("window", [(-1, -1), (32, 8)], ids=["nowin", "win"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("mix", range(len(VARLEN_MIXES)))
def test_fp8_varlen(mix, D, causal, window, gpu):
    lq, lk = VARLEN_MIXES[mix]
    check_varlen(lq, lk, 4, 2, D, causal, 300 + 10 * mix + D, gpu, window=window)


@pytest.mark.parametrize("g", [1, 4])
def test_fp8_varlen_gqa_f16_out(g, gpu):
    check_varlen([77, 3, 150], [77, 3, 150], 8, 8 // g, 128, True, 340 + g, gpu,
                 out_dtype=torch.float16, scale=-0.09)


def test_fp8_varlen_equals_dense_batch(gpu):
    """Equal-length sequences starting on the 64-key grid take the same tile
    walk as the dense batch: bit-identical O and lse."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd_fp8, flash_attn_varlen_fp8

    B, L, Hq, Hkv, D = 3, 192, 4, 2, 128
    q8, k8, vt8, ds = W.fp8_varlen_inputs(B * L, B * L, Hq, Hkv, D, 350)
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32)
    kw = dict(q_descale=ds, k_descale=ds, v_descale=ds, causal=True)
    o_p, l_p = flash_attn_varlen_fp8(q8.to(gpu), k8.to(gpu), vt8.to(gpu), cu.to(gpu), cu.to(gpu),
                                     L, L, **kw)
    vt_dense = vt8[..., :B * L].reshape(Hkv, D, B, L).permute(2, 0, 1, 3).contiguous()
    o_d, l_d = flash_attn_fwd_fp8(q8.view(B, L, Hq, D).to(gpu), k8.view(B, L, Hkv, D).to(gpu),
                                  vt_dense.to(gpu), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_p.cpu().view(B, L, Hq, D), o_d.cpu())
    assert torch.equal(l_p.cpu().view(Hq, B, L).permute(1, 0, 2), l_d.cpu())


def test_fp8_long_sequence_sampled_rows(gpu):
    """Q and O of 147456 rows x 128 heads x 128 dims (2.4e9 elements, offsets
    past 2^31; Q repeats one random 16-head block over the 8 head groups).
    A causal row i with Lq = Lk is one query against its i + 1 first keys:
    the oracle's decode_ref on the decoded values gives it (and, on |v|, the
    magnitude the bound needs)."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd_fp8

    B, L, Hq, Hkv, D = 1, 147456, 128, 8, 128
    q16, k8, vt8, ds = W.fp8_inputs(B, L, L, 16, Hkv, D, 360)
    q8 = q16.repeat(1, 1, Hq // 16, 1)
    assert q8.numel() > 2 ** 31
    scale = f32(D ** -0.5)
    say(f"fp8 long causal L={L} Hq={Hq} Hkv={Hkv} D={D}")
    o, lse = flash_attn_fwd_fp8(q8.to(gpu), k8.to(gpu), vt8.to(gpu), q_descale=ds, k_descale=ds,
                                v_descale=ds, softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    k = oracle.e4m3_decode(k8) * ds
    v = np.ascontiguousarray(oracle.e4m3_decode(vt8)[..., :L].transpose(0, 3, 1, 2)) * ds
    heads = [0, 17, 120, 127]
    sel = np.array(heads)
    hs = [(0, h) for h in heads]
    for i in [0, 1, 63, 64, 127, 128, 65537, L - 1]:
        qi = oracle.e4m3_decode(q8[:, i]) * ds
        o_ref, l_ref = oracle.decode_ref(qi, k, v, [i + 1], scale, heads=hs)
        mag, _ = oracle.decode_ref(qi, k, np.abs(v), [i + 1], scale, heads=hs)
        compare_fp8(o[:, i][:, sel], lse[:, sel, i], o_ref[:, sel], l_ref[:, sel], mag[:, sel],
                    torch.bfloat16, f"row {i}")
