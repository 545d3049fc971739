"""Seeded random sweep over the parameter space of every entry point, at sizes
the oracle finishes quickly: shapes, head groups, head sizes, dtypes, causal or
not, windows, packed sequence mixes (with empty ones), scales, page sizes,
cache formats and split counts drawn per case from a fixed seed.  Each case is
held to the same bound as the hand-picked tests of its entry point."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import compare, f32, say

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float16]


def draw_window(rng):
    r = rng.integers(0, 4)
    if r == 0:
        return (-1, -1)
    left = int(rng.integers(0, 200)) if rng.random() < 0.8 else -1
    right = int(rng.integers(0, 50)) if rng.random() < 0.6 else -1
    return (left, right)


def draw_heads(rng):
    """Small head counts, or (about a third of the draws) 16 to 64 query
    heads in multiples of 8, where the forward deals heads to the XCDs in
    windows (several heads per XCD) and the backward walks heads per XCD."""
    if rng.random() < 0.35:
        Hkv = int(rng.choice([2, 4, 8]))
        return Hkv * int(rng.choice([2, 4, 8])) if Hkv < 8 else 8 * int(rng.choice([2, 4, 8])), Hkv
    Hkv = int(rng.choice([1, 2, 3]))
    return Hkv * int(rng.choice([1, 2, 4, 5])), Hkv


@pytest.mark.parametrize("case", range(40))
def test_random_forward_dense(case, gpu):
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd

    rng = np.random.default_rng(1000 + case)
    B = int(rng.integers(1, 4))
    Lq, Lk = (int(x) for x in rng.integers(1, 600, 2))
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    scale = f32(float(rng.uniform(-0.3, 0.3)) if rng.random() < 0.2 else D ** -0.5)
    tag = (f"fwd B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} D={D} {str(dtype)[6:]} causal={causal} "
           f"window={window} s={scale:.4g}")
    say(tag)
    q, k, v = W.randn_qkv(B, Lq, Lk, Hq, Hkv, D, dtype, 2000 + case)
    o, lse = flash_attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), softmax_scale=scale, causal=causal,
                            window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal, window=window)
    compare(o.cpu(), lse.cpu(), o_ref, l_ref, tag)


def draw_lens(rng, n, hi):
    lens = [int(x) for x in rng.integers(0, hi, n)]
    for i in range(n):
        if rng.random() < 0.15:
            lens[i] = 0
    if max(lens) == 0:
        lens[0] = 1
    return lens


@pytest.mark.parametrize("case", range(30))
def test_random_forward_packed(case, gpu):
    from test_gpu_fwd import run_varlen

    rng = np.random.default_rng(3000 + case)
    n = int(rng.integers(1, 7))
    lens_q = draw_lens(rng, n, 400)
    lens_k = lens_q if rng.random() < 0.5 else draw_lens(rng, n, 400)
    if max(lens_k) == 0:
        lens_k = [max(1, x) for x in lens_k]
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    tag = f"packed q={lens_q} k={lens_k} Hq={Hq} Hkv={Hkv} D={D} causal={causal} window={window}"
    say(tag)
    o, lse, o_ref, l_ref = run_varlen(lens_q, lens_k, Hq, Hkv, D, dtype, causal, window,
                                      4000 + case, gpu)
    compare(o, lse, o_ref, l_ref, tag)


@pytest.mark.parametrize("case", range(20))
def test_random_backward(case, gpu):
    from test_gpu_bwd import check

    rng = np.random.default_rng(5000 + case)
    B = int(rng.integers(1, 3))
    Lq, Lk = (int(x) for x in rng.integers(1, 350, 2))
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    check(B, Lq, Lk, Hq, Hkv, D, dtype, causal, 6000 + case, gpu, window=window)


@pytest.mark.parametrize("case", range(12))
def test_random_backward_packed(case, gpu):
    from test_gpu_bwd_varlen import check

    rng = np.random.default_rng(7000 + case)
    n = int(rng.integers(1, 5))
    lens_q = draw_lens(rng, n, 300)
    lens_k = lens_q if rng.random() < 0.5 else draw_lens(rng, n, 300)
    if max(lens_k) == 0:
        lens_k = [max(1, x) for x in lens_k]
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    check(lens_q, lens_k, Hq, Hkv, D, dtype, causal, window, 8000 + case, gpu)


@pytest.mark.parametrize("case", range(30))
def test_random_decode_paged(case, gpu):
    from test_gpu_decode_paged import make_paged, run

    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 1500, B)]
    Hq, Hkv = draw_heads(rng)
    Hq = Hkv * int(rng.choice([1, 4, 8, 17]))
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    page = int(rng.choice([16, 32, 128, 512]))
    k8, v8 = [(False, False), (True, False), (True, True)][int(rng.integers(0, 3))]
    splits = int(rng.choice([1, 2, 5, 8, 13]))
    scale = f32(D ** -0.5)
    tag = f"paged B={B} lens={lens} Hq={Hq} Hkv={Hkv} D={D} page={page} k8={k8} v8={v8} S={splits}"
    say(tag)
    q, kp, vp, ks, vs, table, ln = make_paged(B, Hq, Hkv, D, lens, page, dtype, 10000 + case,
                                              k_int8=k8, v_int8=v8)
    o, lse = run(q, kp, vp, ks, vs, table, ln, scale, splits, gpu)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, ln, scale, k_scales=ks, v_scales=vs)
    compare(o, lse, o_ref, l_ref, tag)


@pytest.mark.parametrize("case", range(24))
def test_random_forward_fp8(case, gpu):
    """The FP8 forward over random shapes, head groups, D, causal, windows,
    scales and output types, held to the FP8 tests' derived bound."""
    from test_gpu_fp8 import check as fp8_check

    rng = np.random.default_rng(5000 + case)
    B = int(rng.integers(1, 3))
    Lq, Lk = (int(x) for x in rng.integers(1, 500, 2))
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    scale = float(rng.uniform(-0.3, 0.3)) if rng.random() < 0.2 else None
    out_dtype = DTYPES[int(rng.integers(0, 2))]
    fp8_check(B, Lq, Lk, Hq, Hkv, D, causal, 6000 + case, gpu, window=window, scale=scale,
              out_dtype=out_dtype)


@pytest.mark.parametrize("case", range(24))
def test_random_decode(case, gpu):
    """Split-KV decode over a dense cache: random batch, lengths (zero and
    past the cache length included), head groups up to 32, D, dtypes, split
    counts and scales; NaN in every cache row no sequence owns."""
    from test_gpu_decode import make_cache
    from test_gpu_decode import run as decode_run

    rng = np.random.default_rng(7000 + case)
    B = int(rng.integers(1, 6))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * int(rng.choice([1, 4, 5, 16, 32]))
    D = int(rng.choice([64, 128, 256]))
    dtype = DTYPES[int(rng.integers(0, 2))]
    lmax = int(rng.integers(1, 3000))
    lens = [int(rng.integers(0, lmax + 40)) for _ in range(B)]
    splits = int(rng.choice([1, 2, 3, 8, 16, 64]))
    scale = f32(float(rng.uniform(-0.3, 0.3)) if rng.random() < 0.2 else D ** -0.5)
    tag = (f"decode B={B} Hq={Hq} Hkv={Hkv} D={D} {str(dtype)[6:]} lmax={lmax} lens={lens} "
           f"splits={splits} s={scale:.4g}")
    say(tag)
    q, kc, vc, lens_t = make_cache(B, Hq, Hkv, D, lens, lmax, dtype, seed=8000 + case)
    o, lse = decode_run(q, kc, vc, lens_t, scale, splits, gpu)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens, scale)
    compare(o, lse, o_ref, l_ref, tag)


@pytest.mark.parametrize("case", range(12))
def test_random_forward_fp8_packed(case, gpu):
    """The FP8 forward over random packed mixes (empty sequences, starts off
    the 16-key grid), head groups, D, causal, windows and output types."""
    from test_gpu_fp8 import check_varlen

    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 6))
    lens_q = draw_lens(rng, B, 300)
    lens_k = lens_q if rng.random() < 0.5 else draw_lens(rng, B, 300)
    Hq, Hkv = draw_heads(rng)
    D = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    window = draw_window(rng)
    out_dtype = DTYPES[int(rng.integers(0, 2))]
    check_varlen(lens_q, lens_k, Hq, Hkv, D, causal, 9500 + case, gpu, window=window,
                 out_dtype=out_dtype)
