"""Backward parity for sequences packed back to back: libfa's fa_bwd_ex
(through the C ABI), fed by libfa's packed forward, against the exact
gradients of the fp64 oracle (``oracle.varlen_bwd_ref``).  The per-element
bound is the dense backward's (see test_gpu_bwd.py)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import f32, say
from test_gpu_bwd import compare_grad

pytestmark = pytest.mark.gpu


def run_varlen_bwd(q, k, v, do, cu_q, cu_k, max_q, max_k, scale, causal, window, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_varlen, flash_attn_varlen_bwd

    q, k, v, do, cq, ck = (t.to(dev) for t in (q, k, v, do, cu_q, cu_k))
    o, lse = flash_attn_varlen(q, k, v, cq, ck, max_q, max_k, softmax_scale=scale, causal=causal,
                               window=window)
    dq, dk, dv = flash_attn_varlen_bwd(q, k, v, o, lse, do, cq, ck, max_q, max_k,
                                       softmax_scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def packed_inputs(lens_q, lens_k, Hq, Hkv, D, dtype, seed):
    cu_q = torch.tensor(np.cumsum([0] + list(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor(np.cumsum([0] + list(lens_k)), dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((int(cu_q[-1]), Hq, D), generator=g).to(dtype)
    k = torch.randn((int(cu_k[-1]), Hkv, D), generator=g).to(dtype)
    v = torch.randn((int(cu_k[-1]), Hkv, D), generator=g).to(dtype)
    do = torch.randn(q.shape, generator=g).to(dtype)
    return q, k, v, do, cu_q, cu_k


def check(lens_q, lens_k, Hq, Hkv, D, dtype, causal, window, seed, gpu, kv_heads=None):
    q, k, v, do, cu_q, cu_k = packed_inputs(lens_q, lens_k, Hq, Hkv, D, dtype, seed)
    scale = f32(D ** -0.5)
    tag = (f"varlen bwd q={lens_q} k={lens_k} Hq={Hq} Hkv={Hkv} D={D} {str(dtype)[6:]} "
           f"causal={causal} window={window}")
    say(tag)
    dq, dk, dv = run_varlen_bwd(q, k, v, do, cu_q, cu_k, max(lens_q), max(lens_k), scale, causal,
                                window, gpu)
    r = oracle.varlen_bwd_ref(q, k, v, do, cu_q, cu_k, scale, causal, window=window, bounds=True,
                              kv_heads=kv_heads)
    compare_grad(dq, r[0], r[3], dtype, "dq")
    compare_grad(dk, r[1], r[4], dtype, "dk")
    compare_grad(dv, r[2], r[5], dtype, "dv")


CASES = [
    ([1, 130, 0, 257, 64], [5, 130, 3, 300, 64]),   # an empty query sequence: its keys get 0
    ([40, 7, 333], [0, 7, 400]),                    # an empty key sequence: its rows get dq 0
    ([128, 128, 128], [128, 128, 128]),
    ([300, 17], [129, 500]),                        # Lk < Lq and Lk > Lq (bottom-right causal)
]


@pytest.mark.parametrize("window", [(-1, -1), (32, 8)], ids=["nowin", "win32_8"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_bwd(case, D, causal, window, gpu):
    lens_q, lens_k = CASES[case]
    dtype = torch.float16 if D == 64 else torch.bfloat16
    check(lens_q, lens_k, 8, 2, D, dtype, causal, window, 11 * case + D, gpu)


def test_varlen_bwd_d256(gpu):
    check([1, 130, 0, 257, 64], [5, 130, 3, 300, 64], 4, 2, 256, torch.float16, True, (-1, -1),
          90, gpu)
    check([300, 17], [129, 500], 4, 4, 256, torch.bfloat16, False, (32, 8), 91, gpu)


@pytest.mark.parametrize("g", [1, 4])
def test_varlen_bwd_gqa(g, gpu):
    check([200, 65, 129], [200, 65, 129], 8, 8 // g, 128, torch.bfloat16, True, (-1, -1), 60 + g,
          gpu)


def test_varlen_bwd_equals_dense_batch(gpu):
    """Equal-length packing gives bit-identical gradients to the dense batch."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_bwd, flash_attn_fwd

    B, L, Hq, Hkv, D = 3, 300, 8, 2, 128
    q, k, v = (t.to(gpu) for t in W.randn_qkv(B, L, L, Hq, Hkv, D, torch.bfloat16, 70))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(71)).to(q.dtype).to(gpu)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32)
    for causal in (False, True):
        o, lse = flash_attn_fwd(q, k, v, causal=causal)
        g1 = flash_attn_bwd(q, k, v, o, lse, do, causal=causal)
        flat = lambda t: t.reshape(B * L, t.shape[2], D)
        g2 = run_varlen_bwd(flat(q).cpu(), flat(k).cpu(), flat(v).cpu(), flat(do).cpu(), cu, cu,
                            L, L, f32(D ** -0.5), causal, (-1, -1), gpu)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(flat(a).cpu(), b)


def test_varlen16_full_size(gpu):
    """The varlen16 workload (16 packed causal sequences, lengths U[256, 4096],
    Hq=32, Hkv=8, D=128) in full; the oracle computes the gradients of every
    (sequence, K/V head)."""
    cfg = W.MASKED["varlen16"]
    q, k, v, cu = W.masked_inputs(cfg)
    lens = cfg.lengths()
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(cfg.seed + 2)).to(cfg.dtype)
    scale = f32(cfg.scale)
    say(f"varlen16 bwd lens={lens}")
    dq, dk, dv = run_varlen_bwd(q, k, v, do, cu, cu, max(lens), max(lens), scale, True,
                                (-1, -1), gpu)
    r = oracle.varlen_bwd_ref(q, k, v, do, cu, cu, scale, True, bounds=True, workers=16)
    compare_grad(dq, r[0], r[3], cfg.dtype, "dq all sequences")
    compare_grad(dk, r[1], r[4], cfg.dtype, "dk all sequences")
    compare_grad(dv, r[2], r[5], cfg.dtype, "dv all sequences")
