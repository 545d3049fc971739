"""Paged / int8 KV-cache decode parity: libfa's fa_decode_paged (through the C
ABI) against the fp64 oracle's decode_paged_ref."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import compare, f32, say

pytestmark = pytest.mark.gpu

FORMATS = {"native": (False, False), "k8": (True, False), "kv8": (True, True)}


def make_paged(B, Hq, Hkv, D, lens, page_size, dtype, seed, *, k_int8=False, v_int8=False,
               extra_pages=3):
    """Pages in shuffled physical order; everything no sequence owns is NaN
    (int8: NaN scales), and table entries past a sequence's end point at a
    NaN page, so any read of them shows in the output."""
    g = torch.Generator().manual_seed(seed)
    need = [(n + page_size - 1) // page_size for n in lens]
    max_pages = max(1, max(need))
    num_pages = sum(need) + extra_pages
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((B, max_pages), int(perm[-1]), dtype=torch.int32)

    def pool(i8):
        if i8:
            return (torch.full((num_pages, page_size, Hkv, D), 127, dtype=torch.int8),
                    torch.full((num_pages, Hkv, page_size), float("nan")))
        return torch.full((num_pages, page_size, Hkv, D), float("nan"), dtype=dtype), None

    kp, ks = pool(k_int8)
    vp, vs = pool(v_int8)
    q = torch.randn((B, Hq, D), generator=g).to(dtype)
    nxt = 0
    for b, n in enumerate(lens):
        pages = perm[nxt:nxt + need[b]].tolist()
        nxt += need[b]
        table[b, :need[b]] = torch.tensor(pages, dtype=torch.int32)
        for pool_x, pool_s, i8 in ((kp, ks, k_int8), (vp, vs, v_int8)):
            x = torch.randn((n, Hkv, D), generator=g)
            if i8:
                codes = torch.round(x * 45).clamp(-127, 127).to(torch.int8)
                sc = torch.rand((n, Hkv), generator=g) * 0.008 + 0.018
            for i, pg in enumerate(pages):
                r0, r1 = i * page_size, min(n, (i + 1) * page_size)
                if i8:
                    pool_x[pg, :r1 - r0] = codes[r0:r1]
                    pool_s[pg, :, :r1 - r0] = sc[r0:r1].T
                else:
                    pool_x[pg, :r1 - r0] = x[r0:r1].to(dtype)
    return q, kp, vp, ks, vs, table, torch.tensor(lens, dtype=torch.int32)


def run(q, kp, vp, ks, vs, table, lens, scale, splits, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_decode_paged

    to = lambda t: None if t is None else t.to(dev)
    o, lse = flash_attn_decode_paged(q.to(dev), kp.to(dev), vp.to(dev), table.to(dev),
                                     lens.to(dev), k_scales=to(ks), v_scales=to(vs),
                                     softmax_scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


LENS = [0, 1, 15, 16, 17, 100, 511, 777]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("splits", [1, 3, 8])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_paged_small(D, dtype, splits, page_size, fmt, gpu):
    k8, v8 = FORMATS[fmt]
    B, Hq, Hkv = len(LENS), 8, 2
    scale = f32(D ** -0.5)
    q, kp, vp, ks, vs, table, lens = make_paged(B, Hq, Hkv, D, LENS, page_size, dtype,
                                                seed=D + 7 * splits + page_size, k_int8=k8,
                                                v_int8=v8)
    tag = f"paged D={D} {str(dtype)[6:]} splits={splits} page={page_size} {fmt}"
    say(tag)
    o, lse = run(q, kp, vp, ks, vs, table, lens, scale, splits, gpu)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens, scale, k_scales=ks, v_scales=vs)
    compare(o, lse, o_ref, l_ref, tag)
    assert torch.all(o[0] == 0) and torch.all(lse[0] == float("-inf"))  # empty cache


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2), (64, 2), (40, 8)])
def test_paged_head_groups(Hq, Hkv, gpu):
    lens = [5, 300, 1024]
    q, kp, vp, ks, vs, table, lens_t = make_paged(3, Hq, Hkv, 128, lens, 32, torch.bfloat16,
                                                  seed=Hq + Hkv, k_int8=True, v_int8=True)
    say(f"paged groups Hq={Hq} Hkv={Hkv}")
    o, lse = run(q, kp, vp, ks, vs, table, lens_t, 0.09, 4, gpu)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens_t, 0.09, k_scales=ks,
                                           v_scales=vs)
    compare(o, lse, o_ref, l_ref, f"groups {Hq}/{Hkv}")


def test_paged_equals_dense_layout(gpu):
    """Pages laid out in order are the padded dense cache: fa_decode_paged
    and fa_decode agree within the parity bounds of the oracle."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_decode, flash_attn_decode_paged

    B, Hq, Hkv, D, L, P = 4, 8, 2, 128, 640, 32
    g = torch.Generator().manual_seed(5)
    q = torch.randn((B, Hq, D), generator=g).to(torch.bfloat16).to(gpu)
    kc = torch.randn((B, L, Hkv, D), generator=g).to(torch.bfloat16).to(gpu)
    vc = torch.randn((B, L, Hkv, D), generator=g).to(torch.bfloat16).to(gpu)
    lens = torch.tensor([640, 1, 333, 32], dtype=torch.int32, device=gpu)
    table = torch.arange(B * (L // P), dtype=torch.int32, device=gpu).reshape(B, L // P)
    o1, l1 = flash_attn_decode(q, kc, vc, lens, num_splits=5)
    o2, l2 = flash_attn_decode_paged(q, kc.reshape(-1, P, Hkv, D), vc.reshape(-1, P, Hkv, D),
                                     table, lens, num_splits=5)
    o_ref, l_ref = oracle.decode_ref(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu(), D ** -0.5)
    compare(o1.cpu(), l1.cpu(), o_ref, l_ref, "dense")
    compare(o2.cpu(), l2.cpu(), o_ref, l_ref, "paged identity table")


def test_paged_table_entries_are_clamped(gpu):
    """A used table entry past num_pages reads the last page (documented
    clamp), never out of bounds."""
    B, Hq, Hkv, D, P = 2, 4, 1, 64, 16
    q, kp, vp, ks, vs, table, lens = make_paged(B, Hq, Hkv, D, [20, 40], P, torch.bfloat16, 3,
                                                extra_pages=0)
    bad = table.clone()
    last = kp.shape[0] - 1
    bad[1, 2] = 10 ** 6            # page 2 of sequence 1 -> clamped to the last page
    fixed = table.clone()
    fixed[1, 2] = last
    o1, l1 = run(q, kp, vp, ks, vs, bad, lens, 0.125, 2, gpu)
    o2, l2 = run(q, kp, vp, ks, vs, fixed, lens, 0.125, 2, gpu)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_deterministic(gpu):
    q, kp, vp, ks, vs, table, lens = make_paged(4, 16, 4, 128, [100, 2000, 5, 999], 16,
                                                torch.bfloat16, 9, k_int8=True, v_int8=True)
    r = [run(q, kp, vp, ks, vs, table, lens, 0.1, 8, gpu) for _ in range(3)]
    for o, l in r[1:]:
        assert torch.equal(o, r[0][0]) and torch.equal(l, r[0][1])


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_paged_full_size(fmt, gpu):
    """The full decode workload (128 sequences, lengths U[512, 8192], Hq=32,
    Hkv=8, D=128, bf16, 8 splits) in 16-slot pages, as the benchmark times it;
    the oracle computes every sequence and head."""
    k8, v8 = FORMATS[fmt]
    cfg = W.DECODE["decode"]
    say(f"paged full-size {fmt}")
    q, kp, vp, ks, vs, table, lens = W.paged_decode_inputs(cfg, 16, k_int8=k8, v_int8=v8)
    scale = f32(cfg.scale)
    o, lse = run(q, kp, vp, ks, vs, table, lens, scale, cfg.num_splits, gpu)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens, scale, k_scales=ks,
                                           v_scales=vs, workers=16)
    compare(o, lse, o_ref, l_ref, f"paged full-size {fmt} (all {cfg.B} sequences)")


@pytest.mark.parametrize("fmt", ["native", "kv8"])
def test_decode_paged_large_pool(fmt, gpu):
    """A pool of 8400 pages x 256 slots x 8 K/V heads x 128 (2.2e9 elements)
    with every page the sequences own at its top, past element 2^31; the rest
    of the pool is NaN (int8: NaN scales)."""
    k8, v8 = FORMATS[fmt]
    B, Hq, Hkv, D, ps = 3, 32, 8, 128, 256
    lens = [3000, 77, 2049]
    q, kp, vp, ks, vs, table, lens_t = make_paged(B, Hq, Hkv, D, lens, ps, torch.bfloat16, 370,
                                                  k_int8=k8, v_int8=v8, extra_pages=1)
    big = 8400
    off = big - kp.shape[0]

    def grow(x, fill):
        if x is None:
            return None
        y = torch.full((big,) + tuple(x.shape[1:]), fill, dtype=x.dtype)
        y[off:] = x
        return y

    kp = grow(kp, 127 if k8 else float("nan"))
    vp = grow(vp, 127 if v8 else float("nan"))
    ks, vs = grow(ks, float("nan")), grow(vs, float("nan"))
    table = table + off
    assert kp.numel() > 2 ** 31 and int(table.min()) * ps * Hkv * D > 2 ** 31
    scale = f32(D ** -0.5)
    say(f"paged large pool {fmt} lens={lens}")
    o, lse = run(q, kp, vp, ks, vs, table, lens_t, scale, 8, gpu)
    heads = [(b, h) for b in range(B) for h in (0, 13, 31)]
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens_t, scale, k_scales=ks,
                                           v_scales=vs, heads=heads)
    compare(o, lse, o_ref, l_ref, f"large pool {fmt}")


@pytest.mark.parametrize("splits", [1, 8])
def test_paged_fp16_int8_values_large_scales(splits, gpu):
    """fp16 with int8 values whose row scales lie in [300, 500] (values up to
    127 * 500 = 63,500, inside fp16): each probability is multiplied by its
    row's scale before the 16-bit rounding, so it must stay <= 1 there or
    p * scale overflows fp16.  The errors here are relative to the values'
    magnitude: O and each p * scale are rounded to fp16 (relative 2^-11), so
    with |values| up to 63,500 the absolute error reaches about
    3 * 2^-11 * 63,500 = 93 (the half-ulp of fp16 above 32,768 alone is 16).
    O and the oracle are compared after dividing by 8000, which maps that
    bound to 0.012, inside the 2e-2 bar; an overflow shows as inf / NaN."""
    B, Hq, Hkv, D, P = 3, 8, 2, 128, 16
    lens = [700, 33, 2048]
    q, kp, vp, ks, vs, table, lens_t = make_paged(B, Hq, Hkv, D, lens, P, torch.float16, 41,
                                                  k_int8=True, v_int8=True)
    g = torch.Generator().manual_seed(42)
    owned = ~torch.isnan(vs)
    vs = torch.where(owned, torch.rand(vs.shape, generator=g) * 200 + 300, vs)
    # sharp scores, so the running max moves within a sequence's keys
    q = (q.float() * 4).to(torch.float16)
    scale = f32(D ** -0.5)
    say(f"paged fp16 int8 values, scales in [300, 500], splits={splits}")
    o, lse = run(q, kp, vp, ks, vs, table, lens_t, scale, splits, gpu)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens_t, scale, k_scales=ks,
                                           v_scales=vs)
    assert torch.all(torch.isfinite(o.float()))
    compare(o.double() / 8000, lse, o_ref / 8000, l_ref, f"fp16 int8-V large scales s={splits}")
