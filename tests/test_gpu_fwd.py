"""Prefill parity: libfa's fa_fwd (through the C ABI) against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import compare, f32, say, to64

pytestmark = pytest.mark.gpu


def run(q, k, v, scale, causal, dev):
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd

    o, lse = flash_attn_fwd(q.to(dev), k.to(dev), v.to(dev), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(B, Lq, Lk, Hq, Hkv, D, dtype, causal, seed, gpu, scale=None, q_scale=1.0):
    scale = f32(scale if scale is not None else 1.0 / np.sqrt(D))
    q, k, v = W.randn_qkv(B, Lq, Lk, Hq, Hkv, D, dtype, seed, q_scale=q_scale)
    tag = f"B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} D={D} {str(dtype)[6:]} causal={causal} s={scale:.4g}"
    say(f"case {tag}")
    o, lse = run(q, k, v, scale, causal, gpu)
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal)
    return compare(o, lse, o_ref, l_ref, tag)


RAGGED = [(1, 1), (17, 17), (63, 63), (64, 64), (65, 65), (127, 127), (128, 128), (129, 129),
          (300, 300), (1000, 1000), (1, 129), (65, 200), (200, 65), (129, 4097)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lq,Lk", RAGGED, ids=[f"{a}x{b}" for a, b in RAGGED])
def test_ragged_sweep(Lq, Lk, D, dtype, causal, gpu):
    check(1, Lq, Lk, 4, 2, D, dtype, causal, seed=Lq * 7919 + Lk + D, gpu=gpu)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gqa_groups(g, D, gpu):
    check(2, 257, 257, 8, 8 // g, D, torch.bfloat16, True, seed=31 * g + D, gpu=gpu)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5, 3.0])
def test_scale_values(scale, gpu):
    check(1, 130, 130, 2, 1, 128, torch.bfloat16, True, seed=77, gpu=gpu, scale=scale)


def test_large_logits(gpu):
    """Scores spanning ~+-60: exercises the lazy rescale of the running max."""
    check(1, 700, 700, 2, 2, 64, torch.float16, False, seed=78, gpu=gpu, q_scale=8.0)
    check(1, 700, 700, 2, 2, 128, torch.bfloat16, True, seed=79, gpu=gpu, q_scale=8.0)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("direction", [1.0, -1.0], ids=["rising", "falling"])
def test_steadily_moving_scores(direction, causal, gpu):
    """Scores along the keys rise (or fall) by about 2 in log2 units every 32
    keys, about 60 over the row: rising, a row's reference max is overtaken
    again and again, so the accept-or-rescale test fires on many tiles;
    falling, the first tile already holds the maximum."""
    B, L, H, D = 1, 1000, 2, 128
    q, k, v = W.randn_qkv(B, L, L, H, H, D, torch.float32, 93)
    u = torch.randn(D, generator=torch.Generator().manual_seed(94))
    u = u / u.norm()
    ramp = direction * torch.arange(L, dtype=torch.float32) / L
    q = (16.0 * u + 0.5 * q).to(torch.bfloat16)
    k = (29.4 * ramp[None, :, None, None] * u + 0.5 * k).to(torch.bfloat16)
    v = v.to(torch.bfloat16)
    scale = f32(D ** -0.5)
    tag = f"moving scores direction={direction} causal={causal}"
    say(f"case {tag}")
    o, lse = run(q, k, v, scale, causal, gpu)
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal)
    compare(o, lse, o_ref, l_ref, tag)


@pytest.mark.parametrize("name", ["tiny", "encoder"])
def test_config_full(name, gpu):
    cfg = W.PREFILL[name]
    say(f"config {name}: {cfg}")
    q, k, v = W.prefill_inputs(cfg)
    o, lse = run(q, k, v, f32(cfg.scale), cfg.causal, gpu)
    o_ref, l_ref = oracle.attention_ref(q, k, v, f32(cfg.scale), cfg.causal)
    compare(o, lse, o_ref, l_ref, name)


@pytest.mark.parametrize("name", ["llama7b", "gqa16k", "d256"])
def test_config_full_size(name, gpu):
    """Full-size launch, the shape the benchmark times; the oracle computes
    every (batch, head) slice, so every workgroup's tile is checked (an
    unwritten tile would hold whatever the output allocation held)."""
    cfg = W.PREFILL[name]
    say(f"config {name}: {cfg}")
    q, k, v = W.prefill_inputs(cfg)
    o, lse = run(q, k, v, f32(cfg.scale), cfg.causal, gpu)
    o_ref, l_ref = oracle.attention_ref(q, k, v, f32(cfg.scale), cfg.causal)
    compare(o, lse, o_ref, l_ref, f"{name} all {cfg.B * cfg.Hq} (batch, head) slices")


def test_long_sequence_sampled_rows(gpu):
    """Q and O of 147456 x 128 heads x 128 dims: 2.4e9 elements, so element
    and byte offsets run past 2^31.  (Q repeats one random 16-head block over
    the 8 head groups, each group on its own K/V head, which keeps the input
    cheap to draw.)  In a causal prefill with Lq = Lk, query row i sees keys
    0..i, which is one query against a cache of length i + 1: the oracle's
    decode_ref gives that row exactly.  Rows at tile edges, the middle and
    the end, in the first and the last heads."""
    B, L, Hq, Hkv, D = 1, 147456, 128, 8, 128
    gen = torch.Generator().manual_seed(95)
    q = torch.randn((B, L, 16, D), generator=gen).to(torch.bfloat16).repeat(1, 1, Hq // 16, 1)
    _, k, v = W.randn_qkv(B, 1, L, 1, Hkv, D, torch.bfloat16, 97)
    assert q.numel() > 2 ** 31
    scale = f32(D ** -0.5)
    say(f"long causal prefill L={L} Hq={Hq} Hkv={Hkv} D={D}")
    o, lse = run(q, k, v, scale, True, gpu)
    heads = [0, 17, 120, 127]
    sel = np.array(heads)
    for i in [0, 1, 31, 32, 127, 128, 65537, 99999, L - 2, L - 1]:
        o_ref, l_ref = oracle.decode_ref(q[:, i], k, v, [i + 1], scale,
                                         heads=[(0, h) for h in heads])
        compare(o[:, i][:, sel], lse[:, sel, i], o_ref[:, sel], l_ref[:, sel], f"row {i}")


def test_causal_row0_is_exact(gpu):
    """Row 0 sees only key 0: P = 1 exactly, so O_0 = V[0] bit for bit and
    lse_0 = scale * q_0.k_0."""
    B, L, H, D = 2, 200, 4, 128
    q, k, v = W.randn_qkv(B, L, L, H, H, D, torch.bfloat16, 90)
    o, lse = run(q, k, v, f32(D ** -0.5), True, gpu)
    assert torch.equal(o[:, 0], v[:, 0])
    s00 = f32(D ** -0.5) * (to64(q[:, 0]) * to64(k[:, 0])).sum(-1)  # [B, H]
    assert np.max(np.abs(lse[:, :, 0].double().numpy() - s00)) < 1e-4


def test_uniform_queries_give_prefix_means(gpu):
    B, L, H, D = 1, 333, 2, 64
    _, k, v = W.randn_qkv(B, L, L, H, H, D, torch.float16, 91)
    q = torch.zeros((B, L, H, D), dtype=torch.float16)
    o, lse = run(q, k, v, 0.125, True, gpu)
    means = np.cumsum(to64(v)[0], axis=0) / np.arange(1, L + 1)[:, None, None]
    assert np.max(np.abs(to64(o)[0] - means)) < 2e-2
    assert np.max(np.abs(lse[0].double().numpy() - np.log(np.arange(1, L + 1))[None])) < 1e-3


def test_constant_values(gpu):
    B, L, H, D = 1, 257, 2, 128
    q, k, _ = W.randn_qkv(B, L, L, H, H, D, torch.bfloat16, 92, q_scale=4.0)
    c = torch.linspace(-3, 3, D).to(torch.bfloat16)
    v = c.expand(B, L, H, D).contiguous()
    o, _ = run(q, k, v, D ** -0.5, True, gpu)
    assert np.max(np.abs(to64(o) - to64(c)[None, None, None, :])) < 2e-2


def test_deterministic(gpu):
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd

    q, k, v = (t.to(gpu) for t in W.randn_qkv(2, 1000, 1000, 8, 2, 128, torch.bfloat16, 93))
    outs = [flash_attn_fwd(q, k, v, causal=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_errors_are_raised(gpu):
    from exact_tiled_attention_fa_amd.attention import FAError, flash_attn_fwd

    q = torch.zeros((1, 8, 2, 96), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(FAError, match="FA_ERR_UNSUPPORTED"):
        flash_attn_fwd(q, q, q)
    q = torch.zeros((1, 8, 3, 64), dtype=torch.bfloat16, device=gpu)
    k = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(FAError, match="FA_ERR_INVALID_ARGUMENT"):
        flash_attn_fwd(q, k, k)


# ---------------------------------------------------------------------------
# Structured masks: sliding windows and block-diagonal packing (fa_fwd_ex).
# ---------------------------------------------------------------------------
WINDOWS = [(0, 0), (5, 3), (64, -1), (-1, 40), (127, 0), (300, 300)]


@pytest.mark.parametrize("window", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lq,Lk", [(300, 300), (129, 331)], ids=["300x300", "129x331"])
def test_window(Lq, Lk, D, causal, window, gpu):
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd

    dtype = torch.bfloat16 if D != 256 else torch.float16
    scale = f32(D ** -0.5)
    q, k, v = W.randn_qkv(1, Lq, Lk, 4, 2, D, dtype, seed=Lq + Lk + D + window[0])
    tag = f"window {window} Lq={Lq} Lk={Lk} D={D} causal={causal}"
    say(tag)
    o, lse = flash_attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), softmax_scale=scale, causal=causal,
                            window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal, window=window)
    compare(o.cpu(), lse.cpu(), o_ref, l_ref, tag)


def run_varlen(lens_q, lens_k, Hq, Hkv, D, dtype, causal, window, seed, gpu, heads=None):
    from exact_tiled_attention_fa_amd.attention import flash_attn_varlen

    cu_q = torch.tensor(np.cumsum([0] + list(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor(np.cumsum([0] + list(lens_k)), dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((int(cu_q[-1]), Hq, D), generator=g).to(dtype)
    k = torch.randn((int(cu_k[-1]), Hkv, D), generator=g).to(dtype)
    v = torch.randn((int(cu_k[-1]), Hkv, D), generator=g).to(dtype)
    scale = f32(D ** -0.5)
    o, lse = flash_attn_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cu_q.to(gpu), cu_k.to(gpu),
                               max(lens_q), max(lens_k), softmax_scale=scale, causal=causal,
                               window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_ref(q, k, v, cu_q, cu_k, scale, causal, window=window, heads=heads)
    return o.cpu(), lse.cpu(), o_ref, l_ref


VARLEN_CASES = [
    ([1, 130, 0, 257, 64], [5, 130, 3, 300, 64]),   # an empty query sequence
    ([40, 7, 333], [0, 7, 400]),                    # an empty key sequence: rows see nothing
    ([128, 128, 128], [128, 128, 128]),
]


@pytest.mark.parametrize("window", [(-1, -1), (32, 8)], ids=["nowin", "win32_8"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_varlen(case, D, causal, window, gpu):
    lens_q, lens_k = VARLEN_CASES[case]
    dtype = torch.float16 if D == 64 else torch.bfloat16
    tag = f"varlen q={lens_q} k={lens_k} D={D} causal={causal} window={window}"
    say(tag)
    o, lse, o_ref, l_ref = run_varlen(lens_q, lens_k, 8, 2, D, dtype, causal, window, 7 * case + D,
                                      gpu)
    compare(o, lse, o_ref, l_ref, tag)


def test_varlen_equals_dense_batch(gpu):
    """Equal-length packing gives bit-identical results to the dense batch."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd, flash_attn_varlen

    B, L, H, D = 3, 300, 4, 128
    q, k, v = (t.to(gpu) for t in W.randn_qkv(B, L, L, H, H, D, torch.bfloat16, 55))
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device=gpu)
    for causal in (False, True):
        o1, l1 = flash_attn_fwd(q, k, v, causal=causal)
        o2, l2 = flash_attn_varlen(q.reshape(B * L, H, D), k.reshape(B * L, H, D),
                                   v.reshape(B * L, H, D), cu, cu, L, L, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1.reshape(B * L, H, D), o2)
        assert torch.equal(l1.permute(1, 0, 2).reshape(H, B * L), l2)


def test_varlen_offsets_past_2_31(gpu):
    """Packed causal prefill with 128 query and 128 K/V heads of 128 dims over
    lengths [131072, 16400]: the second sequence starts at element 2^31 of
    Q, K, V and O.  Each head gathers one of 16 drawn heads for Q, K and V
    through three different maps, so the (Q, K, V) triple differs between
    the checked heads.  Query row i of a sequence sees that sequence's keys
    0..i, which is one query against a cache of length i + 1 (decode_ref)."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_varlen

    lens, H, D = [131072, 16400], 128, 128
    T = sum(lens)
    assert lens[0] * H * D == 2 ** 31
    gen = torch.Generator().manual_seed(96)
    blocks = [torch.randn((T, 16, D), generator=gen).to(torch.bfloat16).to(gpu) for _ in range(3)]
    h = torch.arange(H)
    maps = [h % 16, (5 * h + h // 16) % 16, (3 * h + 7 * (h // 16)) % 16]
    q, k, v = (b.index_select(1, m.to(gpu)) for b, m in zip(blocks, maps))
    del blocks
    assert q.numel() > 2 ** 31 and k.numel() > 2 ** 31
    cu = torch.tensor([0, lens[0], T], dtype=torch.int32, device=gpu)
    scale = f32(D ** -0.5)
    say(f"packed causal prefill lens={lens} H={H} D={D}")
    o, lse = flash_attn_varlen(q, k, v, cu, cu, max(lens), max(lens), softmax_scale=scale,
                               causal=True)
    torch.cuda.synchronize()
    heads = [0, 17, 64, 127]
    sel = torch.tensor(heads, device=gpu)
    for s, rows in ((0, [0, 1, 127, 128, 65537, lens[0] - 1]),
                    (1, [0, 1, 31, 32, 8191, lens[1] - 1])):
        start = [0, lens[0]][s]
        for i in rows:
            r = start + i
            kk = k[start:r + 1].index_select(1, sel).cpu()[None]
            vv = v[start:r + 1].index_select(1, sel).cpu()[None]
            o_ref, l_ref = oracle.decode_ref(q[r].index_select(0, sel).cpu()[None], kk, vv,
                                             [i + 1], scale)
            compare(o[r].index_select(0, sel).cpu()[None], lse[:, r].index_select(0, sel).cpu()[None],
                    o_ref, l_ref, f"sequence {s} row {i}")


@pytest.mark.parametrize("name", ["swa16k", "varlen16"])
def test_masked_full_size(name, gpu):
    """The structured-mask workloads at full size, in the launch the benchmark
    times; the oracle computes every (sequence, head) slice."""
    from exact_tiled_attention_fa_amd.attention import flash_attn_fwd, flash_attn_varlen

    cfg = W.MASKED[name]
    q, k, v, cu = W.masked_inputs(cfg)
    lens = cfg.lengths()
    scale = f32(cfg.scale)
    say(f"{name}: lens={lens}")
    if cfg.packed:
        o, lse = flash_attn_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cu.to(gpu), cu.to(gpu),
                                   max(lens), max(lens), softmax_scale=scale, causal=cfg.causal,
                                   window=cfg.window)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.varlen_ref(q, k, v, cu, cu, scale, cfg.causal, window=cfg.window)
    else:
        o, lse = flash_attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), softmax_scale=scale,
                                causal=cfg.causal, window=cfg.window)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_ref(q, k, v, scale, cfg.causal, window=cfg.window)
    compare(o.cpu(), lse.cpu(), o_ref, l_ref, f"{name} all (sequence, head) slices")


def test_fwd_ex_errors(gpu):
    from exact_tiled_attention_fa_amd import _abi

    x = torch.zeros(64, dtype=torch.float32, device=gpu)
    cu = torch.zeros(4, dtype=torch.int32, device=gpu)
    p = x.data_ptr()
    st = _abi.fa_fwd_ex(p, p, p, p, p, cu.data_ptr(), None, 3, 2, 1, 8, 8, 8, 8, 64, 0.1, 0, -1,
                        -1, _abi.FA_BF16, None)
    assert st == _abi.FA_ERR_INVALID_ARGUMENT and "both be set" in _abi.fa_last_error()
    st = _abi.fa_fwd_ex(p, p, p, p, p, cu.data_ptr(), cu.data_ptr(), 3, 2, 1, 8, 8, 0, 8, 64, 0.1,
                        0, -1, -1, _abi.FA_BF16, None)
    assert st == _abi.FA_ERR_INVALID_ARGUMENT and "total_q" in _abi.fa_last_error()
