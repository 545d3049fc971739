"""The library under HIP graph capture (a serving loop's use): the forward,
the split-KV decode and the backward are captured once into a torch CUDA graph
(on ROCm a HIP graph) and replayed several times, with new inputs copied in
and eager work and synchronisations between the replays.  Every replay must
equal an eager call on the same inputs bit for bit (the kernels are
deterministic, allocate nothing and record no memset)."""

from __future__ import annotations

import pytest
import torch

from exact_tiled_attention_fa_amd import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(gpu):
    from exact_tiled_attention_fa_amd.attention import (decode_workspace, flash_attn_bwd,
                                                        flash_attn_decode, flash_attn_fwd)

    B, L, Hq, Hkv, D = 2, 300, 8, 2, 128
    dt = torch.bfloat16
    q, k, v = (t.to(gpu) for t in W.randn_qkv(B, L, L, Hq, Hkv, D, dt, 120))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(121)).to(dt).to(gpu)
    Bd, Lmax = 5, 700
    g = torch.Generator().manual_seed(122)
    qd = torch.randn((Bd, Hq, D), generator=g).to(dt).to(gpu)
    kc = torch.randn((Bd, Lmax, Hkv, D), generator=g).to(dt).to(gpu)
    vc = torch.randn((Bd, Lmax, Hkv, D), generator=g).to(dt).to(gpu)
    lens = torch.tensor([1, 77, 700, 300, 513], dtype=torch.int32, device=gpu)
    ws = decode_workspace(Bd, Hq, D, 4, gpu)

    o, lse = torch.empty_like(q), torch.empty((B, Hq, L), dtype=torch.float32, device=gpu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    od, ld = torch.empty_like(qd), torch.empty((Bd, Hq), dtype=torch.float32, device=gpu)
    bws = torch.empty((2 * B * Hq * 320 * 4,), dtype=torch.uint8, device=gpu)

    def step(outs):
        o_, lse_, dq_, dk_, dv_, od_, ld_ = outs
        flash_attn_fwd(q, k, v, causal=True, out=o_, lse=lse_)
        flash_attn_bwd(q, k, v, o_, lse_, do, causal=True, dq=dq_, dk=dk_, dv=dv_, workspace=bws)
        flash_attn_decode(qd, kc, vc, lens, num_splits=4, workspace=ws, out=od_, lse=ld_)

    static = (o, lse, dq, dk, dv, od, ld)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(static)
    torch.cuda.synchronize()

    eager = tuple(torch.empty_like(t) for t in static)
    for rep in range(4):
        # new inputs, copied into the captured tensors by eager work
        gen = torch.Generator().manual_seed(200 + rep)
        for t in (q, k, v, do, qd, kc, vc):
            t.copy_(torch.randn(t.shape, generator=gen).to(dt))
        torch.cuda.synchronize()
        for t in static:
            t.fill_(float("nan"))  # a stale result must not pass
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eager)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "o_dec", "lse_dec"), static, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        say(f"graph replay {rep}: 7 outputs equal to eager")
