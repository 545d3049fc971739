"""Calls on two streams at once: the library keeps no state between calls
(no workspace of its own, no counters), so forward and decode calls enqueued
on two concurrent streams give the same bits as the same calls made one after
the other on one stream."""

from __future__ import annotations

import pytest
import torch

from exact_tiled_attention_fa_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_two_streams_match_serial(gpu):
    from exact_tiled_attention_fa_amd.attention import (decode_workspace, flash_attn_decode,
                                                        flash_attn_fwd)

    dt = torch.bfloat16
    qa, ka, va = (t.to(gpu) for t in W.randn_qkv(2, 700, 700, 8, 2, 128, dt, 130))
    qb, kb, vb = (t.to(gpu) for t in W.randn_qkv(3, 333, 900, 4, 4, 64, dt, 131))
    g = torch.Generator().manual_seed(132)
    qd = torch.randn((6, 16, 128), generator=g).to(dt).to(gpu)
    kc = torch.randn((6, 1000, 2, 128), generator=g).to(dt).to(gpu)
    vc = torch.randn((6, 1000, 2, 128), generator=g).to(dt).to(gpu)
    lens = torch.tensor([1, 1000, 17, 500, 999, 256], dtype=torch.int32, device=gpu)

    def work_a(ws):
        outs = []
        for i in range(3):
            outs.append(flash_attn_fwd(qa, ka, va, causal=i % 2 == 0))
            outs.append(flash_attn_decode(qd, kc, vc, lens, num_splits=4, workspace=ws))
        return outs

    def work_b():
        return [flash_attn_fwd(qb, kb, vb, causal=i % 2 == 1, window=(100, 7) if i == 2 else (-1, -1))
                for i in range(3)]

    ws_a = decode_workspace(6, 16, 128, 4, gpu)
    serial_a = work_a(ws_a)
    serial_b = work_b()
    torch.cuda.synchronize()

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    ws_c = decode_workspace(6, 16, 128, 4, gpu)
    for _ in range(3):
        with torch.cuda.stream(sa):
            conc_a = work_a(ws_c)
        with torch.cuda.stream(sb):
            conc_b = work_b()
        torch.cuda.synchronize()
        for x, y in zip(serial_a + serial_b, conc_a + conc_b):
            assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])
