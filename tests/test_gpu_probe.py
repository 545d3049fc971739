"""The matrix-core ceiling probe (the benchmark's measurement helper, in its own
library libfa_probe.so): it executes the MFMAs it counts, on the operands it
is given."""

from __future__ import annotations

import pytest
import torch

from exact_tiled_attention_fa_amd import probe
from exact_tiled_attention_fa_amd.probe import mfma_probe
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [1, 64, 4096])
def test_probe_constant_operands_closed_form(iters, gpu):
    """Every operand 1.0: each MFMA adds 16 to each output, so a thread's
    accumulator sum is 16 outputs x (8 chained + 4 x 2) MFMAs x 16 per
    iteration = 4096 * iters, exact in float32 up to 4096 iterations."""
    say(f"probe iters={iters}")
    ones = torch.ones(4096, dtype=torch.bfloat16, device=gpu)
    out, flops = mfma_probe(ones, iters)
    torch.cuda.synchronize()
    n = probe.out_len()
    assert out.numel() == n and n % 256 == 0
    assert torch.all(out == 4096.0 * iters)
    assert flops == (n // 64) * iters * 16 * 2 * 32 * 32 * 16


def test_probe_reads_the_given_operands(gpu):
    """A buffer of 2.0 doubles every product (4x the all-ones sum); a buffer
    shorter than one thread's 18 operands is read modulo its length."""
    twos = torch.full((8,), 2.0, dtype=torch.bfloat16, device=gpu)  # one 16-byte operand
    out, _ = mfma_probe(twos, 3)
    torch.cuda.synchronize()
    assert torch.all(out == 4 * 4096.0 * 3)
    g = torch.Generator(device="cpu").manual_seed(5)
    rnd = torch.randn((1 << 16,), generator=g).to(torch.bfloat16).to(gpu)
    out, _ = mfma_probe(rnd, 8)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and out.abs().sum() > 0


def test_probe_rejects_short_output(gpu):
    ones = torch.ones(64, dtype=torch.bfloat16, device=gpu)
    out = torch.empty(probe.out_len() - 1, dtype=torch.float32, device=gpu)
    with pytest.raises(RuntimeError):
        mfma_probe(ones, 1, out)
