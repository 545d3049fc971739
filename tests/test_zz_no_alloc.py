"""fa_decode_noalloc (split partials in the library's static device array)
against fa_decode (caller workspace), through the C ABI: bit-identical
outputs on two calls in a row, the second with a smaller input, and both
within the parity bounds of the oracle."""

from __future__ import annotations

import pytest
import torch

import oracle
from exact_tiled_attention_fa_amd import _abi
from gpu_util import compare, f32, say

pytestmark = pytest.mark.gpu


def make(B, Hq, Hkv, D, lens, lmax, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g).to(dtype)
    kc = torch.full((B, lmax, Hkv, D), float("nan"), dtype=dtype)
    vc = torch.full((B, lmax, Hkv, D), float("nan"), dtype=dtype)
    for b, n in enumerate(lens):
        kc[b, :n] = torch.randn((n, Hkv, D), generator=g).to(dtype)
        vc[b, :n] = torch.randn((n, Hkv, D), generator=g).to(dtype)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32)


def call_both(q, kc, vc, lens, splits, dev):
    B, Hq, D = q.shape
    _, lmax, Hkv, _ = kc.shape
    q, kc, vc, lens = q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev)
    dt = _abi.FA_BF16 if q.dtype == torch.bfloat16 else _abi.FA_F16
    scale = f32(D ** -0.5)
    stream = torch.cuda.current_stream(dev).cuda_stream
    o1, l1 = torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device=dev)
    o2, l2 = torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device=dev)
    n = _abi.fa_decode_workspace_size(B, Hq, D, splits)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)  # NaN-filled workspace
    st = _abi.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), o1.data_ptr(),
                        l1.data_ptr(), B, Hq, Hkv, lmax, D, scale, splits, ws.data_ptr(), n, dt,
                        stream)
    assert st == _abi.FA_OK, _abi.fa_last_error()
    st = _abi.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(),
                                o2.data_ptr(), l2.data_ptr(), B, Hq, Hkv, lmax, D, scale, splits,
                                dt, stream)
    assert st == _abi.FA_OK, _abi.fa_last_error()
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu()), scale


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_noalloc_matches_workspace_decode_twice(dtype, gpu):
    cases = [  # first a larger call, then a smaller one that reuses the array
        (16, 32, 8, 128, [8192, 1, 777, 4096, 0, 300, 5000, 2048, 33, 100, 7000, 511, 64, 9, 6000,
                          1234], 8192, 8),
        (3, 8, 2, 64, [5, 0, 300], 300, 3),
    ]
    for i, (B, Hq, Hkv, D, lens, lmax, splits) in enumerate(cases):
        q, kc, vc, lens_t = make(B, Hq, Hkv, D, lens, lmax, dtype, seed=60 + i)
        say(f"noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} splits={splits} {str(dtype)[6:]}")
        (o1, l1), (o2, l2), scale = call_both(q, kc, vc, lens_t, splits, gpu)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {i}: outputs differ"
        o_ref, l_ref = oracle.decode_ref(q, kc, vc, lens_t, scale, workers=16)
        compare(o2, l2, o_ref, l_ref, f"noalloc call {i}")
