"""Pins of the oracle's fp8 path (CPU only): the e4m3 decoder against values
the format fixes and against PyTorch's float8_e4m3fn, and the fp8 forward
against the (separately pinned) definition on decoded inputs."""

from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
from pins import assert_close

# code -> value fixed by the format (sign, 4-bit exponent with bias 7, 3-bit mantissa)
KNOWN = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x39: 1.125, 0x3F: 1.875,
         0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9,
         0x30: 0.5, 0x4A: 5.0}


def pin_known_codes(dec):
    for c, v in KNOWN.items():
        got = float(dec(np.array([c], dtype=np.uint8))[0])
        assert got == v and np.signbit(got) == np.signbit(v), f"code {c:#x}: {got} != {v}"
    assert np.isnan(dec(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def pin_all_codes_vs_torch(dec):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = dec(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"codes differ: {np.nonzero(~same)[0][:8]}"


def pin_monotone(dec):
    pos = dec(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert_close(dec(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos, 0.0, "negative codes")


DEC_PINS = [pin_known_codes, pin_all_codes_vs_torch, pin_monotone]


@pytest.mark.parametrize("pin", DEC_PINS, ids=lambda p: p.__name__)
def test_decoder_pin(pin):
    pin(oracle.e4m3_decode)


DEC_MUTATIONS = {
    "bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "no_implicit_one": ("(1.0 + m / 8.0)", "(m / 8.0)"),
    "subnormal_scale": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "mantissa_bits": ("m = c & 0x7", "m = c & 0x3"),
}


@pytest.mark.parametrize("name", sorted(DEC_MUTATIONS))
def test_planted_mistake_in_decoder_is_caught(name):
    old, new = DEC_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(ofp8.e4m3_decode))
    assert old in src
    ns = dict(vars(ofp8))
    exec(compile(src.replace(old, new), "<m>", "exec"), ns)
    failed = []
    for pin in DEC_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns["e4m3_decode"])
        except AssertionError:
            failed.append(pin.__name__)
    assert failed


def codes(shape, seed, mult):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_forward_is_the_definition_on_decoded_inputs():
    B, Lq, Lk, Hq, Hkv, D, S = 2, 9, 11, 4, 2, 8, 16
    q8, k8 = codes((B, Lq, Hq, D), 1, 16.0), codes((B, Lk, Hkv, D), 2, 16.0)
    vt8 = codes((B, Hkv, D, S), 3, 16.0)
    vt8[..., Lk:] = 0x7F  # NaN padding past Lk must be ignored
    for causal in (False, True):
        o, lse, mag = oracle.attention_fp8_ref(q8, k8, vt8, Lk, 0.35, 1 / 16, 1 / 16, 1 / 8, causal)
        q = torch.from_numpy(q8).view(torch.float8_e4m3fn).double().numpy() / 16
        k = torch.from_numpy(k8).view(torch.float8_e4m3fn).double().numpy() / 16
        vt = torch.from_numpy(np.ascontiguousarray(vt8[..., :Lk])).view(
            torch.float8_e4m3fn).double().numpy() / 8
        v = vt.transpose(0, 3, 1, 2)
        o2, l2 = oracle.attention_ref(q, k, v, 0.35, causal)
        assert_close(o, o2, 0.0, "fp8 O")
        assert_close(lse, l2, 0.0, "fp8 lse")
        m2, _ = oracle.attention_ref(q, k, np.abs(v), 0.35, causal)
        assert_close(mag, m2, 0.0, "fp8 mag")
        assert np.all(np.abs(o) <= mag + 1e-12)
