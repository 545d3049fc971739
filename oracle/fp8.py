"""FP8 (e4m3) attention forward, in float64 -- the oracle of the fp8 path.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed
----------------
Q, K and V arrive as 8-bit e4m3 codes with one float descale factor each
(the stored value times its descale is the real value).  The oracle decodes
every code exactly to float64, applies the descales, and evaluates the plain
attention definition of ``attention.py`` on the result.  V arrives transposed,
[B, Hkv, D, stride] with keys contiguous per dimension.

Sources (page title, section): "FlashAttention-2 (TH)" (systems-analysis.info),
section on FlashAttention-3: an FP8 variant of the method.  The page fixes
neither the 8-bit format nor the scaling; read here as the OCP e4m3 format (1
sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
subnormal, S.1111.111 is NaN, there is no infinity; largest finite 448) with a
per-tensor descale, the common FP8 inference convention.

``e4m3_decode`` is the format's definition written out.  ``attention_fp8_ref``
also returns, per output element, sum_j P_ij |v_j| (the definition applied to
|V|): a kernel that rounds P to e4m3 (relative error <= 2^-4) is off by at most
2^-4 times that.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_ref


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes (any shape) -> float64 values (NaN codes -> NaN)."""
    if hasattr(codes, "detach"):
        import torch

        codes = codes.detach().to("cpu").view(torch.uint8).numpy()
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def attention_fp8_ref(q8, k8, vt8, Lk: int, scale: float, q_descale: float, k_descale: float,
                      v_descale: float, causal: bool, *, heads=None, workers=None):
    """q8 [B, Lq, Hq, D], k8 [B, Lk, Hkv, D] e4m3 codes; vt8 [B, Hkv, D, S]
    e4m3 codes of V transposed (key j of dimension d at [.., d, j], j < Lk;
    columns past Lk are ignored).  Returns (O [B, Lq, Hq, D], lse [B, Hq, Lq],
    mag [B, Lq, Hq, D] = sum_j P_ij |v_j|), float64."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    vt = e4m3_decode(vt8)[..., :Lk] * float(v_descale)
    v = np.ascontiguousarray(vt.transpose(0, 3, 1, 2))  # [B, Lk, Hkv, D]
    o, lse = attention_ref(q, k, v, scale, causal, heads=heads, workers=workers)
    mag, _ = attention_ref(q, k, np.abs(v), scale, causal, heads=heads, workers=workers)
    return o, lse, mag
