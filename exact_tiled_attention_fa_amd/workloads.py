"""Seeded synthetic inputs shaped like the pages' attention workloads.

This module only draws numbers; it holds none of the attention arithmetic,
so both the oracle side and the GPU side of a test may use it.  Everything is
drawn on the CPU with ``torch.Generator(device="cpu")`` (bitwise reproducible
anywhere) as float32 N(0,1), in the order Q, K, V, then cast to the workload's
dtype with round-to-nearest-even.

Workloads (the numbered configurations of the prefill / decode envelope):
  tiny       B=1  H=2        L=128    D=64  fp16 bidirectional, scale 1/8
  llama7b    B=4  Hq=Hkv=32  L=4096   D=128 bf16 causal   (Llama-2-7B shape)
  gqa16k     B=1  Hq=32 Hkv=8 L=16384 D=128 bf16 causal   (long-context GQA)
  d256       B=2  Hq=Hkv=16  L=4096   D=256 fp16 causal
  encoder    B=64 H=12       L=512    D=64  fp16 bidirectional, 1% of key rows x8
  decode     B=128 Hq=32 Hkv=8 D=128 bf16, one query token per sequence,
             cache lengths uniform on [512, 8192], 8 splits
Structured-mask prefill (sliding window, packed sequences):
  swa16k     B=2 Hq=32 Hkv=8 L=16384 D=128 bf16 causal, window (4095, 0):
             each row sees its last 4096 keys (a Mistral-7B-style local window)
  varlen16   16 packed sequences, lengths uniform on [256, 4096], Hq=32
             Hkv=8 D=128 bf16 causal (a packed serving prefill batch)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    dtype: torch.dtype
    causal: bool
    seed: int
    outlier_frac: float = 0.0  # fraction of key rows scaled by outlier_mult
    outlier_mult: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def flops(self) -> int:
        """Algorithmic FLOPs: 4*D per allowed (query, key) pair per query head."""
        pairs = self.L * (self.L + 1) // 2 if self.causal else self.L * self.L
        return 4 * self.D * pairs * self.B * self.Hq

    def hbm_bytes(self) -> int:
        """Algorithmic bytes: Q, K, V read once; O and lse written once."""
        e = 2
        q = self.B * self.L * self.Hq * self.D * e
        kv = 2 * self.B * self.L * self.Hkv * self.D * e
        return 2 * q + kv + self.B * self.Hq * self.L * 4


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    len_lo: int
    len_hi: int  # inclusive
    num_splits: int
    seed: int
    Lk_max: int = field(default=0)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def lmax(self) -> int:
        return self.Lk_max or self.len_hi


@dataclass(frozen=True)
class Masked:
    """Prefill under a structured mask.  Each sequence has equal query and key
    length.  ``packed`` False: a dense batch of equal lengths; True: the
    sequences are packed back to back with cumulative offsets."""
    name: str
    nseq: int
    len_lo: int
    len_hi: int  # inclusive; len_lo == len_hi gives equal lengths
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    causal: bool
    window: tuple
    packed: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def lengths(self) -> list:
        if self.len_lo == self.len_hi:
            return [self.len_lo] * self.nseq
        g = _gen(self.seed)
        return [int(x) for x in torch.randint(self.len_lo, self.len_hi + 1, (self.nseq,),
                                                  generator=g, dtype=torch.int64)]

    def pairs(self) -> int:
        """(query, key) pairs the mask allows, summed over the sequences."""
        left, right = self.window
        total = 0
        for n in self.lengths():
            i = torch.arange(n, dtype=torch.int64)
            lo = torch.zeros_like(i) if left < 0 else (i - left).clamp(min=0)
            hi = torch.full_like(i, n - 1)
            if self.causal:
                hi = torch.minimum(hi, i)
            if right >= 0:
                hi = torch.minimum(hi, i + right)
            total += int((hi - lo + 1).clamp(min=0).sum())
        return total

    def flops(self) -> int:
        return 4 * self.D * self.Hq * self.pairs()

    def hbm_bytes(self) -> int:
        """Algorithmic bytes: Q, K, V read once; O and lse written once."""
        n = sum(self.lengths())
        e = 2
        return 2 * n * self.Hq * self.D * e + 2 * n * self.Hkv * self.D * e + n * self.Hq * 4


PREFILL = {
    "tiny": Prefill("tiny", 1, 2, 2, 128, 64, torch.float16, False, 1),
    "llama7b": Prefill("llama7b", 4, 32, 32, 4096, 128, torch.bfloat16, True, 2),
    "gqa16k": Prefill("gqa16k", 1, 32, 8, 16384, 128, torch.bfloat16, True, 3),
    "d256": Prefill("d256", 2, 16, 16, 4096, 256, torch.float16, True, 31),
    "encoder": Prefill("encoder", 64, 12, 12, 512, 64, torch.float16, False, 4, 0.01, 8.0),
}
MASKED = {
    "swa16k": Masked("swa16k", 2, 16384, 16384, 32, 8, 128, torch.bfloat16, True, (4095, 0),
                     False, 6),
    "varlen16": Masked("varlen16", 16, 256, 4096, 32, 8, 128, torch.bfloat16, True, (-1, -1),
                       True, 7),
}
DECODE = {
    "decode": Decode("decode", 128, 32, 8, 128, torch.bfloat16, 512, 8192, 8, 5),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def randn_qkv(B, Lq, Lk, Hq, Hkv, D, dtype, seed, *, outlier_frac=0.0, outlier_mult=8.0,
              q_scale=1.0):
    """Q [B,Lq,Hq,D], K/V [B,Lk,Hkv,D] on the CPU in ``dtype``.

    Draw order: Q, K, V (float32 N(0,1)); then, if ``outlier_frac`` > 0, a
    Bernoulli(outlier_frac) mask over key rows (b, j, kv head) whose K vectors
    are multiplied by ``outlier_mult`` in float32; then the casts.
    """
    g = _gen(seed)
    q = torch.randn((B, Lq, Hq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    if outlier_frac > 0:
        rows = torch.rand((B, Lk, Hkv), generator=g) < outlier_frac
        k[rows] *= outlier_mult
    if q_scale != 1.0:
        q *= q_scale
    return q.to(dtype), k.to(dtype), v.to(dtype)


def prefill_inputs(cfg: Prefill):
    return randn_qkv(cfg.B, cfg.L, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.dtype, cfg.seed,
                     outlier_frac=cfg.outlier_frac, outlier_mult=cfg.outlier_mult)


def masked_inputs(cfg: Masked):
    """Dense: (q [B,L,Hq,D], k, v [B,L,Hkv,D], None).  Packed: (q [total,Hq,D],
    k, v [total,Hkv,D], cu_seqlens int32 [nseq+1]).  Draw order: the lengths
    (packed only, from the seed), then Q, K, V as float32 N(0,1) from a
    generator seeded with seed + 1, then the casts."""
    lens = cfg.lengths()
    g = _gen(cfg.seed + 1)
    if cfg.packed:
        n = sum(lens)
        q = torch.randn((n, cfg.Hq, cfg.D), generator=g, dtype=torch.float32)
        k = torch.randn((n, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32)
        v = torch.randn((n, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32)
        cu = torch.tensor([0] + lens, dtype=torch.int64).cumsum(0).to(torch.int32)
        return q.to(cfg.dtype), k.to(cfg.dtype), v.to(cfg.dtype), cu
    L = lens[0]
    q = torch.randn((cfg.nseq, L, cfg.Hq, cfg.D), generator=g, dtype=torch.float32)
    k = torch.randn((cfg.nseq, L, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32)
    v = torch.randn((cfg.nseq, L, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32)
    return q.to(cfg.dtype), k.to(cfg.dtype), v.to(cfg.dtype), None


FP8_MULT = 16.0  # codes hold 16 x N(0,1) (|x| well inside e4m3's 448); descale 1/16


def fp8_inputs(B, Lq, Lk, Hq, Hkv, D, seed, *, q_scale=1.0):
    """e4m3 codes as uint8: q8 [B,Lq,Hq,D], k8 [B,Lk,Hkv,D] and vt8
    [B,Hkv,D,S] (V transposed, S = Lk rounded up to 64, zero columns past Lk),
    plus the descale 1/16 of each.  Draw order: Q, K, V as float32 N(0,1)
    (Q times q_scale), each times 16 and cast to e4m3 with round-to-nearest-
    even."""
    g = _gen(seed)
    q = torch.randn((B, Lq, Hq, D), generator=g, dtype=torch.float32) * q_scale
    k = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    cast = lambda x: (x * FP8_MULT).to(torch.float8_e4m3fn).view(torch.uint8)
    S = (Lk + 63) // 64 * 64
    vt = torch.zeros((B, Hkv, D, S), dtype=torch.uint8)
    vt[..., :Lk] = cast(v).permute(0, 2, 3, 1)
    return cast(q), cast(k), vt, 1.0 / FP8_MULT


def fp8_varlen_inputs(total_q, total_k, Hq, Hkv, D, seed, *, q_scale=1.0):
    """Packed e4m3 codes as uint8: q8 [total_q,Hq,D], k8 [total_k,Hkv,D] and
    vt8 [Hkv,D,S] (V transposed, key row r at column r, S = total_k + 64
    rounded up to 64, zero columns past total_k), plus the descale 1/16 of
    each.  Draw order and casts as fp8_inputs."""
    g = _gen(seed)
    q = torch.randn((total_q, Hq, D), generator=g, dtype=torch.float32) * q_scale
    k = torch.randn((total_k, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((total_k, Hkv, D), generator=g, dtype=torch.float32)
    cast = lambda x: (x * FP8_MULT).to(torch.float8_e4m3fn).view(torch.uint8)
    S = (total_k + 64 + 63) // 64 * 64
    vt = torch.zeros((Hkv, D, S), dtype=torch.uint8)
    vt[..., :total_k] = cast(v).permute(1, 2, 0)
    return cast(q), cast(k), vt, 1.0 / FP8_MULT


def decode_lengths(cfg: Decode) -> torch.Tensor:
    """Per-sequence cache lengths, uniform on [len_lo, len_hi], int32 [B]."""
    g = _gen(cfg.seed)
    return torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.B,), generator=g, dtype=torch.int64).to(
        torch.int32)


def decode_inputs(cfg: Decode, *, pad_value=float("nan")):
    """(q [B,Hq,D], k_cache, v_cache [B,Lk_max,Hkv,D], seqlens int32 [B]) on the CPU.

    Draw order: lengths, Q, then for b = 0..B-1 the K rows then the V rows of
    sequence b ([len_b, Hkv, D]).  Cache rows past len_b hold ``pad_value``
    (NaN by default, so that any read of padding shows up in the output).
    """
    g = _gen(cfg.seed)
    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.B,), generator=g, dtype=torch.int64)
    q = torch.randn((cfg.B, cfg.Hq, cfg.D), generator=g, dtype=torch.float32).to(cfg.dtype)
    lmax = cfg.lmax
    kc = torch.full((cfg.B, lmax, cfg.Hkv, cfg.D), pad_value, dtype=cfg.dtype)
    vc = torch.full((cfg.B, lmax, cfg.Hkv, cfg.D), pad_value, dtype=cfg.dtype)
    for b in range(cfg.B):
        n = int(lens[b])
        kc[b, :n] = torch.randn((n, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32).to(cfg.dtype)
        vc[b, :n] = torch.randn((n, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32).to(cfg.dtype)
    return q, kc, vc, lens.to(torch.int32)


def _kv_side(n, cfg: Decode, g, int8: bool):
    """n cached rows [n, Hkv, D] of one side: N(0,1) in cfg.dtype, or int8
    codes round(45 * N(0,1)) clipped to [-127, 127] with float32 scales drawn
    uniform on [0.018, 0.026] per (row, head) -- about the codes and scales a
    symmetric per-row int8 quantiser gives for N(0,1) rows of 128 values."""
    x = torch.randn((n, cfg.Hkv, cfg.D), generator=g, dtype=torch.float32)
    if not int8:
        return x.to(cfg.dtype), None
    codes = torch.round(x * 45.0).clamp(-127, 127).to(torch.int8)
    scales = torch.rand((n, cfg.Hkv), generator=g, dtype=torch.float32) * 0.008 + 0.018
    return codes, scales


def paged_decode_inputs(cfg: Decode, page_size: int, *, k_int8=False, v_int8=False,
                        extra_pages=4):
    """A paged decode cache on the CPU: (q [B,Hq,D], k_pages, v_pages
    [num_pages, page_size, Hkv, D], k_scales, v_scales (float32
    [num_pages, Hkv, page_size] or None), block_table int32 [B, max_pages],
    seqlens int32 [B]).

    Draw order: lengths, Q, a permutation of the physical pages, then for
    b = 0..B-1 sequence b's K rows then V rows (int8 sides: codes, then
    scales).  Sequence b's pages are the next ceil(len_b / page_size) pages of
    the permutation.  Rows no sequence owns -- unused pages, slots past a
    sequence's end, and the page that table entries past a sequence's end
    point at -- hold NaN (int8 sides: code 127 with a NaN scale), so any read
    of them shows in the output.
    """
    g = _gen(cfg.seed)
    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.B,), generator=g, dtype=torch.int64)
    q = torch.randn((cfg.B, cfg.Hq, cfg.D), generator=g, dtype=torch.float32).to(cfg.dtype)
    need = [(int(n) + page_size - 1) // page_size for n in lens]
    max_pages = max(1, (cfg.lmax + page_size - 1) // page_size)
    num_pages = sum(need) + extra_pages
    perm = torch.randperm(num_pages, generator=g)
    junk = int(perm[-1])
    table = torch.full((cfg.B, max_pages), junk, dtype=torch.int32)

    def pool(int8):
        if int8:
            return (torch.full((num_pages, page_size, cfg.Hkv, cfg.D), 127, dtype=torch.int8),
                    torch.full((num_pages, cfg.Hkv, page_size), float("nan"), dtype=torch.float32))
        return torch.full((num_pages, page_size, cfg.Hkv, cfg.D), float("nan"), dtype=cfg.dtype), None

    kp, ks = pool(k_int8)
    vp, vs = pool(v_int8)
    nxt = 0
    for b in range(cfg.B):
        n = int(lens[b])
        pages = perm[nxt:nxt + need[b]]
        nxt += need[b]
        table[b, :need[b]] = pages.to(torch.int32)
        for pool_x, pool_s, (x, xs) in ((kp, ks, _kv_side(n, cfg, g, k_int8)),
                                         (vp, vs, _kv_side(n, cfg, g, v_int8))):
            full, rest = divmod(n, page_size)
            if full:
                pool_x[pages[:full]] = x[:full * page_size].reshape(full, page_size, cfg.Hkv, cfg.D)
                if xs is not None:
                    pool_s[pages[:full]] = xs[:full * page_size].reshape(
                        full, page_size, cfg.Hkv).transpose(1, 2)
            if rest:
                pool_x[int(pages[full]), :rest] = x[full * page_size:]
                if xs is not None:
                    pool_s[int(pages[full]), :, :rest] = xs[full * page_size:].T
    return q, kp, vp, ks, vs, table, lens.to(torch.int32)


def paged_decode_bytes(cfg: Decode, lens, page_size: int, *, k_int8=False, v_int8=False) -> int:
    """Algorithmic HBM bytes of one paged decode step: every cached row of
    every sequence read once (2 bytes per element, or 1 plus a 4-byte scale
    per row for an int8 side), the table entries of the used pages (4 bytes
    each), q read once, o and lse written once."""
    lens = [int(x) for x in lens]
    rows = sum(lens) * cfg.Hkv
    side = lambda i8: rows * (cfg.D + 4) if i8 else rows * cfg.D * 2
    entries = sum((n + page_size - 1) // page_size for n in lens)
    return (side(k_int8) + side(v_int8) + 4 * entries + 2 * cfg.B * cfg.Hq * cfg.D * 2
            + cfg.B * cfg.Hq * 4)


def decode_bytes(cfg: Decode, lens) -> int:
    """Algorithmic HBM bytes of one decode step: the K and V rows of every
    sequence's cache read once, q read once, o and lse written once."""
    e = 2
    kv = int(sum(int(x) for x in lens)) * cfg.Hkv * cfg.D * e * 2
    return kv + 2 * cfg.B * cfg.Hq * cfg.D * e + cfg.B * cfg.Hq * 4


def decode_flops(cfg: Decode, lens) -> int:
    return int(sum(int(x) for x in lens)) * 4 * cfg.Hq * cfg.D
