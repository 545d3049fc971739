"""The benchmark's probes (``_lib/libfa_probe.so``): measurement helpers, not
attention, and not part of libfa's ABI.

Matrix-core probe:
On the MI355X the MFMA rate depends on the values multiplied (operands whose
mantissas toggle draw more power and the clock drops), so the published dense
peak is not reached on random data.  The probe runs only
v_mfma_f32_32x32x16_bf16, in the forward step's chain pattern (one 8-deep
dependent chain and four 2-deep ones per iteration), two 256-thread
workgroups per compute unit, with its operands read once from a given buffer:
timed on a workload's own data it gives the matrix cores' rate for that data.
"""

from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_P, _Z, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_lib = None


def lib_path() -> Path:
    return Path(__file__).resolve().parent / "_lib" / "libfa_probe.so"


def load():
    global _lib
    if _lib is None:
        p = lib_path()
        if not p.exists():
            raise RuntimeError(f"{p} is missing: build it first (__graft_entry__.build())")
        lib = ctypes.CDLL(str(p))
        lib.fa_probe_mfma_out_len.restype = _Z
        lib.fa_probe_mfma_out_len.argtypes = []
        lib.fa_probe_mfma_bf16.restype = _I
        lib.fa_probe_mfma_bf16.argtypes = [_P, _Z, _P, _Z, _I, ctypes.POINTER(ctypes.c_double), _P]
        for fn in (lib.fa_probe_rates, lib.fa_probe_rates_vgpr):
            fn.restype = _I
            fn.argtypes = [_I, _P, _Z, _P, _P, _I, _I, _I, _P]
        _lib = lib
    return _lib


def out_len() -> int:
    return int(load().fa_probe_mfma_out_len())


def mfma_probe(operands: torch.Tensor, iters: int, out=None):
    """One launch on the current stream over the bytes of ``operands`` (a
    contiguous GPU tensor, read as bf16, size a multiple of 16 bytes).  Returns
    (out, flops): each thread's accumulator sum (float32, exactly 4096 * iters
    when every operand is 1.0) and the flops the launch executes."""
    if not operands.is_cuda or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous GPU tensor")
    n = out_len()
    if n == 0:
        raise RuntimeError("fa_probe_mfma_out_len: the device cannot be queried")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=operands.device)
    if out.dtype != torch.float32 or not out.is_cuda:
        raise ValueError("out must be a float32 GPU tensor")
    flops = ctypes.c_double(0.0)
    stream = torch.cuda.current_stream(operands.device).cuda_stream
    st = load().fa_probe_mfma_bf16(operands.data_ptr(), operands.numel() * operands.element_size(),
                                   out.data_ptr(), out.numel(), int(iters), ctypes.byref(flops),
                                   ctypes.c_void_p(stream))
    if st != 0:
        raise RuntimeError(f"fa_probe_mfma_bf16 returned {st}")
    return out, flops.value


# Instruction mixes of fa_probe_rates (csrc/probe/rate_probe.hip), and the
# instructions one iteration of each issues per wave.
RATE_MIXES = {
    "mfma_chain8": (0, "8 dependent 32x32x16 bf16 MFMAs"),
    "mfma_4x2": (1, "8 MFMAs in four independent chains"),
    "fma32": (2, "32 independent v_fma_f32"),
    "exp32": (3, "32 independent v_exp_f32"),
    "mfma_4fma": (4, "8 MFMAs (four chains), 4 v_fma_f32 after each"),
    "mfma_2exp": (5, "8 MFMAs (four chains), 2 v_exp_f32 after each"),
    "split_mfma_fma": (6, "per SIMD one wave of 8 MFMAs (four chains), one of 32 v_fma_f32"),
    "split_mfma_exp": (7, "per SIMD one wave of 8 MFMAs (four chains), one of 32 v_exp_f32"),
    "mfma_softmax": (8, "8 MFMAs (four chains), after each 2 fma, 2 exp, 2 add, 1 cvt, 1 xor"),
    "step16": (9, "16 MFMAs (a chain of 8, two chains of 4) with 16 fma, 16 exp, 16 add, 8 cvt, "
                  "8 xor interleaved, 4 VALU after each MFMA"),
}


def rates(operands: torch.Tensor, waves_per_simd: int, iters: int = 4096, cus: int = 256,
          vgpr_acc: bool = False):
    """Cycles per iteration of every mix with ``waves_per_simd`` (1 or 2)
    waves on every SIMD: one workgroup of 4 * waves_per_simd waves per compute
    unit.  For each SIMD (identified by the waves' hardware ids) its span runs
    from its waves' first loop start to their last loop end (s_memtime, the
    shader clock); ``simd_cycles_per_iter`` is the median span / iters, so
    with two waves per SIMD it covers both waves' iterations.  The shader
    clock's rate over the loops is converted with the 100 MHz s_memrealtime.
    Split mixes also report each half's own loop time."""
    if not operands.is_cuda or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous GPU tensor")
    nw = cus * 4 * waves_per_simd
    out = torch.empty(64 * nw, dtype=torch.float32, device=operands.device)
    rec = torch.empty((nw, 5), dtype=torch.int64, device=operands.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(operands.device).cuda_stream)
    res = {}
    for name, (mix, about) in RATE_MIXES.items():
        if name.startswith("split") and waves_per_simd != 2:
            continue
        fn = load().fa_probe_rates_vgpr if vgpr_acc else load().fa_probe_rates
        for _ in range(2):  # the first launch warms the clocks and caches
            st = fn(mix, operands.data_ptr(), operands.numel() * operands.element_size(),
                    out.data_ptr(), rec.data_ptr(), cus, waves_per_simd, int(iters), stream)
            if st != 0:
                raise RuntimeError(f"fa_probe_rates({name}) returned {st}")
        torch.cuda.synchronize()
        r = rec.cpu()
        t0, t1, r0, r1, hwid = (r[:, i] for i in range(5))
        mhz = float(((t1 - t0).double() / (r1 - r0).double()).median()) * 100.0
        simd = (hwid >> 4) & 0x3
        blk = torch.arange(nw) // (4 * waves_per_simd)
        key = blk * 4 + simd
        spans, counts = [], []
        for k_ in torch.unique(key):
            sel = key == k_
            counts.append(int(sel.sum()))
            spans.append(float(t1[sel].max() - t0[sel].min()))
        spans = torch.tensor(spans, dtype=torch.float64)
        entry = {"about": about, "shader_mhz": round(mhz, 1),
                 "waves_per_simd_seen": sorted(set(counts)),
                 "simd_cycles_per_iter": round(float(spans.median()) / iters, 1)}
        if name.startswith("split"):
            w = torch.arange(nw) % (4 * waves_per_simd)
            own = (t1 - t0).double() / iters
            entry["mfma_wave_cycles_per_iter"] = round(float(own[w < 4].median()), 1)
            entry["valu_wave_cycles_per_iter"] = round(float(own[w >= 4].median()), 1)
        res[name] = entry
    return res
