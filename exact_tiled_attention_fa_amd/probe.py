"""The benchmark's matrix-core probe (``_lib/libfa_probe.so``): a measurement
helper, not attention, and not part of libfa's ABI.

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
