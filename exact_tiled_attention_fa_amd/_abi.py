"""ctypes binding of libfa's C ABI (include/fa.h), same names, marshalling only.

The library is loaded on first use from ``_lib/libfa.so`` next to this file
(override with the environment variable ``FA_GFX950_LIB``).  If it is missing
every call raises -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3

FA_F16 = 0
FA_BF16 = 1

FA_KV_NATIVE = 0
FA_KV_INT8 = 1

STATUS_NAMES = {
    FA_OK: "FA_OK",
    FA_ERR_INVALID_ARGUMENT: "FA_ERR_INVALID_ARGUMENT",
    FA_ERR_UNSUPPORTED: "FA_ERR_UNSUPPORTED",
    FA_ERR_HIP: "FA_ERR_HIP",
}

# Every symbol include/fa.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                       _I, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _F, _F, _I, _I, _I,
                        _I, _P]),
    "fa_fwd_fp8_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _F,
                           _F, _F, _I, _I, _I, _I, _P]),
    "fa_decode_workspace_size": (_Z, [_I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _I, _P]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                             _I, _I, _I, _P, _Z, _I, _P]),
    "fa_bwd_workspace_size": (_Z, [_I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P,
                    _Z, _I, _P]),
    "fa_bwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                       _F, _I, _I, _I, _P, _Z, _I, _P]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_info": (ctypes.c_char_p, []),
}

_lib = None


def lib_path() -> Path:
    env = os.environ.get("FA_GFX950_LIB")
    if env:
        return Path(env)
    return Path(__file__).resolve().parent / "_lib" / "libfa.so"


def load() -> ctypes.CDLL:
    """Load libfa.so once and attach the C signatures; raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not path.exists():
        raise RuntimeError(
            f"libfa.so not found at {path}; build it first with "
            "`python -m exact_tiled_attention_fa_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(str(path))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype, stream) -> int:
    """Raw C call; pointers are ints (device addresses), returns the status."""
    return load().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype, stream)


def fa_fwd_ex(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Lq, Lk, total_q, total_k,
              D, scale, causal, window_left, window_right, dtype, stream) -> int:
    return load().fa_fwd_ex(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Lq, Lk,
                            total_q, total_k, D, scale, causal, window_left, window_right, dtype,
                            stream)


def fa_fwd_fp8(q8, k8, vt8, o, lse, B, Hq, Hkv, Lq, Lk, D, vt_stride, scale, q_descale, k_descale,
               v_descale, causal, window_left, window_right, out_dtype, stream) -> int:
    return load().fa_fwd_fp8(q8, k8, vt8, o, lse, B, Hq, Hkv, Lq, Lk, D, vt_stride, scale,
                             q_descale, k_descale, v_descale, causal, window_left, window_right,
                             out_dtype, stream)


def fa_fwd_fp8_ex(q8, k8, vt8, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Lq, Lk, total_q,
                  total_k, D, vt_stride, scale, q_descale, k_descale, v_descale, causal,
                  window_left, window_right, out_dtype, stream) -> int:
    return load().fa_fwd_fp8_ex(q8, k8, vt8, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Lq,
                                Lk, total_q, total_k, D, vt_stride, scale, q_descale, k_descale,
                                v_descale, causal, window_left, window_right, out_dtype, stream)


def fa_decode_workspace_size(B, Hq, D, num_splits) -> int:
    return load().fa_decode_workspace_size(B, Hq, D, num_splits)


def fa_decode(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale, num_splits,
              workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_decode(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale,
                            num_splits, workspace, workspace_bytes, dtype, stream)


def fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D, scale,
                      num_splits, dtype, stream) -> int:
    return load().fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lk_max, D,
                                    scale, num_splits, dtype, stream)


def fa_decode_paged(q, k_pages, v_pages, k_scales, v_scales, block_table, seqlens, o, lse, B, Hq,
                    Hkv, D, num_pages, page_size, max_pages, scale, num_splits, k_format, v_format,
                    workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_decode_paged(q, k_pages, v_pages, k_scales, v_scales, block_table, seqlens, o,
                                  lse, B, Hq, Hkv, D, num_pages, page_size, max_pages, scale,
                                  num_splits, k_format, v_format, workspace, workspace_bytes,
                                  dtype, stream)


def fa_bwd_workspace_size(B, Hq, Lq) -> int:
    return load().fa_bwd_workspace_size(B, Hq, Lq)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal, window_left,
           window_right, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                         window_left, window_right, workspace, workspace_bytes, dtype, stream)


def fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, Lq, Lk,
              total_q, total_k, D, scale, causal, window_left, window_right, workspace,
              workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, Hq,
                            Hkv, Lq, Lk, total_q, total_k, D, scale, causal, window_left,
                            window_right, workspace, workspace_bytes, dtype, stream)


def fa_last_error() -> str:
    return (load().fa_last_error() or b"").decode()


def fa_info() -> str:
    return (load().fa_info() or b"").decode()
