"""Exact tiled attention (FlashAttention forward + split-KV decode) for MI355X.

The compute lives in ``libfa.so`` (hand-written HIP for gfx950, C ABI in
``include/fa.h``).  ``_abi`` binds that ABI with ctypes under the same names;
``attention`` adds thin PyTorch wrappers.  ``workloads`` holds the seeded
synthetic input generators.
"""

from . import _abi
from ._abi import (fa_bwd, fa_bwd_ex, fa_bwd_workspace_size, fa_decode, fa_decode_paged,
                   fa_decode_workspace_size, fa_fwd, fa_fwd_ex, fa_fwd_fp8, fa_fwd_fp8_ex,
                   fa_info, fa_last_error)

__all__ = [
    "fa_fwd",
    "fa_fwd_ex",
    "fa_fwd_fp8",
    "fa_fwd_fp8_ex",
    "fa_bwd",
    "fa_bwd_ex",
    "fa_bwd_workspace_size",
    "fa_decode",
    "fa_decode_paged",
    "fa_decode_workspace_size",
    "fa_info",
    "fa_last_error",
    "flash_attn_fwd",
    "flash_attn_bwd",
    "flash_attn_varlen_bwd",
    "flash_attn_fwd_fp8",
    "flash_attn_varlen_fp8",
    "flash_attn_decode",
    "flash_attn_decode_paged",
    "flash_attn_varlen",
    "decode_workspace",
]


def __getattr__(name):  # torch-facing wrappers are imported lazily
    if name in ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_varlen_bwd", "flash_attn_fwd_fp8",
                "flash_attn_varlen_fp8", "flash_attn_varlen", "flash_attn_decode",
                "flash_attn_decode_paged",
                "decode_workspace", "FAError"):
        from . import attention

        return getattr(attention, name)
    raise AttributeError(name)
