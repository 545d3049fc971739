"""PyTorch-facing wrappers over libfa.  Torch supplies device memory and the
current stream; every step of the computation runs in libfa's HIP kernels.

The argument set follows the usage example of "FlashAttention in the CANN
ops-transformer library" (ai6s.net), section 4: q, k, v in [batch, seq,
heads, head_dim], ``dropout_p`` (only 0.0 is supported: this is the
inference forward), ``softmax_scale`` (default 1/sqrt(head_dim)) and
``is_causal``.
"""

from __future__ import annotations

import math

import torch

from . import _abi

_DTYPES = {torch.float16: _abi.FA_F16, torch.bfloat16: _abi.FA_BF16}


class FAError(RuntimeError):
    """A non-OK status from libfa; ``status`` holds the code."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_abi.STATUS_NAMES.get(status, status)}: {_abi.fa_last_error()}")


def _check_dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, softmax_scale=None,
                   causal: bool = False, dropout_p: float = 0.0, window=(-1, -1), out=None,
                   lse=None):
    """Exact attention forward.  q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] (fp16/bf16).

    Returns (o [B,Lq,Hq,D] in q's dtype, lse [B,Hq,Lq] float32).  Causal
    masking is bottom-right aligned (row i sees keys j <= i + Lk - Lq).
    ``window`` = (left, right) limits row i to keys i+Lk-Lq-left ..
    i+Lk-Lq+right (a negative value leaves that side open).
    """
    if dropout_p != 0.0:
        raise ValueError("dropout_p must be 0.0 (the forward has no dropout)")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D] with equal shapes")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("batch or head_dim mismatch between q and k")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    wl, wr = (int(window[0]), int(window[1]))
    if wl < 0 and wr < 0:
        st = _abi.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, Hq, Hkv, Lq, Lk, D, scale, 1 if causal else 0, _DTYPES[q.dtype],
                         _stream_handle(q.device))
        where = "fa_fwd"
    else:
        st = _abi.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), None, None, B, Hq, Hkv, Lq, Lk, 0, 0, D, scale,
                            1 if causal else 0, wl, wr, _DTYPES[q.dtype], _stream_handle(q.device))
        where = "fa_fwd_ex"
    if st != _abi.FA_OK:
        raise FAError(st, where)
    return out, lse


def _as_bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError(f"{name} must hold e4m3 codes (torch.float8_e4m3fn or uint8)")
    return t


def flash_attn_fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor, *, q_descale: float,
                       k_descale: float, v_descale: float, softmax_scale=None,
                       causal: bool = False, window=(-1, -1), out_dtype=torch.bfloat16, out=None,
                       lse=None):
    """FP8 forward.  q8 [B,Lq,Hq,D], k8 [B,Lk,Hkv,D] e4m3; vt8 [B,Hkv,D,S]
    e4m3 (V transposed, S a multiple of 64 >= Lk, columns past Lk zero).  The
    real values are code * descale.  Returns (o [B,Lq,Hq,D] in out_dtype, lse
    [B,Hq,Lq])."""
    for t, n in ((q8, "q8"), (k8, "k8"), (vt8, "vt8")):
        _check_dev(t, n)
    q8, k8, vt8 = _as_bytes(q8, "q8"), _as_bytes(k8, "k8"), _as_bytes(vt8, "vt8")
    if q8.dim() != 4 or k8.dim() != 4 or vt8.dim() != 4:
        raise ValueError("expected q8 [B,Lq,Hq,D], k8 [B,Lk,Hkv,D], vt8 [B,Hkv,D,S]")
    B, Lq, Hq, D = q8.shape
    Bk, Lk, Hkv, Dk = k8.shape
    if Bk != B or Dk != D or tuple(vt8.shape[:3]) != (B, Hkv, D):
        raise ValueError("shape mismatch between q8, k8 and vt8")
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be float16 or bfloat16")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = torch.empty((B, Lq, Hq, D), dtype=out_dtype, device=q8.device) if out is None else out
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q8.device)
    st = _abi.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), B, Hq, Hkv, Lq, Lk, D, vt8.shape[3], scale,
                         float(q_descale), float(k_descale), float(v_descale),
                         1 if causal else 0, int(window[0]), int(window[1]), _DTYPES[out_dtype],
                         _stream_handle(q8.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return out, lse


def flash_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                   lse: torch.Tensor, dout: torch.Tensor, *, softmax_scale=None,
                   causal: bool = False, window=(-1, -1), dq=None, dk=None, dv=None,
                   workspace=None):
    """Gradients of flash_attn_fwd: returns (dq [B,Lq,Hq,D], dk, dv [B,Lk,Hkv,D])
    in q's dtype from the forward's inputs, its output ``out`` and ``lse``,
    and the output gradient ``dout``.  D in {64, 128, 256}."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse"), (dout, "dout")):
        _check_dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or out.shape != q.shape:
        raise ValueError("expected q, out [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D]")
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout must share dtype float16 or bfloat16")
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, Lq):
        raise ValueError("lse must be float32 [B, Hq, Lq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        n = _abi.fa_bwd_workspace_size(B, Hq, Lq)
        workspace = torch.empty((max(n, 16),), dtype=torch.uint8, device=q.device)
    st = _abi.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Lq,
                     Lk, D, scale, 1 if causal else 0, int(window[0]), int(window[1]),
                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                     _DTYPES[q.dtype], _stream_handle(q.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def flash_attn_varlen_fp8(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                          max_seqlen_q: int, max_seqlen_k: int, *, q_descale: float,
                          k_descale: float, v_descale: float, softmax_scale=None,
                          causal: bool = False, window=(-1, -1), out_dtype=torch.bfloat16,
                          out=None, lse=None):
    """FP8 forward over packed sequences: q8 [total_q,Hq,D], k8 [total_k,Hkv,D]
    e4m3; vt8 [Hkv,D,S] e4m3 (V transposed, key row r of k8 at column r, S a
    multiple of 64 >= total_k + 64, columns past total_k zero); cu_seqlens_*
    int32 [B+1] on the device.  Returns (o [total_q,Hq,D] in out_dtype, lse
    [Hq,total_q])."""
    for t, n in ((q8, "q8"), (k8, "k8"), (vt8, "vt8"), (cu_seqlens_q, "cu_seqlens_q"),
                 (cu_seqlens_k, "cu_seqlens_k")):
        _check_dev(t, n)
    q8, k8, vt8 = _as_bytes(q8, "q8"), _as_bytes(k8, "k8"), _as_bytes(vt8, "vt8")
    if q8.dim() != 3 or k8.dim() != 3 or vt8.dim() != 3:
        raise ValueError("expected q8 [total_q,Hq,D], k8 [total_k,Hkv,D], vt8 [Hkv,D,S]")
    total_q, Hq, D = q8.shape
    total_k, Hkv, Dk = k8.shape
    if Dk != D or tuple(vt8.shape[:2]) != (Hkv, D):
        raise ValueError("shape mismatch between q8, k8 and vt8")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be float16 or bfloat16")
    B = cu_seqlens_q.shape[0] - 1
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = torch.empty((total_q, Hq, D), dtype=out_dtype, device=q8.device) if out is None else out
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q8.device)
    st = _abi.fa_fwd_fp8_ex(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B,
                            Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, D,
                            vt8.shape[2], scale, float(q_descale), float(k_descale),
                            float(v_descale), 1 if causal else 0, int(window[0]), int(window[1]),
                            _DTYPES[out_dtype], _stream_handle(q8.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_fwd_fp8_ex")
    return out, lse


def flash_attn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                      cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                      softmax_scale=None, causal: bool = False, window=(-1, -1), out=None,
                      lse=None):
    """Packed sequences: q [total_q,Hq,D], k/v [total_k,Hkv,D]; cu_seqlens_*
    int32 [B+1] cumulative offsets on the device; each sequence attends only
    to itself.  Returns (o [total_q,Hq,D], lse [Hq,total_q] float32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q"),
                 (cu_seqlens_k, "cu_seqlens_k")):
        _check_dev(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [total_q,Hq,D] and k, v [total_k,Hkv,D]")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D:
        raise ValueError("head_dim mismatch between q and k")
    B = cu_seqlens_q.shape[0] - 1
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    st = _abi.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv,
                        int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, D, scale,
                        1 if causal else 0, int(window[0]), int(window[1]), _DTYPES[q.dtype],
                        _stream_handle(q.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_fwd_ex")
    return out, lse


def flash_attn_varlen_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                          lse: torch.Tensor, dout: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                          softmax_scale=None, causal: bool = False, window=(-1, -1), dq=None,
                          dk=None, dv=None, workspace=None):
    """Gradients of flash_attn_varlen for packed sequences: q, out, dout
    [total_q,Hq,D], k, v [total_k,Hkv,D], lse [Hq,total_q] float32 as the
    forward wrote it.  Returns (dq, dk, dv) in q's dtype.  D in {64, 128, 256}."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse"), (dout, "dout"),
                 (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _check_dev(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or out.shape != q.shape:
        raise ValueError("expected q, out [total_q,Hq,D] and k, v [total_k,Hkv,D]")
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout must share dtype float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D:
        raise ValueError("head_dim mismatch between q and k")
    if lse.dtype != torch.float32 or lse.shape != (Hq, total_q):
        raise ValueError("lse must be float32 [Hq, total_q]")
    B = cu_seqlens_q.shape[0] - 1
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        n = _abi.fa_bwd_workspace_size(B, Hq, int(max_seqlen_q))
        workspace = torch.empty((max(n, 16),), dtype=torch.uint8, device=q.device)
    st = _abi.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                        dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq,
                        Hkv, int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, D, scale,
                        1 if causal else 0, int(window[0]), int(window[1]), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), _DTYPES[q.dtype],
                        _stream_handle(q.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_bwd_ex")
    return dq, dk, dv


def decode_workspace(B: int, Hq: int, D: int, num_splits: int, device) -> torch.Tensor:
    """A byte tensor large enough for fa_decode's workspace."""
    n = _abi.fa_decode_workspace_size(B, Hq, D, num_splits)
    if n == 0:
        raise ValueError("invalid sizes for the decode workspace")
    return torch.empty((n,), dtype=torch.uint8, device=device)


def flash_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      seqlens: torch.Tensor, *, softmax_scale=None, num_splits: int = 8,
                      workspace=None, out=None, lse=None, noalloc: bool = False):
    """One query token per sequence.  q [B,Hq,D]; caches [B,Lk_max,Hkv,D];
    seqlens int32 [B] on the device.  Returns (o [B,Hq,D], lse [B,Hq] float32).
    With ``noalloc`` the call goes to fa_decode_noalloc, whose split partials
    live in the library's fixed device array (no workspace; with ``out`` and
    ``lse`` given, nothing is allocated at all).
    """
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seqlens, "seqlens")):
        _check_dev(t, n)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,D] and k_cache, v_cache [B,Lk_max,Hkv,D]")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype float16 or bfloat16")
    if seqlens.dtype != torch.int32 or seqlens.shape != (q.shape[0],):
        raise ValueError("seqlens must be int32 [B]")
    B, Hq, D = q.shape
    _, Lk_max, Hkv, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D:
        raise ValueError("batch or head_dim mismatch between q and the caches")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        st = _abi.fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                    Lk_max, D, scale, num_splits, _DTYPES[q.dtype],
                                    _stream_handle(q.device))
        if st != _abi.FA_OK:
            raise FAError(st, "fa_decode_noalloc")
        return out, lse
    if workspace is None:
        workspace = decode_workspace(B, Hq, D, num_splits, q.device)
    st = _abi.fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                        out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Lk_max, D, scale, num_splits,
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        _DTYPES[q.dtype], _stream_handle(q.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_decode")
    return out, lse


def flash_attn_decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                            block_table: torch.Tensor, seqlens: torch.Tensor, *, k_scales=None,
                            v_scales=None, softmax_scale=None, num_splits: int = 8,
                            workspace=None, out=None, lse=None):
    """Decode against a paged cache.  q [B,Hq,D]; k_pages, v_pages
    [num_pages, page_size, Hkv, D] in q's dtype, or int8 codes with float32
    scales [num_pages, Hkv, page_size] in k_scales / v_scales; block_table
    int32 [B, max_pages]; seqlens int32 [B].  Returns (o [B,Hq,D], lse [B,Hq])."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                 (seqlens, "seqlens")):
        _check_dev(t, n)
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("expected q [B,Hq,D] and k_pages, v_pages [num_pages,page_size,Hkv,D]")
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float16 or bfloat16")
    fmts = []
    for pages, sc, n in ((k_pages, k_scales, "k"), (v_pages, v_scales, "v")):
        if pages.dtype == torch.int8:
            if sc is None:
                raise ValueError(f"{n}_pages is int8: {n}_scales is required")
            _check_dev(sc, f"{n}_scales")
            want = (pages.shape[0], pages.shape[2], pages.shape[1])
            if sc.dtype != torch.float32 or tuple(sc.shape) != want:
                raise ValueError(f"{n}_scales must be float32 [num_pages, Hkv, page_size]")
            fmts.append(_abi.FA_KV_INT8)
        elif pages.dtype == q.dtype:
            fmts.append(_abi.FA_KV_NATIVE)
        else:
            raise ValueError(f"{n}_pages must be int8 or q's dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [B, max_pages]")
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or block_table.shape[0] != B:
        raise ValueError("head_dim or batch mismatch")
    if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
        raise ValueError("seqlens must be int32 [B]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, D, num_splits, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = _abi.fa_decode_paged(
        q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
        k_scales.data_ptr() if fmts[0] == _abi.FA_KV_INT8 else None,
        v_scales.data_ptr() if fmts[1] == _abi.FA_KV_INT8 else None,
        block_table.data_ptr(), seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, D,
        num_pages, page_size, block_table.shape[1], scale, num_splits, fmts[0], fmts[1],
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _DTYPES[q.dtype],
        _stream_handle(q.device))
    if st != _abi.FA_OK:
        raise FAError(st, "fa_decode_paged")
    return out, lse
