"""fp64 CPU oracle for exact (FlashAttention-style) attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, helpers, headers, constants or pre/post-processing) and
imports nothing from the package ``exact_tiled_attention_fa_amd``.

Contents
--------
``attention.attention_ref``
    The plain definition of softmax attention (scores, mask, row softmax,
    weighted sum of values, per-row logsumexp), evaluated in float64.
``attention.varlen_ref``
    Block-diagonal packing (several sequences in one row range, given by
    cumulative offsets), each attending only to itself; also takes a
    sliding window (left, right) like ``attention_ref``.
``attention.decode_ref``
    The same definition for one query token per sequence against a padded
    KV cache with per-sequence lengths.
``attention.decode_paged_ref``
    Decode against a paged KV cache (page table per sequence), optionally
    with int8 keys and/or values carrying one scale per cached row.
``backward.attention_bwd_ref`` / ``backward.varlen_bwd_ref``
    The gradients of the definition with respect to Q, K and V given dO
    (the chain rule through scores, row softmax and weighted sum), float64;
    the second for sequences packed back to back as in ``varlen_ref``.
``fp8.attention_fp8_ref`` / ``fp8.e4m3_decode``
    The forward on e4m3-coded Q, K and V (transposed) with per-tensor
    descales: exact decoding of the codes, then ``attention_ref``.
``online.online_attention_ref`` / ``online.split_combine_ref``
    The blockwise online-softmax recurrence and the logsumexp merge of
    key-chunk summaries, restated in float64 from the pages.  These are
    checked against ``attention_ref`` (the pages claim the two agree exactly)
    and are never used as the reference for the GPU.

Every function is pinned by tests in ``tests/test_oracle.py`` to things other
than itself: a 40-digit ``decimal`` brute force, PyTorch's fp64 CPU
``scaled_dot_product_attention``, closed forms and invariants.
"""

from .attention import (attention_ref, causal_allowed, decode_paged_ref, decode_ref, key_bounds,
                        varlen_ref)
from .backward import attention_bwd_ref, varlen_bwd_ref
from .fp8 import attention_fp8_ref, e4m3_decode
from .online import online_attention_ref, split_combine_ref

__all__ = [
    "attention_ref",
    "attention_bwd_ref",
    "varlen_bwd_ref",
    "attention_fp8_ref",
    "e4m3_decode",
    "decode_ref",
    "decode_paged_ref",
    "causal_allowed",
    "key_bounds",
    "varlen_ref",
    "online_attention_ref",
    "split_combine_ref",
]
