"""Plain softmax attention in float64 -- the oracle's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
For batch b, query head h, key/value head kv = floor(h / (Hq / Hkv)) and query
row i:

  s_ij   = scale * sum_d q[b,i,h,d] * k[b,j,kv,d]              (scaled scores)
  A_i    = { j : not causal  or  j <= i + (Lk - Lq) }          (allowed keys)
  m_i    = max_{j in A_i} s_ij
  l_i    = sum_{j in A_i} exp(s_ij - m_i)
  P_ij   = exp(s_ij - m_i) / l_i  on A_i,  0 elsewhere
  O[b,i,h,:] = sum_j P_ij * v[b,j,kv,:]
  lse[b,h,i] = m_i + ln l_i                                   (natural log)
  A_i empty  ->  O = 0, lse = -inf

Sources (page title, section):
* "FlashAttention in the CANN ops-transformer library" (ai6s.net), section 1:
  the standard computation materialises Q K^T and its softmax (O(N^2)); the
  method tiles it and must give the same result (section 2, step 2).
* same page, section 2 step 3: an output O and a per-row normaliser L are
  produced.  Read here as L = the per-row logsumexp of the scaled scores over
  the allowed keys, natural log, laid out [B, Hq, Lq].
* same page, section 4 (usage): arguments q, k, v in [batch, seq, heads,
  head_dim] layout, ``softmax_scale`` defaulting to 1/sqrt(head_dim),
  ``is_causal``; section 5: causal keys "above the diagonal" take no part in
  the softmax (their probability is 0; the page's "scores set to zero" is read
  as probabilities zero, since it also says they leave the softmax), and
  bidirectional (BERT-style) use has no mask.
* "Enable Flash Attention with llama.cpp" (qualllm.com), FAQ on GQA, and
  "MNN LLM attention_mode" (lpnh.cn), section on choosing a mode: K/V heads
  shared by groups of query heads (group 1/2/4/8).  Read as consecutive query
  heads sharing one K/V head.
* Causal alignment when Lq != Lk is not on the pages; read as bottom-right
  (the last query row sees every key), which equals the usual lower triangle
  when Lq == Lk and makes a one-token decode see its whole cache.
* "5 years, 10K stars: xformers" (cloud.tencent.com) lists structured masks
  that spare the kernel a dense mask read: causal, local (sliding window) and
  block-diagonal (several sequences packed into one batch row).  Read here as
  a window (left, right): row i sees keys j with i + shift - left <= j <=
  i + shift + right, a negative bound meaning unbounded on that side (causal
  additionally caps j <= i + shift); and block-diagonal packing as sequences
  given by cumulative offsets cu_q / cu_k, each attending only to itself.

* "FlashAttention-2 (TH)" (systems-analysis.info), references, cite
  PagedAttention: a KV cache kept in fixed-size pages reached through a
  per-sequence page table.  Read here as pages [num_pages, P, Hkv, D] and a
  table [B, max_pages]: key j of sequence b is slot j % P of page
  table[b, j // P].
* "MNN LLM attention_mode" (lpnh.cn), encoding section: KV-cache modes with
  the keys, or the keys and the values, stored as int8.  The page gives no
  quantiser; read here as a symmetric int8 code with one float scale per
  cached row (page, slot, kv head), the cached value being code * scale; the
  scales are laid out [num_pages, Hkv, P].

Implementation notes: each (b, h) pair is independent; rows are processed in
blocks of ``row_block`` so that at most row_block x Lk scores exist at once.
That is still the plain definition -- each row's max, sum and weighted sum run
over its whole allowed key set.  Under causal masking, keys that no row of the
block may see are simply not formed (their probability is exactly 0).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep BLAS single-threaded inside the (b, h) worker pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover - optional
    threadpool_limits = None


def causal_allowed(i: int, Lq: int, Lk: int) -> int:
    """Largest key index query row ``i`` may attend to under the causal mask
    (bottom-right alignment: j <= i + Lk - Lq).  Negative means none."""
    return i + (Lk - Lq)


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor -> exact float64 copy
        import torch

        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def row_bounds(rows, Lq: int, Lk: int, causal: bool, window=(-1, -1)):
    """Inclusive key ranges [lo, hi] that query rows ``rows`` may see
    (lo > hi: none), as two integer arrays."""
    left, right = window
    rows = np.asarray(rows, dtype=np.int64)
    shift = Lk - Lq
    lo = np.zeros_like(rows) if left < 0 else np.maximum(0, rows + shift - left)
    hi = np.full_like(rows, Lk - 1)
    if right >= 0:
        hi = np.minimum(hi, rows + shift + right)
    if causal:
        hi = np.minimum(hi, rows + shift)
    return lo, hi


def key_bounds(i: int, Lq: int, Lk: int, causal: bool, window=(-1, -1)):
    """Inclusive range [lo, hi] of keys query row i may see (lo > hi: none)."""
    lo, hi = row_bounds([i], Lq, Lk, causal, window)
    return int(lo[0]), int(hi[0])


def _head_attention(qh, kh, vh, scale, causal, row_block, window=(-1, -1)):
    """Plain attention for one (batch, head): qh [Lq,D], kh/vh [Lk,D]."""
    Lq, D = qh.shape
    Lk = kh.shape[0]
    Dv = vh.shape[1]
    out = np.zeros((Lq, Dv), dtype=np.float64)
    lse = np.full((Lq,), -np.inf, dtype=np.float64)
    if Lk == 0:
        return out, lse
    for r0 in range(0, Lq, row_block):
        r1 = min(Lq, r0 + row_block)
        lo, hi = row_bounds(np.arange(r0, r1), Lq, Lk, causal, window)
        kbeg = max(0, int(lo.min()))
        kend = min(Lk, int(hi.max()) + 1)
        if kend <= kbeg:
            continue  # every row of this block has an empty key set
        s = scale * (qh[r0:r1] @ kh[kbeg:kend].T)  # [rows, kend - kbeg]
        cols = np.arange(kbeg, kend)[None, :]
        s = np.where((cols >= lo[:, None]) & (cols <= hi[:, None]), s, -np.inf)
        m = s.max(axis=1)
        nonempty = np.isfinite(m)
        m_safe = np.where(nonempty, m, 0.0)
        p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on masked keys
        l = p.sum(axis=1)
        o = p @ vh[kbeg:kend]
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(nonempty[:, None], o / l[:, None], 0.0)
            blk_lse = np.where(nonempty, m_safe + np.log(l), -np.inf)
        out[r0:r1] = o
        lse[r0:r1] = blk_lse
    return out, lse


def _default_workers() -> int:
    env = os.environ.get("ORACLE_WORKERS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def run_jobs(fn, jobs, workers):
    """fn(job) for every job: in order on this thread when workers <= 1,
    else in a thread pool of ``workers`` threads (None: the host's core
    count) with BLAS held to one thread per worker.  The jobs write disjoint
    slices of their outputs, so the order does not matter."""
    nw = workers if workers is not None else _default_workers()
    if nw <= 1 or len(jobs) <= 1:
        for j in jobs:
            fn(j)
        return
    import contextlib
    ctx = threadpool_limits(limits=1) if threadpool_limits is not None else contextlib.nullcontext()
    with ctx, ThreadPoolExecutor(max_workers=nw) as ex:
        list(ex.map(fn, jobs))


def attention_ref(q, k, v, scale: float, causal: bool, *, row_block: int = 1024,
                  workers: int | None = None, heads=None, window=(-1, -1)):
    """Plain fp64 attention.

    q: [B, Lq, Hq, D]; k, v: [B, Lk, Hkv, D] (any float type; converted to
    float64 exactly).  ``scale`` is applied as given (pass the float32 value
    that the GPU receives).  Returns (O [B, Lq, Hq, D], lse [B, Hq, Lq]) in
    float64.  ``heads`` optionally restricts the work to a list of (b, h)
    pairs; other outputs are left as NaN.  ``window`` = (left, right) limits
    row i to keys i + Lk - Lq - left .. i + Lk - Lq + right (negative: no
    limit on that side).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch between q, k, v")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    scale = float(scale)
    out = np.full((B, Lq, Hq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, Lq), np.nan)
    jobs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]

    def run(job):
        b, h = job
        kv = h // g
        o, l = _head_attention(q[b, :, h, :], k[b, :, kv, :], v[b, :, kv, :],
                               scale, causal, row_block, tuple(window))
        out[b, :, h, :] = o
        lse[b, h, :] = l

    run_jobs(run, jobs, workers)
    return out, lse


def decode_ref(q, k_cache, v_cache, seqlens, scale: float, *, heads=None, workers: int | None = 1):
    """One query token per sequence against a padded KV cache.

    q: [B, Hq, D]; k_cache, v_cache: [B, Lk_max, Hkv, D]; seqlens: [B] ints.
    Sequence b attends to keys 0 .. seqlens[b]-1 (all of them: the query is
    the newest token, so the bottom-right causal mask admits its whole
    cache).  Padding rows beyond seqlens[b] are never read.  Returns
    (O [B, Hq, D], lse [B, Hq]) in float64.  ``workers`` > 1 runs the
    sequences in a thread pool (None: the host's core count).
    """
    q = _as_f64(q)
    B, Hq, D = q.shape
    lens = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    out = np.full((B, Hq, v_cache.shape[3]), np.nan)
    lse = np.full((B, Hq), np.nan)
    jobs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    by_seq = {}
    for b, h in jobs:
        by_seq.setdefault(b, []).append(h)

    def run(b):
        n = max(0, min(lens[b], k_cache.shape[1]))
        cache_k, cache_v = {}, {}
        for h in by_seq[b]:
            kv = h // g
            if kv not in cache_k:  # slice first: padding (possibly NaN) is never touched
                cache_k[kv] = _as_f64(k_cache[b, :n, kv, :])
                cache_v[kv] = _as_f64(v_cache[b, :n, kv, :])
            o, l = _head_attention(q[b, h, :][None, :], cache_k[kv], cache_v[kv],
                                   float(scale), False, 1)
            out[b, h, :] = o[0]
            lse[b, h] = l[0]

    run_jobs(run, list(by_seq), workers)
    return out, lse


def _paged_rows(pages, scales, rows_page, rows_slot, kv):
    """Cached rows (page, slot, kv head) as float64, times their scales."""
    if hasattr(pages, "detach"):  # torch: index before converting
        import torch

        ip, isl = torch.as_tensor(rows_page), torch.as_tensor(rows_slot)
        x = _as_f64(pages[ip, isl, kv])
        sc = None if scales is None else _as_f64(scales[ip, kv, isl])
    else:
        x = _as_f64(np.asarray(pages)[rows_page, rows_slot, kv])
        sc = None if scales is None else _as_f64(np.asarray(scales)[rows_page, kv, rows_slot])
    return x if sc is None else x * sc[:, None]


def decode_paged_ref(q, k_pages, v_pages, block_table, seqlens, scale: float, *, k_scales=None,
                     v_scales=None, heads=None, workers: int | None = 1):
    """One query token per sequence against a paged, optionally int8, cache.

    q: [B, Hq, D]; k_pages, v_pages: [num_pages, P, Hkv, D]; block_table:
    [B, max_pages] page numbers; seqlens: [B].  Key j of sequence b is slot
    j % P of page block_table[b, j // P]; sequence b sees keys 0 ..
    min(seqlens[b], max_pages * P) - 1.  With k_scales ([num_pages, Hkv, P])
    k_pages holds integer codes and the cached key is code * scale (exact in
    float64); likewise v_scales for the values.  Then the definition of
    ``decode_ref``.  Returns (O [B, Hq, D], lse [B, Hq]) in float64.
    ``workers`` > 1 runs the sequences in a thread pool (None: the host's
    core count).
    """
    q = _as_f64(q)
    B, Hq, D = q.shape
    P, Hkv = int(k_pages.shape[1]), int(k_pages.shape[2])
    bt = np.asarray(block_table).astype(np.int64).reshape(B, -1)
    lens = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    out = np.full((B, Hq, int(v_pages.shape[3])), np.nan)
    lse = np.full((B, Hq), np.nan)
    jobs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    by_seq = {}
    for b, h in jobs:
        by_seq.setdefault(b, []).append(h)

    def run(b):
        n = max(0, min(lens[b], bt.shape[1] * P))
        j = np.arange(n)
        page, slot = bt[b, j // P], j % P
        cache = {}
        for h in by_seq[b]:
            kv = h // g
            if kv not in cache:
                cache[kv] = (_paged_rows(k_pages, k_scales, page, slot, kv),
                             _paged_rows(v_pages, v_scales, page, slot, kv))
            kb, vb = cache[kv]
            o, l = _head_attention(q[b, h, :][None, :], kb, vb, float(scale), False, 1)
            out[b, h, :] = o[0]
            lse[b, h] = l[0]

    run_jobs(run, list(by_seq), workers)
    return out, lse


def varlen_ref(q, k, v, cu_q, cu_k, scale: float, causal: bool, *, window=(-1, -1),
               workers: int | None = None, heads=None):
    """Block-diagonal packing: sequence b is rows cu_q[b] .. cu_q[b+1]-1 of
    q [total_q, Hq, D] and rows cu_k[b] .. cu_k[b+1]-1 of k, v [total_k, Hkv, D];
    each sequence attends only to its own keys, with the causal / window
    rules of ``attention_ref`` applied inside it.  Returns (O [total_q, Hq, D],
    lse [Hq, total_q]).  ``heads`` optionally restricts to (b, h) pairs.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cu_q = [int(x) for x in np.asarray(cu_q).reshape(-1)]
    cu_k = [int(x) for x in np.asarray(cu_k).reshape(-1)]
    B = len(cu_q) - 1
    total_q, Hq, _ = q.shape
    out = np.full((total_q, Hq, v.shape[2]), np.nan)
    lse = np.full((Hq, total_q), np.nan)
    for b in range(B):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        hs = None if heads is None else [(0, h) for (bb, h) in heads if bb == b]
        if hs is not None and not hs:
            continue
        if q1 <= q0:
            continue
        o_b, l_b = attention_ref(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], scale, causal,
                                 window=window, workers=workers, heads=hs)
        sel = range(Hq) if hs is None else [h for _, h in hs]
        for h in sel:
            out[q0:q1, h] = o_b[0, :, h]
            lse[h, q0:q1] = l_b[0, h]
    return out, lse
