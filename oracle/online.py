"""Blockwise online softmax and split-KV merge, restated in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are *not* the reference the GPU is compared with -- that is the plain
definition in ``attention.py``.  They restate, step by step, the algorithm
the pages describe, so that the tests can check the pages' central claim in
exact-ish arithmetic: the blockwise computation reaches the same result as
the standard one.

Sources (page title, section):
* "FlashAttention in the CANN ops-transformer library" (ai6s.net), section 2,
  step 1 (cut K/V into blocks), step 2 (after each block update the running
  row max and row sum; the end result equals standard attention) and step 3
  (O and the normaliser L accumulated block by block).
* "FlashAttention-2 (TH)" (systems-analysis.info), technical architecture,
  item 1: non-matmul work is kept small -- read as deferring the division by
  the row sum to the end (the accumulator holds unnormalised sums).
* The split-KV merge: "5 years, 10K stars: xformers" (cloud.tencent.com)
  names a split-K decoding backend and "FlashAttention-2 (TH)", references,
  cites FlashDecoding++; neither gives formulas.  Read here as: each key chunk
  yields its own (normalised output, logsumexp); the chunks are merged with
  weights exp(lse_chunk - lse_total), which is the same identity as the
  online update applied to chunk summaries.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64


def _online_head(qh, kh, vh, scale, causal, block):
    Lq, D = qh.shape
    Lk = kh.shape[0]
    shift = Lk - Lq
    m = np.full((Lq,), -np.inf)       # running row max of scaled scores
    l = np.zeros((Lq,))               # running row sum of exp(s - m)
    acc = np.zeros((Lq, vh.shape[1]))  # running unnormalised output
    rows = np.arange(Lq)[:, None]
    for j0 in range(0, Lk, block):
        j1 = min(Lk, j0 + block)
        s = scale * (qh @ kh[j0:j1].T)
        if causal:
            cols = np.arange(j0, j1)[None, :]
            s = np.where(cols <= rows + shift, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)             # rows that have seen a key
        m_ref = np.where(live, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        p = np.exp(s - m_ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ vh[j0:j1]
        m = m_new
    nonempty = np.isfinite(m)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(nonempty[:, None], acc / l[:, None], 0.0)
        lse = np.where(nonempty, m + np.log(l), -np.inf)
    return out, lse


def online_attention_ref(q, k, v, scale: float, causal: bool, block: int):
    """Online-softmax attention over key blocks of ``block`` keys.

    Same shapes and outputs as ``attention_ref``; single-threaded, meant for
    small inputs.
    """
    if block < 1:
        raise ValueError("block must be >= 1")
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Lq, Hq, _ = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Lq, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            o, s = _online_head(q[b, :, h], k[b, :, h // g], v[b, :, h // g],
                                float(scale), causal, block)
            out[b, :, h] = o
            lse[b, h] = s
    return out, lse


def split_combine_ref(q, k, v, scale: float, causal: bool, num_splits: int):
    """Attention computed per contiguous key chunk, then merged by logsumexp.

    The keys [0, Lk) are cut into ``num_splits`` chunks of ceil(Lk/num_splits)
    keys (the last ones may be short or empty).  Each chunk gives the plain
    softmax attention restricted to it, (O_s, lse_s); an empty chunk, or one
    whose keys are all masked for a row, has lse_s = -inf and weight 0.  The
    merge is  L = M + ln sum_s exp(lse_s - M)  with M = max_s lse_s  and
    O = sum_s exp(lse_s - L) * O_s.
    """
    from .attention import _head_attention

    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Lq, Hq, _ = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    chunk = -(-Lk // num_splits) if Lk else 0
    out = np.zeros((B, Lq, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, Lq))
    shift = Lk - Lq
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            parts_o, parts_l = [], []
            for s_idx in range(num_splits):
                j0 = min(Lk, s_idx * chunk)
                j1 = min(Lk, j0 + chunk)
                qh = q[b, :, h]
                if j1 <= j0:
                    parts_o.append(np.zeros((Lq, v.shape[3])))
                    parts_l.append(np.full((Lq,), -np.inf))
                    continue
                # scores of the chunk; the causal bound is expressed on global
                # key indices, so shift the query rows instead of the keys.
                kc, vc = k[b, j0:j1, kv], v[b, j0:j1, kv]
                if causal:
                    # row i may see chunk key t (global j0+t) iff j0+t <= i+shift
                    o_c = np.zeros((Lq, v.shape[3]))
                    l_c = np.full((Lq,), -np.inf)
                    for i in range(Lq):
                        n = min(j1, i + shift + 1) - j0
                        if n <= 0:
                            continue
                        oi, li = _head_attention(qh[i:i + 1], kc[:n], vc[:n],
                                                 float(scale), False, 1)
                        o_c[i], l_c[i] = oi[0], li[0]
                else:
                    o_c, l_c = _head_attention(qh, kc, vc, float(scale), False, 1024)
                parts_o.append(o_c)
                parts_l.append(l_c)
            L = np.stack(parts_l)            # [S, Lq]
            O = np.stack(parts_o)            # [S, Lq, D]
            M = L.max(axis=0)
            live = np.isfinite(M)
            M_ref = np.where(live, M, 0.0)
            w = np.exp(L - M_ref[None, :])  # exp(-inf) = 0 for empty chunks
            tot = w.sum(axis=0)
            with np.errstate(divide="ignore", invalid="ignore"):
                Lt = np.where(live, M_ref + np.log(tot), -np.inf)
                wn = np.where(live[None, :], w / tot[None, :], 0.0)
            out[b, :, h] = (wn[:, :, None] * O).sum(axis=0)
            lse[b, h] = Lt
    return out, lse
