"""Gradients of the attention definition, in float64 -- the oracle's backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed
----------------
The forward (``attention.py``) maps Q, K, V to O with, for one (batch, query
head), scores s_ij = scale * q_i . k_j, the allowed key sets A_i (causal /
window rules), P_ij = softmax over A_i of s_i. (0 off A_i) and O_i =
sum_j P_ij v_j.  The backward takes the gradient dO of some loss with respect
to O and returns the gradients with respect to Q, K and V -- the chain rule
through those three lines, written out:

  dv_j   = sum_i P_ij dO_i
  dP_ij  = dO_i . v_j
  D_i    = sum_j P_ij dP_ij            (equals dO_i . O_i)
  dS_ij  = P_ij (dP_ij - D_i)          (the softmax Jacobian applied to dP)
  dq_i   = scale * sum_j dS_ij k_j
  dk_j   = scale * sum_i dS_ij q_i

With grouped K/V heads (query head h reads K/V head h // (Hq / Hkv)) dK and
dV of a K/V head sum the contributions of every query head of its group.
Rows with no allowed key have P = 0 and contribute nothing.

Sources (page title, section): the pages define only the forward; "FlashAttention-
2 (TH)" (systems-analysis.info), performance, reports forward-plus-backward
training throughput, and "5 years, 10K stars: xformers" (cloud.tencent.com)
pairs each forward operator with a backward one.  The gradient of the forward
definition is fixed by calculus; it is pinned in tests by finite differences
of the forward oracle and by PyTorch autograd.

Implementation notes: one (batch, K/V head) at a time, its query heads in
turn, query rows in blocks of ``row_block``; P is recomputed from the
definition (the kernel's saved lse is not an input here).  For sequences
packed back to back (``varlen_bwd_ref``) every sequence is its own batch
entry: the forward it differentiates (``attention.varlen_ref``) lets no
sequence see another's keys, so the gradients of one sequence's rows come
from that sequence alone.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, row_bounds, run_jobs


def _head_backward(qh, kh, vh, doh, scale, causal, window, row_block, bounds):
    """One (batch, query head): qh, doh [Lq, D]; kh, vh [Lk, D].  Returns
    dq [Lq, D], dk [Lk, D], dv [Lk, Dv] and, with ``bounds``, the sums of the
    absolute values of the terms of each of them (same shapes)."""
    Lq, D = qh.shape
    Lk = kh.shape[0]
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros((Lk, vh.shape[1]))
    abs_q = np.zeros_like(qh) if bounds else None
    abs_k = np.zeros_like(kh) if bounds else None
    abs_v = np.zeros((Lk, vh.shape[1])) if bounds else None
    if Lk == 0:
        return dq, dk, dv, abs_q, abs_k, abs_v
    cols = np.arange(Lk)[None, :]
    for r0 in range(0, Lq, row_block):
        r1 = min(Lq, r0 + row_block)
        lo, hi = row_bounds(np.arange(r0, r1), Lq, Lk, causal, window)
        allowed = (cols >= lo[:, None]) & (cols <= hi[:, None])
        s = np.where(allowed, scale * (qh[r0:r1] @ kh.T), -np.inf)
        m = s.max(axis=1)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m_safe[:, None])
        l = e.sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            p = np.where(l[:, None] > 0, e / l[:, None], 0.0)        # P, 0 off A_i
        do = doh[r0:r1]
        dv += p.T @ do
        dp = do @ vh.T
        d_i = (p * dp).sum(axis=1)
        ds = p * (dp - d_i[:, None])
        dq[r0:r1] = scale * (ds @ kh)
        dk += scale * (ds.T @ qh[r0:r1])
        if bounds:
            # magnitudes for error bounds: |terms| of each sum, plus the
            # sensitivity of dS to an error in D_i (relative to sum_d |dO O|)
            abs_v += p.T @ np.abs(do)
            abs_d = np.abs(do * (p @ vh)).sum(axis=1)
            wgt = np.abs(ds) + p * abs_d[:, None]
            abs_q[r0:r1] = abs(scale) * (wgt @ np.abs(kh))
            abs_k += abs(scale) * (wgt.T @ np.abs(qh[r0:r1]))
    return dq, dk, dv, abs_q, abs_k, abs_v


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool, *, window=(-1, -1),
                      kv_heads=None, row_block: int = 512, bounds: bool = False,
                      workers: int | None = 1):
    """Gradients of ``attention_ref``'s O with respect to q, k, v, given dO.

    q, do: [B, Lq, Hq, D]; k, v: [B, Lk, Hkv, D].  Returns (dq, dk, dv) in
    float64 with the shapes of q, k, v; with ``bounds`` also (abs_dq, abs_dk,
    abs_dv), the per-element sums of |terms| of each gradient (for error
    bounds).  ``kv_heads`` optionally restricts the work to a list of
    (b, kv head) pairs: their dK, dV and the dQ of their query heads are
    computed, everything else is NaN.  ``workers`` > 1 runs the (b, kv head)
    pairs in a thread pool (BLAS held to one thread per worker); None picks
    the host's core count.

    The bounds are abs_dv_j = sum_i P_ij |dO_i|, abs_dq_i = |scale| sum_j
    w_ij |k_j| and abs_dk_j = |scale| sum_i w_ij |q_i| with w_ij = |dS_ij| +
    P_ij sum_d |dO_id O_id| (the second part: how much dS moves when D_i is
    off by a relative amount).  A kernel whose P, dS and D carry relative
    errors e has gradient errors of about e times these.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if Hkv < 1 or Hq % Hkv or do.shape != q.shape:
        raise ValueError("shape mismatch")
    g = Hq // Hkv
    scale = float(scale)
    out = [np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan)]
    absd = [np.full(x.shape, np.nan) for x in out] if bounds else None
    jobs = list(kv_heads) if kv_heads is not None else [(b, c) for b in range(B)
                                                          for c in range(Hkv)]
    def run(job):
        b, c = job
        dk_acc = np.zeros((Lk, D))
        dv_acc = np.zeros((Lk, v.shape[3]))
        ak_acc = np.zeros((Lk, D))
        av_acc = np.zeros((Lk, v.shape[3]))
        for h in range(c * g, (c + 1) * g):
            dq, dk, dv, aq, ak, av = _head_backward(q[b, :, h], k[b, :, c], v[b, :, c],
                                                    do[b, :, h], scale, causal, tuple(window),
                                                    row_block, bounds)
            out[0][b, :, h] = dq
            dk_acc += dk
            dv_acc += dv
            if bounds:
                absd[0][b, :, h] = aq
                ak_acc += ak
                av_acc += av
        out[1][b, :, c] = dk_acc
        out[2][b, :, c] = dv_acc
        if bounds:
            absd[1][b, :, c] = ak_acc
            absd[2][b, :, c] = av_acc

    run_jobs(run, jobs, workers)
    if bounds:
        return tuple(out) + tuple(absd)
    return tuple(out)


def varlen_bwd_ref(q, k, v, do, cu_q, cu_k, scale: float, causal: bool, *, window=(-1, -1),
                   kv_heads=None, bounds: bool = False, workers: int | None = 1):
    """Gradients of ``varlen_ref``'s O: sequence b is rows cu_q[b] ..
    cu_q[b+1]-1 of q, do [total_q, Hq, D] and rows cu_k[b] .. cu_k[b+1]-1 of
    k, v [total_k, Hkv, D].  Returns (dq, dk, dv) in float64 with the shapes
    of q, k, v (and, with ``bounds``, the |term| sums of attention_bwd_ref).
    Keys of a sequence that no query row sees get dk = dv = 0.  ``kv_heads``
    optionally restricts the work to (b, kv head) pairs; everything else is
    NaN.  ``workers``: the thread pool of attention_bwd_ref, per sequence."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    cu_q = [int(x) for x in np.asarray(cu_q).reshape(-1)]
    cu_k = [int(x) for x in np.asarray(cu_k).reshape(-1)]
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    out = [np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan)]
    absd = [np.full(x.shape, np.nan) for x in out] if bounds else None
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sel = None if kv_heads is None else [(0, c) for (bb, c) in kv_heads if bb == b]
        if sel is not None and not sel:
            continue
        res = attention_bwd_ref(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], do[None, q0:q1],
                                scale, causal, window=window, kv_heads=sel, bounds=bounds,
                                workers=workers)
        cs = range(Hkv) if sel is None else [c for _, c in sel]
        for c in cs:
            hs = slice(c * g, (c + 1) * g)
            for n, (lo, hi, hsl) in enumerate(((q0, q1, hs), (k0, k1, c), (k0, k1, c))):
                out[n][lo:hi, hsl] = res[n][0, :, hsl]
                if bounds:
                    absd[n][lo:hi, hsl] = res[3 + n][0, :, hsl]
    if bounds:
        return tuple(out) + tuple(absd)
    return tuple(out)
