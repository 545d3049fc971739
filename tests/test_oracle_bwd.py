"""Pins of the oracle's backward (CPU only).

``oracle.attention_bwd_ref`` is held to facts outside itself: central finite
differences of the (separately pinned) forward oracle, PyTorch fp64 autograd
through ``scaled_dot_product_attention``, and closed-form identities of the
softmax gradient.  Planted mistakes in its source must each fail a pin.
"""

from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as obwd
from pins import assert_close, rand_qkv


def loss(q, k, v, do, scale, causal, window):
    o, _ = oracle.attention_ref(q, k, v, scale, causal, window=window, workers=1)
    return float((o * do).sum())


# (B, Lq, Lk, Hq, Hkv, D, causal, scale, window)
FD_CASES = [
    (1, 3, 3, 1, 1, 2, False, 0.7, (-1, -1)),
    (1, 4, 4, 2, 1, 3, True, 0.5, (-1, -1)),
    (1, 3, 5, 2, 2, 2, True, 1.1, (-1, -1)),   # Lk > Lq, bottom-right causal
    (1, 5, 3, 2, 1, 2, True, 0.9, (-1, -1)),   # Lk < Lq: rows with no key
    (1, 5, 5, 2, 1, 2, False, -0.6, (1, 1)),   # window, negative scale
]


def pin_finite_differences(fn, h=1e-6, tol=2e-8):
    for n, (B, Lq, Lk, Hq, Hkv, D, causal, scale, win) in enumerate(FD_CASES):
        q, k, v = rand_qkv(300 + n, B, Lq, Lk, Hq, Hkv, D)
        do = np.random.default_rng(400 + n).standard_normal(q.shape)
        dq, dk, dv = fn(q, k, v, do, scale, causal, window=win)
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*args_p, do, scale, causal, win)
                            - loss(*args_m, do, scale, causal, win)) / (2 * h)
            assert_close(grad, num, tol, f"finite differences d{name} case {n}")


def pin_torch_autograd(fn):
    """fp64 autograd through torch sdpa (causal only at Lq == Lk; GQA by
    repeating K/V, whose gradients then sum over the group)."""
    for n, (B, L, Hq, Hkv, D, causal) in enumerate([(2, 7, 4, 2, 8, True), (1, 9, 3, 3, 5, False),
                                                    (1, 6, 8, 1, 4, True)]):
        q, k, v = rand_qkv(500 + n, B, L, L, Hq, Hkv, D)
        do = np.random.default_rng(600 + n).standard_normal(q.shape)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        g = Hq // Hkv
        o = torch.nn.functional.scaled_dot_product_attention(
            tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(g, dim=1),
            tv.permute(0, 2, 1, 3).repeat_interleave(g, dim=1), is_causal=causal, scale=0.4)
        (o.permute(0, 2, 1, 3) * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = fn(q, k, v, do, 0.4, causal)
        assert_close(dq, tq.grad.numpy(), 1e-12, f"autograd dq {n}")
        assert_close(dk, tk.grad.numpy(), 1e-12, f"autograd dk {n}")
        assert_close(dv, tv.grad.numpy(), 1e-12, f"autograd dv {n}")


def pin_identities(fn):
    """Softmax is invariant to adding one vector to every key, so the key
    gradients of a head sum to 0; the value gradients sum to the sum of dO over
    rows that see a key; a row that sees a single key has dq = 0."""
    B, L, Hq, Hkv, D = 2, 11, 4, 2, 6
    q, k, v = rand_qkv(700, B, L, L, Hq, Hkv, D)
    do = np.random.default_rng(701).standard_normal(q.shape)
    for causal, win in ((False, (-1, -1)), (True, (-1, -1)), (True, (3, -1))):
        dq, dk, dv = fn(q, k, v, do, 0.8, causal, window=win)
        assert_close(dk.sum(axis=1), np.zeros((B, Hkv, D)), 1e-12, "sum of dk")
        g = Hq // Hkv
        want = do.reshape(B, L, Hkv, g, D).sum(axis=(1, 3))
        assert_close(dv.sum(axis=1), want, 1e-12, "sum of dv")
        if causal:
            assert_close(dq[:, 0], np.zeros((B, Hq, D)), 1e-15, "row 0 dq")
    dq, dk, dv = fn(q, k, v, do, 0.8, False, window=(0, 0))
    assert_close(dq, np.zeros_like(dq), 1e-15, "window (0,0) dq")
    assert_close(dk, np.zeros_like(dk), 1e-15, "window (0,0) dk")
    assert_close(dv, do.reshape(B, L, Hkv, Hq // Hkv, D).sum(axis=3), 1e-14, "window (0,0) dv")


def pin_empty_rows_and_bounds(fn):
    """Rows with no allowed key give dq = 0 and add nothing to dk, dv; the
    |term| sums bound the gradients."""
    q, k, v = rand_qkv(800, 1, 6, 3, 2, 1, 4)
    do = np.random.default_rng(801).standard_normal(q.shape)
    dq, dk, dv, aq, ak, av = fn(q, k, v, do, 0.7, True, bounds=True)
    assert np.all(dq[0, :3] == 0.0)  # rows 0..2 see no key (bottom-right causal, Lk < Lq)
    for x, a in ((dq, aq), (dk, ak), (dv, av)):
        assert np.all(np.abs(x) <= a + 1e-15)
    dq2, dk2, dv2 = fn(q[:, 3:], k, v, do[:, 3:], 0.7, True)
    assert_close(dk, dk2, 1e-15, "empty rows add nothing to dk")
    assert_close(dv, dv2, 1e-15, "empty rows add nothing to dv")


BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_identities, pin_empty_rows_and_bounds]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_pin(pin):
    pin(oracle.attention_bwd_ref)


def test_kv_head_selection_matches_full():
    q, k, v = rand_qkv(900, 2, 9, 9, 4, 2, 5)
    do = np.random.default_rng(901).standard_normal(q.shape)
    full = oracle.attention_bwd_ref(q, k, v, do, 0.3, True)
    part = oracle.attention_bwd_ref(q, k, v, do, 0.3, True, kv_heads=[(1, 0)])
    assert np.array_equal(part[0][1, :, 0:2], full[0][1, :, 0:2])
    assert np.array_equal(part[1][1, :, 0], full[1][1, :, 0])
    assert np.array_equal(part[2][1, :, 0], full[2][1, :, 0])
    assert np.isnan(part[0][0]).all() and np.isnan(part[1][1, :, 1]).all()


def test_row_blocking_is_invisible():
    q, k, v = rand_qkv(902, 1, 37, 37, 2, 1, 4)
    do = np.random.default_rng(903).standard_normal(q.shape)
    a = oracle.attention_bwd_ref(q, k, v, do, 0.5, True, row_block=512)
    b = oracle.attention_bwd_ref(q, k, v, do, 0.5, True, row_block=5)
    for x, y in zip(a, b):
        assert_close(x, y, 1e-14, "row blocks")


BWD_MUTATIONS = {
    "no_D_term": ("ds = p * (dp - d_i[:, None])", "ds = p * dp"),
    "D_sign": ("ds = p * (dp - d_i[:, None])", "ds = p * (dp + d_i[:, None])"),
    "dq_no_scale": ("dq[r0:r1] = scale * (ds @ kh)", "dq[r0:r1] = ds @ kh"),
    "dk_uses_do": ("dk += scale * (ds.T @ qh[r0:r1])", "dk += scale * (ds.T @ doh[r0:r1])"),
    "dv_without_p": ("dv += p.T @ do", "dv += (p > 0).T @ do"),
    "mask_dropped": ("s = np.where(allowed, scale * (qh[r0:r1] @ kh.T), -np.inf)",
                     "s = scale * (qh[r0:r1] @ kh.T)"),
    "D_from_o_unnormalised": ("d_i = (p * dp).sum(axis=1)", "d_i = (e * dp).sum(axis=1)"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_planted_mistake_in_backward_is_caught(name):
    old, new = BWD_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(obwd._head_backward))
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(vars(obwd))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mutant_head = ns["_head_backward"]
    ns2 = dict(vars(obwd))
    ns2["_head_backward"] = mutant_head
    exec(compile(textwrap.dedent(inspect.getsource(obwd.attention_bwd_ref)), "<m>", "exec"), ns2)
    fn = ns2["attention_bwd_ref"]
    failed = []
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {name}"


GQA_MUTATION = ("for h in range(c * g, (c + 1) * g):", "for h in range((c + 1) * g - 1, (c + 1) * g):")


def test_planted_mistake_in_group_sum_is_caught():
    src = textwrap.dedent(inspect.getsource(obwd.attention_bwd_ref))
    assert GQA_MUTATION[0] in src
    ns = dict(vars(obwd))
    exec(compile(src.replace(*GQA_MUTATION), "<m>", "exec"), ns)
    failed = []
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns["attention_bwd_ref"])
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed


# Packed sequences: (lengths q, lengths k) per case; causal / window inside each
VARLEN_FD_CASES = [
    (([2, 0, 3], [2, 2, 3]), 2, 1, 2, True, 0.8, (-1, -1)),    # an empty query sequence
    (([3, 1, 2], [1, 3, 0]), 2, 2, 2, True, 0.6, (-1, -1)),    # Lk < Lq, Lk > Lq, no keys
    (([4, 2], [4, 3]), 2, 1, 2, False, -0.7, (1, 0)),          # window, negative scale
]


def _packed(seed, lq, lk, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    do = rng.standard_normal(q.shape)
    return q, k, v, do, cu_q, cu_k


def test_varlen_bwd_finite_differences():
    pin_varlen_finite_differences(oracle.varlen_bwd_ref)


def pin_varlen_finite_differences(fn):
    """Central differences of the packed forward oracle (sum of O * dO)."""
    h = 1e-6
    for n, ((lq, lk), Hq, Hkv, D, causal, scale, win) in enumerate(VARLEN_FD_CASES):
        q, k, v, do, cu_q, cu_k = _packed(1000 + n, lq, lk, Hq, Hkv, D)

        def f(q_, k_, v_):
            o, _ = oracle.varlen_ref(q_, k_, v_, cu_q, cu_k, scale, causal, window=win, workers=1)
            return float(np.nansum(o * do))

        dq, dk, dv = fn(q, k, v, do, cu_q, cu_k, scale, causal, window=win)
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                a = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                b = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (f(*a) - f(*b)) / (2 * h)
            assert_close(grad, num, 2e-8, f"packed finite differences d{name} case {n}")


def test_varlen_bwd_kv_head_selection_and_bounds():
    q, k, v, do, cu_q, cu_k = _packed(1100, [5, 3], [4, 6], 4, 2, 3)
    full = oracle.varlen_bwd_ref(q, k, v, do, cu_q, cu_k, 0.5, True, bounds=True)
    part = oracle.varlen_bwd_ref(q, k, v, do, cu_q, cu_k, 0.5, True, kv_heads=[(1, 1)])
    assert np.array_equal(part[0][5:, 2:4], full[0][5:, 2:4])
    assert np.array_equal(part[1][4:, 1], full[1][4:, 1])
    assert np.isnan(part[0][:5]).all() and np.isnan(part[2][:4]).all()
    for x, a in zip(full[:3], full[3:]):
        assert np.all(np.abs(x) <= a + 1e-15)


VARLEN_MUTATIONS = {
    "keys_at_query_rows": ("k[None, k0:k1], v[None, k0:k1], do[None, q0:q1]",
                           "k[None, q0:q1], v[None, q0:q1], do[None, q0:q1]"),
    "dk_written_to_query_rows": ("enumerate(((q0, q1, hs), (k0, k1, c), (k0, k1, c)))",
                                 "enumerate(((q0, q1, hs), (q0, q1, c), (k0, k1, c)))"),
}


@pytest.mark.parametrize("name", sorted(VARLEN_MUTATIONS))
def test_planted_mistake_in_varlen_backward_is_caught(name):
    old, new = VARLEN_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(obwd.varlen_bwd_ref))
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(vars(obwd))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        with np.errstate(all="ignore"):
            pin_varlen_finite_differences(ns["varlen_bwd_ref"])
