"""Checks that pin an attention implementation to facts outside itself.

Each ``pin_*`` takes ``attn(q, k, v, scale, causal) -> (O, lse)`` (the
oracle's signature, float64 numpy in and out) and raises AssertionError when
the implementation disagrees with what the pages and the mathematics fix.
``tests/test_oracle.py`` runs them on the oracle, and runs them again on
oracles with planted mistakes to show that each mistake is caught.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from bruteforce import attention_decimal

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(seed, B, Lq, Lk, Hq, Hkv, D, scale_q=1.0, scale_k=1.0):
    r = rng(seed)
    q = r.standard_normal((B, Lq, Hq, D)) * scale_q
    k = r.standard_normal((B, Lk, Hkv, D)) * scale_k
    v = r.standard_normal((B, Lk, Hkv, D))
    return q, k, v


def assert_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinite entries differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# Tiny shapes for the decimal brute force: (B, Lq, Lk, Hq, Hkv, D, causal, scale)
BRUTE_CASES = [
    (1, 3, 3, 1, 1, 2, False, 0.7),
    (1, 4, 4, 2, 1, 3, True, 0.5),
    (2, 2, 5, 2, 2, 2, True, 1.3),   # Lk > Lq, bottom-right causal
    (1, 5, 2, 2, 1, 2, True, 0.9),   # Lk < Lq: empty rows
    (1, 3, 4, 4, 2, 3, False, -0.6),  # negative scale, GQA group 2
]


def pin_bruteforce(attn, tol=1e-13):
    for n, (B, Lq, Lk, Hq, Hkv, D, causal, scale) in enumerate(BRUTE_CASES):
        q, k, v = rand_qkv(100 + n, B, Lq, Lk, Hq, Hkv, D, scale_q=1.5)
        o, l = attn(q, k, v, scale, causal)
        ob, lb = attention_decimal(q, k, v, scale, causal)
        assert_close(o, ob, tol, f"brute O case {n}")
        assert_close(l, lb, tol, f"brute lse case {n}")


def pin_torch_sdpa(attn, tol=1e-12):
    """fp64 CPU torch.nn.functional.scaled_dot_product_attention (library),
    GQA expanded by repeat_interleave; lse from scipy.special.logsumexp of the
    library matmul's scores."""
    import torch
    from scipy.special import logsumexp

    for n, (B, L, Lk, Hq, Hkv, D, causal, scale) in enumerate([
        (2, 33, 33, 4, 2, 16, False, 0.25),
        (1, 40, 40, 2, 2, 8, True, 0.35),
        (1, 17, 29, 2, 1, 8, False, 0.3),
    ]):
        q, k, v = rand_qkv(200 + n, B, L, Lk, Hq, Hkv, D)
        o, l = attn(q, k, v, scale, causal)
        g = Hq // Hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=scale)
        assert_close(o, ref.permute(0, 2, 1, 3).numpy(), tol, f"sdpa O case {n}")
        s = (torch.matmul(tq, tk.transpose(-1, -2)) * scale).numpy()
        if causal:
            s = np.where(np.tril(np.ones((L, Lk), dtype=bool)), s, -np.inf)
        assert_close(l, logsumexp(s, axis=-1), tol, f"sdpa lse case {n}")


def pin_rows_are_distributions(attn):
    """With V = identity (D = Lk), O equals the probability matrix P: rows are
    non-negative, sum to 1, and are exactly 0 on masked keys."""
    for causal in (False, True):
        L = 12
        r = rng(300)
        q = r.standard_normal((1, L, 2, L))
        k = r.standard_normal((1, L, 1, L))
        v = np.eye(L)[None, :, None, :]
        o, _ = attn(q, k, v, 0.4, causal)
        P = o[0].transpose(1, 0, 2)  # [H, L, L]
        assert np.all(P >= 0), "negative probability"
        assert np.max(np.abs(P.sum(-1) - 1)) <= 1e-12, "rows of P do not sum to 1"
        if causal:
            upper = np.triu(np.ones((L, L), dtype=bool), 1)
            assert np.all(P[:, upper] == 0), "masked keys got probability"


def pin_constant_v(attn):
    for causal in (False, True):
        q, k, _ = rand_qkv(400, 2, 21, 21, 2, 1, 8, scale_q=3.0)
        c = rng(401).standard_normal(8)
        v = np.broadcast_to(c, (2, 21, 1, 8)).copy()
        o, _ = attn(q, k, v, 0.5, causal)
        assert_close(o, np.broadcast_to(c, o.shape), 1e-13, "constant V")


def pin_causal_row0(attn):
    q, k, v = rand_qkv(500, 2, 9, 9, 4, 2, 8)
    o, l = attn(q, k, v, 0.3, True)
    g = 2
    for b in range(2):
        for h in range(4):
            kv = h // g
            assert_close(o[b, 0, h], v[b, 0, kv], 1e-15, "causal row 0 O")
            s00 = 0.3 * float(np.dot(q[b, 0, h], k[b, 0, kv]))
            assert abs(l[b, h, 0] - s00) <= 1e-14, "causal row 0 lse"


def pin_uniform_q(attn):
    L = 16
    _, k, v = rand_qkv(600, 1, L, L, 2, 2, 8)
    q = np.zeros((1, L, 2, 8))
    o, l = attn(q, k, v, 0.7, True)
    means = np.cumsum(v[0], axis=0) / np.arange(1, L + 1)[:, None, None]
    assert_close(o[0], means, 1e-13, "Q=0 causal prefix means")
    assert_close(l[0], np.log(np.arange(1, L + 1))[None, :].repeat(2, 0), 1e-13, "Q=0 lse")
    o, l = attn(q, k, v, 0.7, False)
    assert_close(o[0], np.broadcast_to(v[0].mean(0), o[0].shape), 1e-13, "Q=0 full mean")
    assert_close(l, np.full(l.shape, math.log(L)), 1e-13, "Q=0 lse ln L")


def pin_key_shift(attn):
    """Adding u to every key leaves O unchanged and shifts lse_i by scale*q_i.u."""
    q, k, v = rand_qkv(700, 1, 10, 13, 2, 1, 6)
    u = rng(701).standard_normal(6)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, 0.45, causal)
        o2, l2 = attn(q, k + u, v, 0.45, causal)
        assert_close(o2, o1, 1e-12, "key shift O")
        shift = 0.45 * np.einsum("blhd,d->bhl", q, u)
        assert_close(l2, l1 + shift, 1e-12, "key shift lse")


def pin_value_affine(attn):
    q, k, v = rand_qkv(800, 1, 11, 11, 2, 2, 5)
    a, c = -1.7, 0.3
    o1, _ = attn(q, k, v, 0.6, True)
    o2, _ = attn(q, k, a * v + c, 0.6, True)
    assert_close(o2, a * o1 + c, 1e-12, "V affine")


def pin_permutation(attn):
    q, k, v = rand_qkv(900, 1, 8, 14, 2, 2, 4)
    perm = rng(901).permutation(14)
    o1, l1 = attn(q, k, v, 0.8, False)
    o2, l2 = attn(q, k[:, perm], v[:, perm], 0.8, False)
    assert_close(o2, o1, 1e-12, "joint K/V permutation O")
    assert_close(l2, l1, 1e-12, "joint K/V permutation lse")


def pin_gqa_equals_repeated_mha(attn):
    q, k, v = rand_qkv(1000, 2, 9, 9, 8, 2, 4)
    o1, l1 = attn(q, k, v, 0.5, True)
    o2, l2 = attn(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.5, True)
    assert_close(o1, o2, 1e-13, "GQA vs repeated MHA O")
    assert_close(l1, l2, 1e-13, "GQA vs repeated MHA lse")


def pin_bounds(attn):
    q, k, v = rand_qkv(1100, 1, 20, 20, 2, 2, 6, scale_q=4.0)
    for causal in (False, True):
        o, l = attn(q, k, v, 0.5, causal)
        for h in range(2):
            for i in range(20):
                n = i + 1 if causal else 20
                vv = v[0, :n, h]
                assert np.all(o[0, i, h] >= vv.min(0) - 1e-12)
                assert np.all(o[0, i, h] <= vv.max(0) + 1e-12)
                s = 0.5 * k[0, :n, h] @ q[0, i, h]
                assert s.max() - 1e-12 <= l[0, h, i] <= s.max() + math.log(n) + 1e-12


def _eval_expr(x):
    ns = {"e": math.e, "ln": math.log, "exp": math.exp, "tanh": math.tanh, "inf": math.inf,
          "__builtins__": {}}
    return float(eval(str(x), ns))  # expressions come from the repository's own fixture


def load_hand_cases():
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        return json.load(f)["cases"]


def pin_hand_cases(attn):
    for c in load_hand_cases():
        q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
        o_exp = np.vectorize(_eval_expr)(np.array(c["o"], dtype=object)).astype(np.float64)
        l_exp = np.vectorize(_eval_expr)(np.array(c["lse"], dtype=object)).astype(np.float64)
        o, l = attn(q, k, v, c["scale"], c["causal"])
        assert_close(o, o_exp, 1e-14, f"hand case {c['name']} O")
        assert_close(l, l_exp, 1e-14, f"hand case {c['name']} lse")


def pin_large_scores(attn):
    """Scores around 1e3: only a max-subtracted softmax stays finite; the
    answer is a closed form (the top key dominates by e^-100)."""
    q = np.zeros((1, 1, 1, 1))
    q[0, 0, 0, 0] = 1.0
    k = np.array([1000.0, 900.0, 950.0]).reshape(1, 3, 1, 1)
    v = np.array([1.0, 2.0, 3.0]).reshape(1, 3, 1, 1)
    o, l = attn(q, k, v, 1.0, False)
    # P = [1, e^-100, e^-50] / (1 + e^-100 + e^-50)
    z = 1 + math.exp(-100) + math.exp(-50)
    assert_close(o, np.array((1 + 2 * math.exp(-100) + 3 * math.exp(-50)) / z).reshape(o.shape),
                 1e-14, "large scores O")
    assert_close(l, np.array(1000 + math.log(z)).reshape(l.shape), 1e-12, "large scores lse")


# (B, Lq, Lk, Hq, Hkv, D, causal, scale, window)
WINDOW_CASES = [
    (1, 6, 6, 1, 1, 2, False, 0.8, (1, 2)),
    (1, 5, 7, 2, 1, 2, True, 0.6, (2, -1)),
    (1, 6, 4, 1, 1, 3, False, 1.1, (0, 0)),
    (1, 4, 6, 2, 2, 2, True, 0.5, (-1, 3)),
]


def pin_window_bruteforce(attn, tol=1e-13):
    for n, (B, Lq, Lk, Hq, Hkv, D, causal, scale, win) in enumerate(WINDOW_CASES):
        q, k, v = rand_qkv(150 + n, B, Lq, Lk, Hq, Hkv, D, scale_q=1.5)
        o, l = attn(q, k, v, scale, causal, window=win)
        ob, lb = attention_decimal(q, k, v, scale, causal, window=win)
        assert_close(o, ob, tol, f"window brute O case {n}")
        assert_close(l, lb, tol, f"window brute lse case {n}")


def pin_window_closed_forms(attn):
    """Window (0, 0) leaves each row its diagonal key; Q = 0 turns any window
    into a plain mean over it; open windows reduce to the unwindowed cases."""
    q, k, v = rand_qkv(160, 1, 9, 9, 2, 2, 4)
    o, l = attn(q, k, v, 0.7, False, window=(0, 0))
    assert_close(o, v, 1e-15, "window (0,0) O")
    assert_close(l, 0.7 * np.einsum("blhd,blhd->bhl", q, k), 1e-14, "window (0,0) lse")
    L, left, right = 13, 3, 2
    _, k, v = rand_qkv(161, 1, L, L, 1, 1, 4)
    q = np.zeros((1, L, 1, 4))
    o, l = attn(q, k, v, 0.5, False, window=(left, right))
    for i in range(L):
        lo, hi = max(0, i - left), min(L - 1, i + right)
        assert_close(o[0, i, 0], v[0, lo:hi + 1, 0].mean(0), 1e-14, f"window mean row {i}")
        assert abs(l[0, 0, i] - math.log(hi - lo + 1)) <= 1e-14
    q, k, v = rand_qkv(162, 1, 11, 11, 2, 1, 4)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, 0.4, causal)
        o2, l2 = attn(q, k, v, 0.4, causal, window=(-1, -1))
        o3, l3 = attn(q, k, v, 0.4, causal, window=(11, 11))
        assert_close(o2, o1, 0.0, "open window O")
        assert_close(o3, o1, 1e-15, "wide window O")
        assert_close(l3, l1, 1e-15, "wide window lse")
    o1, l1 = attn(q, k, v, 0.4, True)
    o2, l2 = attn(q, k, v, 0.4, False, window=(-1, 0))
    assert_close(o2, o1, 1e-15, "window (-1,0) == causal O")
    assert_close(l2, l1, 1e-15, "window (-1,0) == causal lse")


ALL_PINS = [
    pin_bruteforce,
    pin_torch_sdpa,
    pin_rows_are_distributions,
    pin_constant_v,
    pin_causal_row0,
    pin_uniform_q,
    pin_key_shift,
    pin_value_affine,
    pin_permutation,
    pin_gqa_equals_repeated_mha,
    pin_bounds,
    pin_hand_cases,
    pin_large_scores,
    pin_window_bruteforce,
    pin_window_closed_forms,
]
