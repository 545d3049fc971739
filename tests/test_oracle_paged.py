"""Pins of the oracle's paged / int8 KV-cache decode (CPU only).

``oracle.decode_paged_ref`` is held to facts outside itself: a 40-digit
decimal evaluation over a cache gathered with plain Python loops, PyTorch's
fp64 CPU ``scaled_dot_product_attention`` over a cache gathered another way,
invariance under renumbering the physical pages, and the identities of the
per-row scales.  Planted mistakes in its source must each fail a pin.
"""

from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
from bruteforce import attention_decimal
from pins import assert_close


def paged_case(seed, B, Hq, Hkv, D, P, lens, *, int8_k=False, int8_v=False, extra_pages=3,
               max_pages=None):
    """A random paged cache: each sequence gets its own pages, in a shuffled
    physical order, plus unused pages filled with large junk.  int8 sides hold
    integer codes in [-127, 127] with positive per-row scales
    ([num_pages, Hkv, P])."""
    r = np.random.default_rng(seed)
    need = [(n + P - 1) // P for n in lens]
    mp = max_pages or max(1, max(need))
    num_pages = sum(need) + extra_pages
    perm = r.permutation(num_pages)
    table = np.zeros((B, mp), dtype=np.int64)
    nxt = 0
    for b in range(B):
        for p in range(need[b]):
            table[b, p] = perm[nxt]
            nxt += 1
        table[b, need[b]:] = perm[-1]  # unused entries point at a junk page

    def side(is_int8):
        if is_int8:
            codes = r.integers(-127, 128, (num_pages, P, Hkv, D)).astype(np.float64)
            scales = r.uniform(0.01, 0.05, (num_pages, Hkv, P))
            return codes, scales
        return r.standard_normal((num_pages, P, Hkv, D)), None

    kp, ks = side(int8_k)
    vp, vs = side(int8_v)
    used = set(table[b, p] for b in range(B) for p in range(need[b]))
    for pg in range(num_pages):
        if pg not in used:
            kp[pg] = 1e6
            vp[pg] = -1e6
    q = r.standard_normal((B, Hq, D))
    return q, kp, vp, table, np.asarray(lens), ks, vs


def logical_cache_loops(kp, vp, table, ks, vs, b, n):
    """Sequence b's first n keys and values, gathered by explicit loops."""
    P, Hkv, D = kp.shape[1], kp.shape[2], kp.shape[3]
    K = np.zeros((1, n, Hkv, D))
    V = np.zeros((1, n, Hkv, D))
    for j in range(n):
        page = int(table[b][j // P])
        slot = j - (j // P) * P
        for h in range(Hkv):
            for d in range(D):
                K[0, j, h, d] = kp[page, slot, h, d] * (1.0 if ks is None else ks[page, h, slot])
                V[0, j, h, d] = vp[page, slot, h, d] * (1.0 if vs is None else vs[page, h, slot])
    return K, V


CASES = [
    # seed, B, Hq, Hkv, D, P, lens, int8_k, int8_v
    (1, 2, 2, 1, 3, 2, [3, 5], False, False),
    (2, 2, 4, 2, 2, 4, [7, 1], True, False),
    (3, 3, 2, 2, 2, 2, [0, 4, 6], True, True),
]


def pin_decimal(fn):
    for seed, B, Hq, Hkv, D, P, lens, i8k, i8v in CASES:
        q, kp, vp, table, ln, ks, vs = paged_case(seed, B, Hq, Hkv, D, P, lens, int8_k=i8k,
                                                  int8_v=i8v)
        o, l = fn(q, kp, vp, table, ln, 0.8, k_scales=ks, v_scales=vs)
        for b in range(B):
            if lens[b] == 0:
                assert np.all(o[b] == 0.0) and np.all(np.isneginf(l[b])), "empty sequence"
                continue
            K, V = logical_cache_loops(kp, vp, table, ks, vs, b, lens[b])
            ob, lb = attention_decimal(q[b][None, None], K, V, 0.8, False)
            assert_close(o[b], ob[0, 0], 1e-13, f"paged decimal O seed {seed} b {b}")
            assert_close(l[b], lb[0, :, 0], 1e-13, f"paged decimal lse seed {seed} b {b}")


def pin_torch_sdpa(fn):
    """Library cross-check: gather with torch indexing, dequantize, sdpa in fp64."""
    B, Hq, Hkv, D, P = 3, 8, 2, 16, 4
    lens = [13, 1, 30]
    q, kp, vp, table, ln, ks, vs = paged_case(7, B, Hq, Hkv, D, P, lens, int8_k=True, int8_v=True)
    o, l = fn(q, kp, vp, table, ln, 0.3, k_scales=ks, v_scales=vs)
    tk = torch.from_numpy(kp * ks.transpose(0, 2, 1)[..., None]).reshape(-1, Hkv, D)
    tv = torch.from_numpy(vp * vs.transpose(0, 2, 1)[..., None]).reshape(-1, Hkv, D)
    for b in range(B):
        rows = torch.tensor([int(table[b][j // P]) * P + j % P for j in range(lens[b])])
        K = tk.index_select(0, rows).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        V = tv.index_select(0, rows).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        qb = torch.from_numpy(q[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, K, V, scale=0.3)
        s = 0.3 * torch.einsum("hqd,hkd->hqk", qb, K)
        lse = torch.logsumexp(s, dim=-1)[:, 0]
        assert_close(o[b], ref[:, 0].numpy(), 1e-12, "paged sdpa O")
        assert_close(l[b], lse.numpy(), 1e-12, "paged sdpa lse")


def pin_page_renumbering(fn):
    """Moving pages to other physical slots (and updating the table) changes
    nothing, bit for bit."""
    q, kp, vp, table, ln, ks, vs = paged_case(11, 2, 4, 2, 4, 4, [9, 14], int8_k=True,
                                              int8_v=True)
    o1, l1 = fn(q, kp, vp, table, ln, 0.5, k_scales=ks, v_scales=vs)
    r = np.random.default_rng(12)
    perm = r.permutation(kp.shape[0])          # new slot of old page p is perm[p]
    kp2, vp2, ks2, vs2 = (np.empty_like(x) for x in (kp, vp, ks, vs))
    kp2[perm], vp2[perm], ks2[perm], vs2[perm] = kp, vp, ks, vs
    o2, l2 = fn(q, kp2, vp2, perm[table], ln, 0.5, k_scales=ks2, v_scales=vs2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "page renumbering changed O"


def pin_scale_identities(fn):
    """Key scales multiply the scores (c * k_scales == c * softmax scale);
    value scales multiply O and leave lse alone."""
    q, kp, vp, table, ln, ks, vs = paged_case(13, 2, 4, 1, 4, 2, [5, 8], int8_k=True,
                                              int8_v=True)
    o1, l1 = fn(q, kp, vp, table, ln, 0.25, k_scales=ks, v_scales=vs)
    o2, l2 = fn(q, kp, vp, table, ln, 0.5, k_scales=ks / 2, v_scales=vs)
    assert_close(o2, o1, 1e-13, "k scale vs softmax scale O")
    assert_close(l2, l1, 1e-13, "k scale vs softmax scale lse")
    o3, l3 = fn(q, kp, vp, table, ln, 0.25, k_scales=ks, v_scales=3 * vs)
    assert_close(o3, 3 * o1, 1e-12, "v scale O")
    assert_close(l3, l1, 0.0, "v scale lse")


def pin_length_clamp(fn):
    """Lengths beyond the table's capacity are cut to it; negative ones are 0."""
    q, kp, vp, table, ln, ks, vs = paged_case(17, 2, 2, 1, 3, 2, [4, 3], max_pages=2)
    o1, l1 = fn(q, kp, vp, table, np.array([4, 3]), 0.7)
    o2, l2 = fn(q, kp, vp, table, np.array([100, 3]), 0.7)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = fn(q, kp, vp, table, np.array([-5, 3]), 0.7)
    assert np.all(o3[0] == 0.0) and np.all(np.isneginf(l3[0]))


PAGED_PINS = [pin_decimal, pin_torch_sdpa, pin_page_renumbering, pin_scale_identities,
              pin_length_clamp]


@pytest.mark.parametrize("pin", PAGED_PINS, ids=lambda p: p.__name__)
def test_paged_pin(pin):
    pin(oracle.decode_paged_ref)


def test_identity_table_equals_dense_decode():
    """A table that lays the pages out in order is the padded dense cache."""
    B, Hq, Hkv, D, P, L = 3, 4, 2, 8, 4, 12
    r = np.random.default_rng(21)
    q = r.standard_normal((B, Hq, D))
    kc = r.standard_normal((B, L, Hkv, D))
    vc = r.standard_normal((B, L, Hkv, D))
    lens = np.array([12, 5, 0])
    table = np.arange(B * (L // P)).reshape(B, L // P)
    o1, l1 = oracle.decode_ref(q, kc, vc, lens, 0.4)
    o2, l2 = oracle.decode_paged_ref(q, kc.reshape(-1, P, Hkv, D), vc.reshape(-1, P, Hkv, D),
                                     table, lens, 0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_torch_inputs_are_indexed_before_conversion():
    """Torch int8 pages give the same result as their float64 copies."""
    q, kp, vp, table, ln, ks, vs = paged_case(23, 2, 4, 2, 8, 4, [6, 11], int8_k=True,
                                              int8_v=True)
    o1, l1 = oracle.decode_paged_ref(q, kp, vp, table, ln, 0.3, k_scales=ks, v_scales=vs)
    o2, l2 = oracle.decode_paged_ref(
        torch.from_numpy(q), torch.from_numpy(kp).to(torch.int8), torch.from_numpy(vp).to(torch.int8),
        torch.from_numpy(table).to(torch.int32), torch.from_numpy(ln).to(torch.int32), 0.3,
        k_scales=torch.from_numpy(ks), v_scales=torch.from_numpy(vs))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


PAGED_MUTATIONS = {
    "slot_off_by_one": ("page, slot = bt[b, j // P], j % P", "page, slot = bt[b, j // P], (j + 1) % P"),
    "page_off_by_one": ("page, slot = bt[b, j // P], j % P",
                        "page, slot = bt[b, np.minimum(j // P + 1, bt.shape[1] - 1)], j % P"),
    "k_scale_ignored": ("_paged_rows(k_pages, k_scales, page, slot, kv)",
                        "_paged_rows(k_pages, None, page, slot, kv)"),
    "v_scale_for_k": ("_paged_rows(k_pages, k_scales, page, slot, kv)",
                      "_paged_rows(k_pages, v_scales, page, slot, kv)"),
    "no_length_clamp": ("n = max(0, min(lens[b], bt.shape[1] * P))", "n = max(0, lens[b])"),
    "gqa_modulo": ("kv = h // g", "kv = h % Hkv"),
}


@pytest.mark.parametrize("name", sorted(PAGED_MUTATIONS))
def test_planted_mistake_in_paged_decode_is_caught(name):
    old, new = PAGED_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oatt.decode_paged_ref))
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(vars(oatt))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mutant = ns["decode_paged_ref"]
    failed = []
    for pin in PAGED_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {name}"
