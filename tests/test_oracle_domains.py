"""Pins of the top-p / competition-domain oracle (oracle/domains.py).

Checks against real-arithmetic top-p (float64 cumulative mass of sorted
scores), the threshold's defining property computed with Python integers,
scipy's entropy, numpy's norm and hand-built domains.
"""
import math

import numpy as np
import pytest
from scipy.stats import entropy as scipy_entropy

import oracle.domains as dm
from oracle.reference import F32
from helpers import geometry_of, tiny


def _rows(rng, n_rows, n, sharp=3.0):
    z = sharp * rng.standard_normal((n_rows, n))
    e = np.exp(z - z.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def test_order_keys_and_fixed_mass():
    s = np.array([0.0, 1e-30, 2.0 ** -33, 2.0 ** -32, 0.25, 0.5, 1.0, 3.5], dtype=np.float32)
    k = dm.order_keys(s)
    assert (np.diff(k.astype(np.int64)) > 0).all()
    assert dm.fixed_mass(s).tolist() == [1, 1, 1, 2, 2 ** 30 + 1, 2 ** 31 + 1, 2 ** 32 + 1, 7 * 2 ** 31 + 1]


def test_threshold_has_its_defining_property():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 300))
        s = (rng.random(n) ** 3).astype(np.float32)
        if trial % 3 == 0:
            s = np.round(s * 8).astype(np.float32) / 8          # many ties
        p = float(rng.uniform(0.01, 1.0))
        T = dm.top_p_threshold(s, p)
        keys = [int(x) for x in dm.order_keys(s)]
        mass = [int(math.floor(float(x) * 2.0 ** 32)) + 1 for x in s]
        target = math.ceil(p * sum(mass))
        kept = sum(m for m, k in zip(mass, keys) if k >= T)
        assert T in keys and kept >= target
        above = [k for k in set(keys) if k > T]
        for k2 in above:                                         # every larger score keeps too little
            assert sum(m for m, k in zip(mass, keys) if k >= k2) < target


def test_row_top_p_is_the_smallest_prefix_of_sorted_probabilities():
    rng = np.random.default_rng(1)
    P = _rows(rng, 200, 97)
    checked = 0
    for row in P:
        for p in (0.5, 0.9, 0.99):
            T = dm.top_p_threshold(row, p)
            kept = dm.order_keys(row) >= T
            o = np.argsort(-row.astype(np.float64), kind="stable")
            c = np.cumsum(row[o].astype(np.float64))
            goal = p * c[-1]
            n = int(np.argmax(c >= goal)) + 1                    # shortest prefix reaching p of the mass
            near = abs(c[n - 1] - goal) < 1e-5 or (n >= 2 and abs(c[n - 2] - goal) < 1e-5)
            if near or (n < len(row) and row[o[n - 1]] == row[o[n]]):
                continue                                          # fixed-point rounding could tip it
            assert set(np.nonzero(kept)[0].tolist()) == set(o[:n].tolist())
            checked += 1
    assert checked > 500


def test_value_norms_and_entropy():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((2, 3, 11, 64)).astype(np.float32)
    np.testing.assert_allclose(dm.value_norms(v), np.linalg.norm(v.astype(np.float64), axis=-1), rtol=2e-6)
    P = _rows(rng, 2 * 3 * 5, 13).reshape(2, 3, 5, 13)
    H = dm.head_entropy(P, 1e-20)
    ref = np.array([[np.mean([scipy_entropy(P[b, h, i].astype(np.float64)) for i in range(5)])
                     for h in range(3)] for b in range(2)])
    np.testing.assert_allclose(H, ref, rtol=1e-6)


def test_median_split_and_pool_ids():
    Hs = np.array([[0.5, 0.1, 0.9, 0.1, 0.3, 0.7]])              # tie at 0.1: head 1 before head 3
    pool = dm.head_pools(Hs, "eg")
    assert pool[0].tolist() == [-1, 0, -1, 0, 0, -1]
    assert dm.head_pools(Hs, "split")[0].tolist() == [1, 0, 1, 0, 0, 1]
    assert dm.head_pools(Hs, "row")[0].tolist() == [-1] * 6
    assert dm.head_pools(Hs, "head")[0].tolist() == list(range(6))
    assert dm.head_pools(np.zeros((2, 3)), "all").tolist() == [[0, 0, 0], [1, 1, 1]]


def _geo(H=3, bq=8, bk=8):
    return geometry_of(tiny(text_len=5, frames=3, lh=4, lw=6, bq=bq, bk=bk, D=16, H=H))


def test_domains_row_head_all_and_safeguard():
    g = _geo(H=3)
    rng = np.random.default_rng(3)
    P = _rows(rng, g.H * g.nqb, g.nkb).reshape(1, g.H, g.nqb, g.nkb)
    m, cnt, idx, _ = dm.select_top_p(P, g, "row", 0.8)
    for h in range(g.H):
        for i in range(g.nqb):
            T = dm.top_p_threshold(P[0, h, i], 0.8)
            assert np.array_equal(m[0, h, i], dm.order_keys(P[0, h, i]) >= T)
    # per-head global: one pool per head; a row with almost no mass still keeps one block
    P2 = P.copy()
    P2[0, 1, 2] = (P2[0, 1, 2] * 1e-6).astype(np.float32)
    m2, cnt2, _, _ = dm.select_top_p(P2, g, "head", 0.8)
    assert cnt2[0, 1, 2] == 1 and m2[0, 1, 2, int(np.argmax(P2[0, 1, 2]))]
    flat = P2[0, 0].ravel()
    T = dm.top_p_threshold(flat, 0.8)
    base = (dm.order_keys(P2[0, 0]) >= T)
    assert np.array_equal(m2[0, 0] | ~base, np.ones_like(base))  # head 0: its pool's set plus safeguards
    # all-head global over one head equals per-head global
    one = P[:, :1]
    g1 = _geo(H=1)
    a, _, _, _ = dm.select_top_p(one, g1, "all", 0.7)
    b, _, _, _ = dm.select_top_p(one, g1, "head", 0.7)
    assert np.array_equal(a, b)
    assert (cnt >= 1).all() and (idx[..., 0] >= 0).all()


def test_value_aware_scores_rank_by_output_contribution():
    g = _geo(H=2, bq=64, bk=8)
    P = np.zeros((1, 2, g.nqb, g.nkb), dtype=np.float32)
    P[..., 0] = 0.30
    P[..., 1] = 0.29
    P[..., 2:] = (0.41 / (g.nkb - 2))
    vp = np.zeros((1, 2, g.nkb, 16), dtype=np.float32)
    vp[..., 0, 0] = 0.01                                          # block 0: almost no output
    vp[..., 1, 0] = 10.0
    vp[..., 2:, 0] = 1.0
    m_plain, _, _, _ = dm.select_top_p(P, g, "all", 0.25)
    m_va, _, _, _ = dm.select_top_p(P, g, "all", 0.25, vp=vp)
    assert m_plain[0, 0, 0, 0] and not m_plain[0, 0, 0, 1]
    assert m_va[0, 0, 0, 1] and not m_va[0, 0, 0, 0]


def test_overrides_after_selection():
    g = _geo(H=2)
    rng = np.random.default_rng(4)
    P = _rows(rng, g.H * g.nqb, g.nkb).reshape(1, g.H, g.nqb, g.nkb)
    m, cnt, idx, _ = dm.select_top_p(P, g, "eg", 0.5, frame0_dense=True, text_columns=True)
    for i in g.frame0_q_blocks():
        assert m[:, :, i].all()
    for j in g.text_k_blocks():
        assert m[..., j].all()
    for h in range(g.H):
        for i in range(g.nqb):
            assert idx[0, h, i, :cnt[0, h, i]].tolist() == np.nonzero(m[0, h, i])[0].tolist()
