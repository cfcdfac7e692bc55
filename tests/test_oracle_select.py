"""Pins of top-k, the sampling primitives and the water-filled inclusion probabilities."""
import math

import numpy as np
import pytest

import oracle
from oracle.reference import F32


# ----------------------------------------------------------------- top-k
def _check_topk_characterisation(z, sel, k):
    """The selected set is the unique one with: k members, every member >= every
    non-member, and at equal values members have lower indices."""
    assert sel.sum() == k
    zs, zu = z[sel], z[~sel]
    if zu.size:
        assert zs.min() >= zu.max()
        t = zs.min()
        if zu.max() == t:
            assert np.nonzero(sel & (z == t))[0].max() < np.nonzero(~sel & (z == t))[0].min()


def test_topk_characterisation_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, n + 1))
        z = (rng.integers(-3, 4, n) * 0.5).astype(np.float32)     # many ties
        sel = oracle.select_topk(z[None], k)[0]
        _check_topk_characterisation(z, sel, k)


def test_topk_agrees_with_float64_ranking_except_near_ties():
    rng = np.random.default_rng(1)
    D = 64
    qp = rng.standard_normal((1, 1, 20, D)).astype(np.float32)
    kp = rng.standard_normal((1, 1, 50, D)).astype(np.float32)
    z = oracle.block_logits(qp, kp, np.full(50, 64), False)[0, 0]
    z64 = (qp[0, 0].astype(np.float64) @ kp[0, 0].astype(np.float64).T) / math.sqrt(D)
    bound = (D + 3) * 2.0 ** -24 * (np.abs(qp[0, 0]).astype(np.float64) @ np.abs(kp[0, 0]).astype(np.float64).T) / math.sqrt(D)
    k = 7
    sel = oracle.select_topk(z, k)
    for i in range(20):
        order = np.argsort(-z64[i])
        kth, nxt = z64[i, order[k - 1]], z64[i, order[k]]
        if kth - nxt > 2 * bound[i].max():
            assert set(np.nonzero(sel[i])[0]) == set(order[:k].tolist())


def test_topk_count_and_full_keep():
    assert oracle.topk_count(512, 0, 0.10) == 52
    assert oracle.topk_count(122, 0, 0.25) == 31
    assert oracle.topk_count(1861, 0, 0.08) == 149
    assert oracle.topk_count(7, 2, 0.0) == 2
    assert oracle.topk_count(7, 0, 1e-9) == 1
    assert oracle.topk_count(9, 0, 1.0) == 9
    z = np.random.default_rng(2).standard_normal((3, 9)).astype(np.float32)
    assert oracle.select_topk(z, 9).all()


# ----------------------------------------------------------------- exp
def test_exp_spec_relative_error():
    t = np.concatenate([np.linspace(-86.5, 0.0, 200001), -np.logspace(-8, 1.9, 5000)]).astype(np.float32)
    e = oracle.exp_spec(t)
    ref = np.exp(t.astype(np.float64))
    rel = np.abs(e.astype(np.float64) - ref) / ref
    assert rel.max() < 4 * 2.0 ** -24, rel.max()
    assert oracle.exp_spec(np.float32([0.0]))[0] == np.float32(1.0)
    assert oracle.exp_spec(np.float32([-87.5, -100.0, -1e30]))[:].tolist() == [0.0, 0.0, 0.0]
    assert e.dtype == np.float32


# ----------------------------------------------------------------- Philox
def test_philox_matches_numpy_bit_generator():
    for seed, row, grp in [(0, 1, 0), (3, 7, 5), (2 ** 63 + 11, 123456789, 511), (42, 2 ** 40, 3)]:
        bg = np.random.Philox(key=np.array([seed, 0], np.uint64),
                              counter=np.array([row - 1, grp, 0, 0], np.uint64))   # numpy steps the counter first
        ref = bg.random_raw(4)
        got = oracle.philox4x64_10((row, grp, 0, 0), (seed, 0))
        assert [int(x) for x in ref] == list(got)


def test_sample_uniforms_are_philox_words():
    seed, row, nkb = 9, 33, 10
    u = oracle.sample_uniforms(seed, row, nkb)
    words = []
    for g in range(3):
        words += [int(x) for x in np.random.Philox(key=[seed, 0], counter=[row - 1, g, 0, 0]).random_raw(4)]
    ref = np.array([(w >> 40) / 2.0 ** 24 for w in words[:nkb]], np.float32)
    assert np.array_equal(u, ref)
    big = np.concatenate([oracle.sample_uniforms(1, r, 64) for r in range(1, 200)])
    assert big.min() >= 0 and big.max() < 1
    assert abs(big.mean() - 0.5) < 5 * math.sqrt(1 / 12 / big.size)


# ----------------------------------------------------------------- fold sum
def test_fold_sum_tree_order_and_accuracy():
    # halves-folding tree: (1e8 + -1e8) + (1 + 1) = 2 ; a left-to-right sum gives 1,
    # an adjacent-pairs tree gives 0
    assert oracle.fold_sum(np.float32([1e8, 1, -1e8, 1])) == np.float32(2.0)
    # 5 elements pad to 8: ((a0+a4)+(a2)) + ((a1)+(a3))
    x = np.float32([1e8, 1.0, 1.0, 1.0, -1e8])
    assert oracle.fold_sum(x) == np.float32(((1e8 + -1e8) + 1.0) + (1.0 + 1.0))
    rng = np.random.default_rng(4)
    for n in (1, 2, 7, 64, 1000, 2048):
        v = rng.random(n).astype(np.float32)
        ref = math.fsum(v.astype(np.float64))
        assert abs(float(oracle.fold_sum(v)) - ref) <= math.ceil(math.log2(max(n, 2))) * 2.0 ** -24 * ref + 1e-30
    ints = rng.integers(0, 1000, 300).astype(np.float32)
    assert oracle.fold_sum(ints) == ints.astype(np.int64).sum()


# ----------------------------------------------------------------- inclusion probabilities
def _bisect_pi(e64, E):
    lo, hi = 0.0, 1.0
    while sum(min(1.0, hi * x) for x in e64) < E:
        hi *= 2
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if sum(min(1.0, mid * x) for x in e64) < E:
            lo = mid
        else:
            hi = mid
    return np.minimum(1.0, hi * e64)


@pytest.mark.parametrize("spread,E", [(0.3, 5.0), (3.0, 5.0), (6.0, 12.5), (1.0, 1.0), (8.0, 0.7)])
def test_inclusion_probabilities_match_float64_water_level(spread, E):
    rng = np.random.default_rng(int(spread * 10 + E))
    z = (rng.standard_normal(64) * spread).astype(np.float32)
    pi, e = oracle.inclusion_probabilities(z, F32(E))
    e64 = np.exp(z.astype(np.float64) - z.max())
    ref = _bisect_pi(e64, E)
    assert np.all(np.abs(pi - ref) <= 2e-5 * np.maximum(ref, 1e-3))
    assert abs(pi.astype(np.float64).sum() - E) <= 1e-4 * E
    assert pi.max() <= 1.0 and pi.min() > 0.0
    # monotone in z
    o = np.argsort(z, kind="stable")
    assert np.all(np.diff(pi[o]) >= 0)


def test_inclusion_probabilities_all_kept_when_expected_exceeds_blocks():
    z = np.float32([0.1, 5.0, -3.0])
    pi, _ = oracle.inclusion_probabilities(z, F32(3.0))
    assert pi.tolist() == [1.0, 1.0, 1.0]


def test_sampling_inclusion_frequencies_match_pi():
    rng = np.random.default_rng(5)
    z = (rng.standard_normal(32) * 2).astype(np.float32)
    E = F32(6.0)
    pi, _ = oracle.inclusion_probabilities(z, E)
    n = 3000
    hits = np.zeros(32)
    for s in range(n):
        sel, lw = oracle.select_sample(z, E, seed=1000 + s, row_id=17)
        hits += sel
        # the weight of a kept block is -ln pi, 0 for pi = 1
        assert np.allclose(lw[sel], -np.log(pi[sel].astype(np.float64)), atol=1e-6)
        assert np.all(lw[~sel] == 0)
    freq = hits / n
    sd = np.sqrt(pi * (1 - pi) / n) + 1e-12
    assert np.all(np.abs(freq - pi) <= 5 * sd + 1.0 / n)


def test_empty_row_safeguard_keeps_argmax():
    z = np.float32([0.5, 2.0, 2.0, -1.0, 1.9])
    E = F32(1e-6)                                  # almost surely nothing is drawn
    for s in range(50):
        sel, lw = oracle.select_sample(z, E, seed=s, row_id=3)
        assert sel.sum() >= 1
        if sel.sum() == 1 and lw.sum() == 0:
            assert np.nonzero(sel)[0].tolist() == [1]   # first of the two maxima
