"""Pins of the intra-block clustering selector oracle (oracle/cluster_select.py).

Each check compares against something other than the oracle's own formula:
a library k-means (scipy's Lloyd iteration in float64), the pooled block
mean, brute-force token-level attention, closed forms for degenerate blocks,
and the top-k / sampling characterisations.
"""
import math

import numpy as np
import pytest
from scipy.cluster.vq import kmeans2

import oracle
from oracle.reference import F32
from helpers import geometry_of, tiny


def _planted(rng, n, D, C, spread=0.01):
    centers = rng.standard_normal((C, D)) * 4.0
    labels = rng.integers(0, C, n)
    labels[:C] = np.arange(C)                 # every cluster present
    rng.shuffle(labels)
    x = centers[labels] + spread * rng.standard_normal((n, D))
    return x.astype(np.float32), labels


def _same_partition(a, b):
    """Two labelings describe the same partition (up to renaming)."""
    pairs = set(zip(a.tolist(), b.tolist()))
    return len(pairs) == len(set(a.tolist())) == len(set(b.tolist()))


def test_kmeans_matches_scipy_lloyd_on_separated_clusters():
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(8, 65))
        C = int(rng.integers(2, 6))
        T = int(rng.integers(1, 5))
        x, labels = _planted(rng, n, 32, C)
        mu, sizes, a = oracle.kmeans_block(x, C, T)
        ce = min(C, n)
        init = np.stack([x[(c * n) // ce] for c in range(ce)]).astype(np.float64)
        cent, lab = kmeans2(x.astype(np.float64), init, iter=T, minit="matrix", missing="raise"
                            if False else "warn")
        # scipy's Lloyd: same init, T rounds; our final assignment against the updated centroids
        d2 = ((x.astype(np.float64)[:, None, :] - cent[None]) ** 2).sum(-1)
        assert np.array_equal(a, d2.argmin(1)), trial
        assert np.array_equal(sizes, np.bincount(a, minlength=ce))
        np.testing.assert_allclose(mu[sizes > 0], cent[sizes > 0], rtol=1e-5, atol=1e-5)


def test_kmeans_recovers_planted_partition():
    rng = np.random.default_rng(1)
    x, labels = _planted(rng, 64, 64, 4, spread=0.001)
    # start from one token of each cluster so Lloyd cannot merge clusters
    order = np.argsort(labels, kind="stable")
    x, labels = x[order], labels[order]
    counts = np.bincount(labels)
    mu, sizes, a = oracle.kmeans_block(x, 4, 3)
    assert _same_partition(a, labels)
    assert sorted(sizes.tolist()) == sorted(counts.tolist())


def test_single_cluster_is_the_pooled_block_mean():
    rng = np.random.default_rng(2)
    for n in (1, 7, 64):
        x = rng.standard_normal((n, 128)).astype(np.float32)
        mu, sizes, a = oracle.kmeans_block(x, 1, 2)
        pooled = oracle.pool_blocks(x[None, None], n, n)[0, 0, 0]
        assert np.array_equal(mu[0], pooled)                        # same order, same roundings
        np.testing.assert_allclose(mu[0], x.astype(np.float64).mean(0), rtol=1e-5, atol=1e-6)
        assert sizes.tolist() == [n]


def test_zero_rounds_keep_the_initial_tokens_and_short_blocks_shrink_c():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 16)).astype(np.float32)
    mu, sizes, a = oracle.kmeans_block(x, 4, 0)
    assert np.array_equal(mu, x[[0, 2, 5, 7]])
    mu, sizes, a = oracle.kmeans_block(x[:3], 8, 2)               # C_eff = n = 3
    assert mu.shape[0] == 3 and sizes.tolist() == [1, 1, 1]
    assert np.array_equal(mu, x[:3])


def _geo(S_frames=3, lh=4, lw=6, bq=8, bk=4, D=16, H=2, text=5):
    w = tiny(text_len=text, frames=S_frames, lh=lh, lw=lw, bq=bq, bk=bk, D=D, H=H)
    return geometry_of(w)


def test_importance_rows_sum_to_one_and_are_nonnegative():
    g = _geo()
    rng = np.random.default_rng(4)
    q = rng.standard_normal((g.B, g.H, g.seq_alloc, g.head_dim)).astype(np.float32)
    k = rng.standard_normal((g.B, g.H, g.seq_alloc, g.head_dim)).astype(np.float32)
    kp = oracle.pool_blocks(k, g.S, g.k_block)
    for C, T in ((1, 1), (3, 2), (8, 4)):
        I = oracle.cluster_importance(q, kp, g, C, T, log_cluster=True)
        assert (I >= 0).all()
        np.testing.assert_allclose(I.astype(np.float64).sum(-1), 1.0, atol=2e-6)


def test_single_cluster_importance_is_the_softmax_of_the_block_logits():
    g = _geo()
    rng = np.random.default_rng(5)
    q = rng.standard_normal((g.B, g.H, g.seq_alloc, g.head_dim)).astype(np.float32)
    k = rng.standard_normal((g.B, g.H, g.seq_alloc, g.head_dim)).astype(np.float32)
    qp = oracle.pool_blocks(q, g.S, g.q_block)
    kp = oracle.pool_blocks(k, g.S, g.k_block)
    I = oracle.cluster_importance(q, kp, g, 1, 1, log_cluster=True)
    z = oracle.block_logits(qp, kp, g.k_block_tokens(), True).astype(np.float64)
    ref = np.exp(z - z.max(-1, keepdims=True))
    ref /= ref.sum(-1, keepdims=True)
    np.testing.assert_allclose(I, ref, rtol=2e-6, atol=1e-7)


def test_importance_is_the_block_mean_of_token_attention_mass():
    """One cluster per token, keys identical within each key block, cluster-size
    term on: the mixture equals the attention mass every query token puts on
    each key block in plain token-level softmax attention, averaged over the
    block's queries (brute force, float64)."""
    g = _geo(S_frames=2, lh=4, lw=5, bq=8, bk=4, D=16, H=1, text=3)
    rng = np.random.default_rng(6)
    q = (0.7 * rng.standard_normal((1, 1, g.seq_alloc, g.head_dim))).astype(np.float32)
    kb = rng.standard_normal((g.nkb, g.head_dim)).astype(np.float32)
    k = np.zeros((1, 1, g.seq_alloc, g.head_dim), np.float32)
    k[0, 0, :g.S] = kb[np.arange(g.S) // g.k_block]
    kp = kb[None, None]                       # the block summaries are the blocks' (shared) keys
    I = oracle.cluster_importance(q, kp, g, g.q_block, 1, log_cluster=True)
    Q = q[0, 0, :g.S].astype(np.float64)
    K = k[0, 0, :g.S].astype(np.float64)
    logits = Q @ K.T / math.sqrt(g.head_dim)
    a = np.exp(logits - logits.max(1, keepdims=True))
    a /= a.sum(1, keepdims=True)
    mass = np.stack([a[:, (np.arange(g.S) // g.k_block) == j].sum(1) for j in range(g.nkb)], 1)
    for i in range(g.nqb):
        lo, hi = i * g.q_block, min((i + 1) * g.q_block, g.S)
        np.testing.assert_allclose(I[0, 0, i], mass[lo:hi].mean(0), rtol=5e-6, atol=1e-7)


def test_importance_weights_clusters_by_their_token_share():
    """Tokens drawn from a few exact points (uneven counts): the importance is the
    token-share-weighted mixture of the points' softmaxes (float64 reference)."""
    g = _geo(S_frames=1, lh=8, lw=8, bq=64, bk=8, D=32, H=1, text=0)
    rng = np.random.default_rng(11)
    pts = (3.0 * rng.standard_normal((3, g.head_dim))).astype(np.float32)
    lab = np.array([0] * 40 + [1] * 16 + [2] * 8)
    rng.shuffle(lab)
    q = pts[lab][None, None].astype(np.float32)
    kp = rng.standard_normal((1, 1, g.nkb, g.head_dim)).astype(np.float32)
    I = oracle.cluster_importance(q, kp, g, 3, 4, log_cluster=False)
    ref = np.zeros(g.nkb)
    for c, m in zip(range(3), (40, 16, 8)):
        z = (pts[c].astype(np.float64) @ kp[0, 0].astype(np.float64).T) / math.sqrt(g.head_dim)
        e = np.exp(z - z.max())
        ref += (m / 64.0) * e / e.sum()
    np.testing.assert_allclose(I[0, 0, 0], ref, rtol=1e-5, atol=1e-7)


def test_identical_tokens_give_one_cluster_for_any_c():
    g = _geo()
    rng = np.random.default_rng(7)
    q = np.repeat(rng.standard_normal((g.B, g.H, 1, g.head_dim)), g.seq_alloc, axis=2).astype(np.float32)
    k = rng.standard_normal((g.B, g.H, g.seq_alloc, g.head_dim)).astype(np.float32)
    kp = oracle.pool_blocks(k, g.S, g.k_block)
    # the token itself as the only representative (no update rounds)
    one = oracle.cluster_importance(q, kp, g, 1, 0, log_cluster=False)
    for C in (2, 5):
        # all tokens join the first centroid (all distances equal): the same rows
        assert np.array_equal(oracle.cluster_importance(q, kp, g, C, 0, log_cluster=False), one)
        # with update rounds the mean of equal tokens may differ from them by rounding only
        np.testing.assert_allclose(oracle.cluster_importance(q, kp, g, C, 2, log_cluster=False), one,
                                   rtol=1e-5, atol=1e-7)


def test_select_blocks_top_k_and_overrides():
    g = _geo()
    rng = np.random.default_rng(8)
    I = rng.random((g.B, g.H, g.nqb, g.nkb)).astype(np.float32)
    I[0, 0, 1, :4] = F32(0.5)                                      # ties
    p = oracle.MaskParams(mode="topk", topk=3, frame0_dense=True, text_columns=True)
    mask, cnt, idx, logw = oracle.select_blocks(I, g, p)
    f0 = set(g.frame0_q_blocks())
    text = set(g.text_k_blocks())
    for h in range(g.H):
        for i in range(g.nqb):
            js = set(np.nonzero(mask[0, h, i])[0].tolist())
            if i in f0:
                assert js == set(range(g.nkb))
                continue
            order = sorted(range(g.nkb), key=lambda j: (-float(I[0, h, i, j]), j))
            assert js == set(order[:3]) | text
            assert cnt[0, h, i] == len(js) and idx[0, h, i, :cnt[0, h, i]].tolist() == sorted(js)
    assert (logw == 0).all()


def test_sampling_from_weights_matches_sampling_from_logits():
    """Weights exp_spec(z - max z) sample exactly as the logits they come from."""
    rng = np.random.default_rng(9)
    for trial in range(40):
        n = int(rng.integers(4, 200))
        z = (2.0 * rng.standard_normal(n)).astype(np.float32)
        E = F32(rng.uniform(0.5, n * 0.6))
        w = oracle.exp_spec(z - z.max())
        s1, l1 = oracle.select_sample(z, E, 11, trial)
        s2, l2 = oracle.select_sample_weights(w, E, 11, trial)
        if s1.sum() == 1 and (l1 == 0).all() and s1[int(np.argmax(z))]:
            continue                                                  # safeguard rows may differ on ties
        assert np.array_equal(s1, s2) and np.array_equal(l1, l2)


def test_water_fill_sums_to_expected_and_caps_at_one():
    rng = np.random.default_rng(10)
    for trial in range(50):
        n = int(rng.integers(2, 300))
        e = rng.random(n).astype(np.float32) ** 4
        E = F32(rng.uniform(0.2, n))
        pi = oracle.water_fill(e, E)
        assert (pi <= 1).all() and (pi >= 0).all()
        if float(E) < n:
            assert abs(float(pi.astype(np.float64).sum()) - float(E)) <= 1e-4 * max(1.0, float(E))
            free = pi < 1
            if free.sum() >= 2:
                r = pi[free].astype(np.float64) / e[free].astype(np.float64)
                np.testing.assert_allclose(r, r[0], rtol=1e-6)            # proportional where uncapped
