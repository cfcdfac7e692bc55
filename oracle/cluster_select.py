"""Intra-block clustering selector: CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module; the library never imports, links or runs it.

Source: "AB-Attention: accurate block-sparse attention for video diffusion"
(AB-Attention page), TL;DR item 1 and the flowchart's "intra-block cluster"
box: the queries of each query block are clustered only within that block
(no token permutation), and the clusters' representatives give a faithful
importance of every key block; blocks are then selected (top-k) or sampled
in proportion to that importance (TL;DR item 2).  The cluster-size-weighted
softmax of a representative against the key-block summaries is the
EG-Sparse page's Eq. 2 (P', the attention mass a representative query puts
on a whole key cluster), as in ``reference.block_logits``.

The pages fix neither the clustering algorithm's details nor how the
clusters' scores combine into one block importance.  The readings taken
here, the plainest ones the rest supports:

* k-means (Lloyd) on the block's valid query tokens, squared Euclidean
  distance, C clusters (C_eff = min(C, n_i) for a short block), initial
  centroid c = token floor(c * n_i / C_eff) of the block, T rounds of
  (assign, update), then one final assignment that gives the cluster sizes;
  a token goes to the nearest centroid, the lowest index among equals; an
  empty cluster keeps its centroid and carries no weight.
* The importance of key block j for query block i is the expected attention
  mass a query of the block puts on j: the mixture over clusters of P'_c,j,
  each weighted by its share m_c / n_i of the block's tokens.  With C = 1
  and T >= 1 it is P' of the block mean, the summary the plain selector
  ranks.

Every step that decides an integer (the assignment, the ranking of the
importance, a Bernoulli draw) is written out in float32 with each rounding
and the operation order fixed, because the GPU takes the same decisions.
"""
from __future__ import annotations

import numpy as np

from .reference import (F32, Geometry, MaskParams, block_logits, exp_spec, fold_sum,
                        sample_uniforms, select_topk, topk_count)


def kmeans_block(x: np.ndarray, C: int, T: int):
    """Lloyd k-means of one block's query tokens, float32 with written-out order.

    ``x``: [n, D] float32 tokens (n >= 1).  Distance of token t to centroid
    c: ``acc = 0; for d ascending: diff = fl32(x_t,d - mu_c,d);
    acc = fl32(acc + fl32(diff * diff))`` (no fused multiply-add).  Update of
    a non-empty cluster: ``acc = 0; for its tokens t ascending:
    acc = fl32(acc + x_t)``, then ``mu_c = fl32(acc / m_c)``.
    Returns (centroids [C_eff, D], sizes [C_eff], assignment [n]).
    """
    x = np.asarray(x, dtype=F32)
    n, D = x.shape
    ce = min(C, n)
    mu = np.stack([x[(c * n) // ce].copy() for c in range(ce)]).astype(F32)

    def assign(mu):
        dist = np.zeros((n, ce), dtype=F32)
        for d in range(D):
            diff = x[:, d][:, None] - mu[:, d][None, :]
            dist = dist + diff * diff
        return np.argmin(dist, axis=1)          # first minimum: lowest cluster index

    for _ in range(T):
        a = assign(mu)
        for c in range(ce):
            members = np.nonzero(a == c)[0]
            if len(members) == 0:
                continue
            acc = np.zeros(D, dtype=F32)
            for t in members:
                acc = acc + x[t]
            mu[c] = acc / F32(len(members))
    a = assign(mu)
    sizes = np.bincount(a, minlength=ce).astype(np.int64)
    return mu, sizes, a


def block_softmax(z: np.ndarray) -> np.ndarray:
    """P' of one row of logits: e_j = exp_spec(z_j - max z), p_j = fl32(e_j / fold_sum(e))."""
    z = np.asarray(z, dtype=F32)
    e = exp_spec(z - z.max())
    return (e / fold_sum(e)).astype(F32)


def cluster_importance(q: np.ndarray, kp: np.ndarray, g: Geometry, C: int, T: int,
                       log_cluster: bool, rows=None) -> np.ndarray:
    """Block importance I [B, H, nqb, nkb] float32 from intra-block clusters.

    For query block i (n_i valid tokens of ``q``, [B, H, seq_alloc, D]) and
    its clusters c (centroid mu_c, m_c tokens, m_c > 0, ascending c):
    ``I_j = sum_c fl32(fl32(m_c / n_i) * P'_c,j)``, accumulated in fp32 in
    that order, with ``P'_c = block_softmax(block_logits(mu_c, k̄))``.
    ``rows``, if given, is a list of (b, h, i); other rows stay 0.
    """
    q = np.asarray(q, dtype=F32)
    n_k = g.k_block_tokens()
    I = np.zeros((g.B, g.H, g.nqb, g.nkb), dtype=F32)
    if rows is None:
        rows = [(b, h, i) for b in range(g.B) for h in range(g.H) for i in range(g.nqb)]
    for (b, h, i) in rows:
        lo = i * g.q_block
        n = min(g.q_block, g.S - lo)
        mu, sizes, _ = kmeans_block(q[b, h, lo:lo + n], C, T)
        z = block_logits(mu[None, None], kp[b:b + 1, h:h + 1], n_k, log_cluster)[0, 0]
        acc = np.zeros(g.nkb, dtype=F32)
        for c in range(mu.shape[0]):
            if sizes[c] == 0:
                continue
            w = F32(F32(sizes[c]) / F32(n))
            acc = acc + w * block_softmax(z[c])
        I[b, h, i] = acc
    return I


def water_fill(e: np.ndarray, expected: np.float32) -> np.ndarray:
    """Inclusion probabilities pi_j = min(1, c * e_j) with sum pi = E, from weights e >= 0.

    The same water-filling as ``reference.inclusion_probabilities``, applied
    to given weights instead of exp(z - max z).
    """
    e = np.asarray(e, dtype=F32)
    n = e.shape[0]
    if float(expected) >= n:
        return np.ones(n, dtype=F32)
    capped = np.zeros(n, dtype=bool)
    while True:
        sigma = fold_sum(np.where(capped, F32(0.0), e))
        num = F32(expected) - F32(capped.sum())
        c = F32(num / sigma) if (num > 0 and sigma > 0) else F32(0.0)
        grown = capped | (c * e >= F32(1.0))
        if np.array_equal(grown, capped):
            break
        capped = grown
    return np.where(capped, F32(1.0), c * e).astype(F32)


def select_sample_weights(w_row: np.ndarray, expected: np.float32, seed: int, row_id: int):
    """Importance sampling of one row from weights: (selected bool, log-weight by j).

    As ``reference.select_sample`` with pi from ``water_fill(w_row)``; the
    safeguard keeps the first block of largest weight.
    """
    w_row = np.asarray(w_row, dtype=F32)
    pi = water_fill(w_row, expected)
    u = sample_uniforms(seed, row_id, w_row.shape[0])
    sel = u < pi
    logw = np.zeros(w_row.shape[0], dtype=F32)
    if not sel.any():
        sel[int(np.argmax(w_row))] = True
        return sel, logw
    logw[sel] = (-np.log(pi[sel].astype(np.float64))).astype(F32)
    logw[sel & (pi >= F32(1.0))] = F32(0.0)
    return sel, logw


def select_blocks(I: np.ndarray, g: Geometry, p: MaskParams, rows=None):
    """Mask and compacted lists from a block-importance matrix.

    Selection on every requested row by ``p.mode``: "topk" keeps the k
    largest I (lower j first among equals), "sample" samples with
    inclusion probabilities proportional to I; then the frame-0 rows and
    the text columns as in ``reference.build_mask``.  Returns (mask, cnt,
    idx, logw) with the layouts of ``reference.build_mask``.
    """
    B, H, nqb, nkb = g.B, g.H, g.nqb, g.nkb
    I = np.asarray(I, dtype=F32)
    mask = np.zeros((B, H, nqb, nkb), dtype=bool)
    wj = np.zeros((B, H, nqb, nkb), dtype=F32)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nqb)]
    rows = list(rows)
    dense_rows = set(g.frame0_q_blocks()) if p.frame0_dense else set()
    text_cols = list(g.text_k_blocks()) if p.text_columns else []
    k = topk_count(nkb, p.topk, p.keep_ratio)
    expected = F32(p.keep_ratio * nkb)
    for (b, h, i) in rows:
        if i in dense_rows:
            mask[b, h, i, :] = True
            continue
        if p.mode == "topk":
            mask[b, h, i] = select_topk(I[b, h, i], k)
        elif p.mode == "sample":
            sel, lw = select_sample_weights(I[b, h, i], expected, p.seed, (b * H + h) * nqb + int(i))
            mask[b, h, i] = sel
            wj[b, h, i] = lw
        else:
            raise ValueError(p.mode)
        for j in text_cols:
            mask[b, h, i, j] = True
            wj[b, h, i, j] = F32(0.0)
    cnt = np.zeros((B, H, nqb), dtype=np.int32)
    idx = np.full((B, H, nqb, nkb), -1, dtype=np.int32)
    logw = np.zeros((B, H, nqb, nkb), dtype=F32)
    for (b, h, i) in rows:
        js = np.nonzero(mask[b, h, i])[0]
        cnt[b, h, i] = len(js)
        idx[b, h, i, :len(js)] = js
        logw[b, h, i, :len(js)] = wj[b, h, i, js]
    return mask, cnt, idx, logw
