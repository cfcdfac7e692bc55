"""Pins of the mask overrides, the compacted lists and the token-expanded attention."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.reference import F32
from helpers import geometry_of, inputs_of, params_of, tiny


def _lists_all_true(g):
    cnt = np.full((g.B, g.H, g.nqb), g.nkb, np.int32)
    idx = np.broadcast_to(np.arange(g.nkb, dtype=np.int32), (g.B, g.H, g.nqb, g.nkb)).copy()
    return cnt, idx, np.zeros(idx.shape, np.float32)


def _mask_for(w, **over):
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    p = params_of(w)
    if over:
        p = oracle.MaskParams(**{**p.__dict__, **over})
    qp = oracle.pool_blocks(q, g.S, g.q_block)
    kp = oracle.pool_blocks(k, g.S, g.k_block)
    return g, (q, k, v), (qp, kp), p, oracle.build_mask(qp, kp, g, p)


# ----------------------------------------------------------------- overrides and lists
def test_frame0_rows_dense_and_other_rows_are_plain_topk():
    w = tiny(text_len=5, frames=3, lh=3, lw=5, bq=8, bk=8, H=2, topk=2)
    g, _, (qp, kp), p, (mask, cnt, idx, logw) = _mask_for(w)
    f0 = list(g.frame0_q_blocks())
    assert f0 == [0, 1, 2]
    z = oracle.block_logits(qp, kp, g.k_block_tokens(), False)
    plain = oracle.select_topk(z, 2)
    for i in range(g.nqb):
        if i in f0:
            assert mask[:, :, i].all()
        else:
            assert np.array_equal(mask[:, :, i], plain[:, :, i])
    # override off -> every row is the plain top-k
    _, _, _, _, (mask2, _, _, _) = _mask_for(w, frame0_dense=False)
    assert np.array_equal(mask2, plain)


def test_text_columns_added_without_reducing_budget():
    w = tiny(text_len=20, frames=3, lh=3, lw=5, bq=8, bk=8, H=2, topk=2, text_columns=True)
    g, _, (qp, kp), p, (mask, cnt, idx, logw) = _mask_for(w)
    tk = list(g.text_k_blocks())
    assert tk == [0, 1, 2]
    z = oracle.block_logits(qp, kp, g.k_block_tokens(), False)
    plain = oracle.select_topk(z, 2)
    for i in range(g.nqb):
        if i in g.frame0_q_blocks():
            continue
        assert mask[:, :, i, tk].all()
        expect = plain[:, :, i].copy()
        expect[:, :, tk] = True
        assert np.array_equal(mask[:, :, i], expect)


def test_lists_are_ascending_and_consistent_with_mask():
    w = tiny(text_len=3, frames=4, lh=4, lw=4, bq=8, bk=8, H=3, topk=3)
    g, _, _, _, (mask, cnt, idx, logw) = _mask_for(w)
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.nqb):
                c = cnt[b, h, i]
                assert c == mask[b, h, i].sum() and c >= 1
                lst = idx[b, h, i, :c]
                assert np.all(np.diff(lst) > 0) and lst.min() >= 0 and lst.max() < g.nkb
                assert mask[b, h, i, lst].all()
                assert np.all(idx[b, h, i, c:] == -1)
    assert np.all(logw == 0)


def test_sampled_mask_rows_nonempty_and_weights():
    w = tiny(text_len=3, frames=4, lh=4, lw=8, bq=16, bk=4, H=2, mode="sample", topk=0,
             keep_ratio=0.2, sample_seed=11)
    g, _, (qp, kp), p, (mask, cnt, idx, logw) = _mask_for(w)
    z = oracle.block_logits(qp, kp, g.k_block_tokens(), False)
    E = F32(0.2 * g.nkb)
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.nqb):
                c = cnt[b, h, i]
                assert c >= 1
                if i in g.frame0_q_blocks():
                    assert c == g.nkb and np.all(logw[b, h, i, :c] == 0)
                    continue
                pi, _ = oracle.inclusion_probabilities(z[b, h, i], E)
                js = idx[b, h, i, :c]
                wexp = np.where(pi[js] >= 1, 0.0, -np.log(pi[js].astype(np.float64)))
                if c == 1 and pi[js[0]] < 1 and logw[b, h, i, 0] == 0:
                    continue       # safeguard row
                assert np.allclose(logw[b, h, i, :c], wexp, atol=1e-6)


# ----------------------------------------------------------------- attention
def test_all_true_mask_equals_sdpa():
    w = tiny(text_len=5, frames=2, lh=3, lw=5, bq=8, bk=8, D=16, H=2)
    g = geometry_of(w)
    q, k, v = inputs_of(w, pad_value=np.nan)
    O, L = oracle.attention(q, k, v, g, *_lists_all_true(g))
    S = g.S
    qt, kt, vt = (torch.from_numpy(a[:, :, :S].astype(np.float64)) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(F32(1 / math.sqrt(16)))).numpy()
    assert np.allclose(O[:, :, :S], ref, atol=1e-12, rtol=1e-10)
    assert np.all(O[:, :, S:] == 0) and np.all(np.isneginf(L[:, :, S:]))
    logits = torch.einsum("bhqd,bhkd->bhqk", qt, kt) * float(F32(0.25))
    assert np.allclose(L[:, :, :S], torch.logsumexp(logits, -1).numpy(), atol=1e-12)


def test_value_ones_gives_ones_and_log_weight_shift_invariance():
    w = tiny(text_len=4, frames=3, lh=4, lw=4, bq=8, bk=8, D=16, H=2, topk=2)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    ones = np.ones_like(v)
    O1, _ = oracle.attention(q, k, ones, g, cnt, idx, logw)
    assert np.allclose(O1[:, :, :g.S], 1.0, atol=1e-12)
    O, L = oracle.attention(q, k, v, g, cnt, idx, logw)
    rng = np.random.default_rng(0)
    shift = rng.standard_normal((g.B, g.H, g.nqb, 1)).astype(np.float32)
    valid = np.arange(g.nkb)[None, None, None, :] < cnt[..., None]
    O2, L2 = oracle.attention(q, k, v, g, cnt, idx, np.where(valid, logw + shift, 0).astype(np.float32))
    assert np.allclose(O2, O, atol=1e-12)
    tok_shift = np.repeat(shift[..., 0], g.q_block, axis=2)[:, :, :g.S]
    assert np.allclose(L2[:, :, :g.S], L[:, :, :g.S] + tok_shift, atol=1e-10)


def test_log_weight_ln2_equals_duplicated_block():
    """w = ln 2 on block j0 is attention in which block j0's keys appear twice."""
    w = tiny(text_len=0, frames=2, lh=4, lw=6, bq=8, bk=8, D=8, H=1, topk=3, frame0_dense=False)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    i = 2
    c = cnt[0, 0, i]
    j0 = idx[0, 0, i, 1]
    lw = logw.copy()
    lw[0, 0, i, 1] = F32(math.log(2.0))
    O, _ = oracle.attention_head(q[0, 0], k[0, 0], v[0, 0], g, cnt[0, 0], idx[0, 0], lw[0, 0], q_blocks=[i])
    keys = [u for j in idx[0, 0, i, :c] for u in range(j * 8, min(j * 8 + 8, g.S))]
    keys += list(range(j0 * 8, min(j0 * 8 + 8, g.S)))
    K = k[0, 0, keys].astype(np.float64)
    V = v[0, 0, keys].astype(np.float64)
    Q = q[0, 0, i * 8:(i + 1) * 8].astype(np.float64)
    s = Q @ K.T * float(F32(1 / math.sqrt(8)))
    pr = np.exp(s - s.max(1, keepdims=True))
    ref = (pr / pr.sum(1, keepdims=True)) @ V
    assert np.allclose(O, ref, atol=1e-12)


def test_bruteforce_token_loops():
    w = tiny(text_len=3, frames=2, lh=3, lw=5, bq=4, bk=8, D=4, H=1, topk=2)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    lw = logw.copy()
    rng = np.random.default_rng(1)
    lw[cnt[..., None] > np.arange(g.nkb)] = rng.standard_normal((cnt.sum(),)).astype(np.float32)
    O, L = oracle.attention(q, k, v, g, cnt, idx, lw)
    sc = float(F32(0.5))
    for t in range(g.S):
        i = t // g.q_block
        terms = []
        for pos in range(cnt[0, 0, i]):
            j = idx[0, 0, i, pos]
            for u in range(j * g.k_block, min(g.S, (j + 1) * g.k_block)):
                s = sum(float(q[0, 0, t, d]) * float(k[0, 0, u, d]) for d in range(4)) * sc + float(lw[0, 0, i, pos])
                terms.append((s, u))
        m = max(s for s, _ in terms)
        den = sum(math.exp(s - m) for s, _ in terms)
        for d in range(4):
            num = sum(math.exp(s - m) * float(v[0, 0, u, d]) for s, u in terms)
            assert abs(O[0, 0, t, d] - num / den) < 1e-12
        assert abs(L[0, 0, t] - (m + math.log(den))) < 1e-12


def test_frame0_rows_equal_dense_attention_and_nan_pads_ignored():
    w = tiny(text_len=6, frames=3, lh=3, lw=5, bq=8, bk=8, D=16, H=2, topk=2)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    O, L = oracle.attention(q, k, v, g, cnt, idx, logw)
    Od, Ld = oracle.attention(q, k, v, g, *_lists_all_true(g))
    for i in g.frame0_q_blocks():
        sl = slice(i * 8, min((i + 1) * 8, g.S))
        assert np.array_equal(O[:, :, sl], Od[:, :, sl])
    # sparse rows really differ from dense ones
    other = [i for i in range(g.nqb) if i not in g.frame0_q_blocks()]
    assert not np.allclose(O[:, :, other[0] * 8], Od[:, :, other[0] * 8])
    qn, kn, vn = inputs_of(w, pad_value=np.nan)
    On, Ln = oracle.attention(qn, kn, vn, g, cnt, idx, logw)
    assert np.array_equal(On, O) and np.array_equal(Ln, L)


def test_empty_list_row_gives_zero():
    w = tiny(text_len=0, frames=2, lh=4, lw=4, bq=8, bk=8, D=8, H=1, topk=1)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    cnt2 = cnt.copy()
    cnt2[0, 0, 1] = 0
    O, L = oracle.attention(q, k, v, g, cnt2, idx, logw)
    assert np.all(O[0, 0, 8:16] == 0) and np.all(np.isneginf(L[0, 0, 8:16]))


def test_horvitz_thompson_parts_are_unbiased():
    """exp(LSE) and O*exp(LSE) of a sampled row average to their dense values
    (AB-Attention page: one pass is an unbiased estimate of dense attention)."""
    w = tiny(text_len=0, frames=2, lh=4, lw=8, bq=8, bk=4, D=8, H=1, mode="sample", topk=0,
             keep_ratio=0.4, frame0_dense=False)
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    qp = oracle.pool_blocks(q, g.S, g.q_block)
    kp = oracle.pool_blocks(k, g.S, g.k_block)
    i = 1
    # this row has a block with pi = 1, so no draw is empty and every draw is
    # a plain Horvitz-Thompson draw (the safeguard never fires)
    z = oracle.block_logits(qp, kp, g.k_block_tokens(), False)[0, 0, i]
    assert oracle.inclusion_probabilities(z, F32(0.4 * g.nkb))[0].max() == 1.0
    _, Ld = oracle.attention_head(q[0, 0], k[0, 0], v[0, 0], g, *[a[0, 0] for a in _lists_all_true(g)], q_blocks=[i])
    Od, _ = oracle.attention_head(q[0, 0], k[0, 0], v[0, 0], g, *[a[0, 0] for a in _lists_all_true(g)], q_blocks=[i])
    den_d = np.exp(Ld)
    num_d = Od * den_d[:, None]
    n = 1500
    den = np.zeros_like(den_d)
    num = np.zeros_like(num_d)
    den2 = np.zeros_like(den_d)
    rows = [(0, 0, i)]
    for s in range(n):
        p = oracle.MaskParams(mode="sample", keep_ratio=0.4, frame0_dense=False, seed=500 + s)
        _, cnt, idx, logw = oracle.build_mask(qp, kp, g, p, rows=rows)
        O, L = oracle.attention_head(q[0, 0], k[0, 0], v[0, 0], g, cnt[0, 0], idx[0, 0], logw[0, 0], q_blocks=[i])
        e = np.exp(L)
        den += e
        den2 += e * e
        num += O * e[:, None]
    mean = den / n
    sd = np.sqrt(np.maximum(den2 / n - mean ** 2, 0) / n)
    assert np.all(np.abs(mean - den_d) <= 5 * sd + 1e-9 * den_d)
    assert np.allclose(num / n, num_d, atol=6 * np.abs(num_d).max() * sd.max() / mean.min() + 0.05 * np.abs(num_d).max())


def test_block_gathered_attention_equals_token_expanded():
    """The block-gathered CPU speed reference is the oracle's softmax: random
    lists (ragged last block), random log-weights, an empty row, pad rows."""
    w = tiny(text_len=5, frames=3, lh=3, lw=7, bq=8, bk=8, D=16, H=2, topk=3)
    g, (q, k, v), _, p, (mask, cnt, idx, logw) = _mask_for(w)
    rng = np.random.default_rng(3)
    lw = logw.copy()
    lw[cnt[..., None] > np.arange(g.nkb)] = rng.standard_normal((cnt.sum(),)).astype(np.float32)
    cnt2 = cnt.copy()
    cnt2[0, 1, 2] = 0
    for b in range(g.B):
        for h in range(g.H):
            O, L = oracle.attention_head(q[b, h], k[b, h], v[b, h], g, cnt2[b, h], idx[b, h], lw[b, h])
            Og, Lg = oracle.attention_head_gathered(q[b, h], k[b, h], v[b, h], g, cnt2[b, h], idx[b, h], lw[b, h])
            assert np.allclose(Og, O, rtol=0, atol=1e-12) and np.array_equal(np.isneginf(Lg), np.isneginf(L))
            fin = np.isfinite(L)
            assert np.allclose(Lg[fin], L[fin], rtol=0, atol=1e-12)
    # the last key block is ragged (S is not a multiple of 8) and is in some list
    assert g.S % g.k_block != 0 and (idx[cnt[..., None] > np.arange(g.nkb)] == g.nkb - 1).any()
