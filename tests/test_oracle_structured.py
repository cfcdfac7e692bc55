"""Pins of the structured mask producers (oracle/structured.py).

The page's own worked example (tests/golden/dhp_example.json), a brute-force
token-level construction of the per-head contexts, and closed forms for the
frame scores.
"""
import json
import os

import numpy as np

import oracle.structured as st
from helpers import geometry_of, tiny


def _golden():
    return json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dhp_example.json")))


def test_dhp_worked_example():
    gd = _golden()
    lh = gd["max_sink_neighbor"]
    rng = np.random.default_rng(0)
    alpha = np.zeros((1, len(lh), 3))
    for h, l in enumerate(lh):                      # a triple whose larger history score is l
        if rng.random() < 0.5:
            alpha[0, h] = [l, l * rng.random(), 1 - l]
        else:
            alpha[0, h] = [l * rng.random(), l, 1 - l]
    cls = st.classify_heads(alpha, gd["n_dummy"])[0]
    assert sorted(np.nonzero(cls == st.DUMMY)[0].tolist()) == gd["dummy_heads"]
    for h in range(len(lh)):
        if cls[h] != st.DUMMY:
            assert cls[h] == (st.SINK if alpha[0, h, 0] > alpha[0, h, 1] else st.NEIGHBOR)
    two = np.array([[gd["step0_neighbor_head"], gd["step0_dummy_head"]]])
    assert st.classify_heads(two, 1)[0].tolist() == [st.NEIGHBOR, st.DUMMY]


def test_hma_worked_example():
    gd = _golden()
    L = gd["window"]
    nb = st.context_frames(st.NEIGHBOR, 10, L, False, False, 21) - {-1}
    sk = st.context_frames(st.SINK, 10, L, False, False, 21) - {-1}
    assert sorted(nb) == gd["neighbor_context_of_frame_10"]
    assert sorted(sk) == gd["sink_context_of_frame_10"]
    assert st.context_frames(st.DUMMY, 10, L, True, False, 21) - {-1} == {9, 10}
    assert st.context_frames(st.DUMMY, 0, L, True, False, 21) - {-1} == {0}


def _brute(g, classes, L, dummy_prev, causal):
    tf = np.array([st.token_frame(g, t) for t in range(g.S)])
    B, H = classes.shape
    out = np.zeros((B, H, g.nqb, g.nkb), dtype=bool)
    for b in range(B):
        for h in range(H):
            c = int(classes[b, h])
            ok = np.zeros((g.S, g.S), dtype=bool)
            for tq in range(g.S):
                fq = tf[tq]
                if fq < 0:
                    ok[tq] = True
                    continue
                for tk in range(g.S):
                    fk = tf[tk]
                    if fk < 0:
                        ok[tq, tk] = True
                    elif c == st.FULL:
                        ok[tq, tk] = (fk <= fq) if causal else True
                    elif c == st.SINK:
                        ok[tq, tk] = fk in (0, fq)
                    elif c == st.NEIGHBOR:
                        ok[tq, tk] = max(0, fq - L + 1) <= fk <= fq
                    else:
                        ok[tq, tk] = fk == fq or (dummy_prev and fk == fq - 1)
            for i in range(g.nqb):
                for j in range(g.nkb):
                    out[b, h, i, j] = ok[i * g.q_block:(i + 1) * g.q_block, j * g.k_block:(j + 1) * g.k_block].any()
    return out


def test_lists_equal_token_level_brute_force():
    # frames of 15 tokens: blocks of 8 straddle frame boundaries; 5 text tokens
    g = geometry_of(tiny(text_len=5, frames=5, lh=3, lw=5, bq=8, bk=4, D=16, H=4))
    classes = np.array([[st.FULL, st.SINK, st.NEIGHBOR, st.DUMMY]])
    for L, dp, causal in ((2, False, False), (3, True, True), (1, True, False)):
        m, cnt, idx = st.structured_lists(g, classes, L, dummy_prev=dp, block_causal=causal)
        assert np.array_equal(m, _brute(g, classes, L, dp, causal)), (L, dp, causal)
        for h in range(4):
            for i in range(g.nqb):
                assert idx[0, h, i, :cnt[0, h, i]].tolist() == np.nonzero(m[0, h, i])[0].tolist()


def test_block_causal_full_heads_and_overrides():
    g = geometry_of(tiny(text_len=0, frames=4, lh=4, lw=4, bq=16, bk=16, D=16, H=1))
    m, _, _ = st.structured_lists(g, np.array([[st.FULL]]), 2, block_causal=True)
    assert np.array_equal(m[0, 0], np.tril(np.ones((4, 4), dtype=bool)))        # one block per frame
    m, _, _ = st.structured_lists(g, np.array([[st.FULL]]), 2)
    assert m.all()
    m, _, _ = st.structured_lists(g, np.array([[st.DUMMY]]), 2, frame0_dense=True)
    assert m[0, 0, 0].all() and np.array_equal(m[0, 0, 1:], np.eye(4, dtype=bool)[1:])


def test_frame_scores_closed_forms():
    g = geometry_of(tiny(text_len=0, frames=6, lh=4, lw=4, bq=16, bk=16, D=16, H=3))
    n = g.nkb
    P = np.zeros((1, 3, g.nqb, n))
    for i in range(g.nqb):
        P[0, 0, i, i] = 1.0                        # all mass on the current frame
        P[0, 1, i, 0] = 1.0                        # all on the sink frame
        P[0, 2, i, :] = 1.0 / n                    # uniform
    a = st.frame_scores(P, g, 3)
    np.testing.assert_allclose(a[0, 0], [0, 0, 1])
    np.testing.assert_allclose(a[0, 1], [1, 0, 0])
    # uniform: frame f >= 1 has 1 sink block, min(2, f-1) neighbor blocks, 1 current block
    ref = np.mean([[1, min(2, f - 1), 1] / np.sum([1, min(2, f - 1), 1]) for f in range(1, 6)], axis=0)
    np.testing.assert_allclose(a[0, 2], ref)
    np.testing.assert_allclose(a.sum(-1), 1.0)
