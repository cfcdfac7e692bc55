"""Geometry pins: the frame-0 page's section-4 formula worked out by hand."""
import json
import os

import oracle
import workloads as W
from helpers import geometry_of, params_of


def test_geometry_matches_hand_worked_values(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "geometry.json")))["cases"]
    assert set(gold) == set(W.WORKLOADS)
    for name, exp in gold.items():
        w = W.workload(name)
        g = geometry_of(w)
        assert g.S == exp["S"], name
        assert g.seq_alloc == exp["seq_alloc"], name
        assert g.nqb == exp["nqb"] and g.nkb == exp["nkb"], name
        f0 = g.frame0_q_blocks()
        assert [f0.start, f0.stop - 1] == exp["frame0_q_blocks"], name
        tk = g.text_k_blocks()
        assert (None if len(tk) == 0 else [tk.start, tk.stop - 1]) == exp["text_k_blocks"], name
        assert int(g.k_block_tokens()[-1]) == exp["last_k_block_tokens"], name
        assert g.k_block_tokens().sum() == g.S and g.q_block_tokens().sum() == g.S
        p = params_of(w)
        if "topk" in exp:
            assert oracle.topk_count(g.nkb, p.topk, p.keep_ratio) == exp["topk"], name
        if "expected_keep" in exp:
            assert abs(float(oracle.reference.F32(p.keep_ratio * g.nkb)) - exp["expected_keep"]) < 1e-4


def test_frame0_range_partial_overlap_and_edges():
    # text_len = 10, frame of 3x4 = 12 tokens -> frame 0 is tokens [10, 22).
    g = oracle.Geometry(1, 1, 10, 2, 3, 4, 8, 8, 8, 40)
    # blocks of 8: [0,8) [8,16) [16,24) -> block 1 and 2 overlap frame 0
    assert list(g.frame0_q_blocks()) == [1, 2]
    assert list(g.text_k_blocks()) == [0, 1]
    # no text: frame 0 starts at block 0
    g = oracle.Geometry(1, 1, 0, 2, 3, 4, 8, 8, 8, 24)
    assert list(g.frame0_q_blocks()) == [0, 1]
    assert list(g.text_k_blocks()) == []
    # frame exactly one block
    g = oracle.Geometry(1, 1, 8, 2, 2, 4, 8, 8, 8, 24)
    assert list(g.frame0_q_blocks()) == [1]
