"""The seeded input generator: determinism, head independence, bf16 rounding."""
import numpy as np
import torch

import workloads as W
from helpers import tiny


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, -3.0e38, 65504.0, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(W.bf16_round(x).view(np.uint32), ref.view(np.uint32))


def test_generator_is_deterministic_and_heads_independent():
    w = tiny(H=3)
    a = W.generate(w)
    b = W.generate(w, heads=range(1, 3))
    for x, y in zip(a, b):
        assert np.array_equal(x[:, 1:], y)
    c = W.generate(w)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)


def test_generator_pad_rows_and_clusters():
    w = W.workload("tiny_f32")
    q, k, v = W.generate(w, pad_value=np.nan)
    assert q.shape == (1, 2, 224, 64)
    assert np.isfinite(q).all()  # S == seq_alloc here
    w2 = tiny()
    q, k, v = W.generate(w2, pad_value=np.nan)
    S = w2.S
    assert np.isnan(q[:, :, S:]).all() and np.isfinite(q[:, :, :S]).all()
    # visual tokens of one patch share a centroid: their mean distance is the noise
    w3 = W.workload("tiny_f32")
    q, k, _ = W.generate(w3)
    t0 = w3.text_len
    same = np.linalg.norm(q[0, 0, t0] - k[0, 0, t0])            # same pixel, same centroid
    other = np.linalg.norm(q[0, 0, t0] - k[0, 0, t0 + 7])        # far patch
    assert same < other
