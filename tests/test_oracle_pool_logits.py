"""Pins of block pooling and block logits against library routines and closed forms."""
import math

import numpy as np
import torch

import oracle
from oracle.reference import F32

U = 2.0 ** -24  # float32 unit roundoff


def _rand(shape, seed=0, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_pool_matches_avg_pool1d_and_ragged_tail():
    B, H, S, D, blk = 2, 3, 45, 16, 8            # 5 full blocks + one of 5 tokens
    Sa = 48
    x = _rand((B, H, Sa, D), 1)
    x[:, :, S:] = np.nan                          # pad rows must never be read
    p = oracle.pool_blocks(x, S, blk)
    assert p.shape == (B, H, 6, D) and p.dtype == np.float32
    xt = torch.from_numpy(x[:, :, :40].astype(np.float64))         # [B,H,40,D]
    ref_full = torch.nn.functional.avg_pool1d(
        xt.permute(0, 1, 3, 2).reshape(B * H * D, 1, 40), blk).reshape(B, H, D, 5).permute(0, 1, 3, 2).numpy()
    ref_tail = x[:, :, 40:S].astype(np.float64).mean(axis=2)
    ref = np.concatenate([ref_full, ref_tail[:, :, None]], axis=2)
    n = np.array([8, 8, 8, 8, 8, 5])
    absx = np.stack([np.abs(x[:, :, i * 8:min(S, i * 8 + 8)].astype(np.float64)).sum(2) for i in range(6)], 2)
    bound = (n[None, None, :, None] - 1) * U * absx / n[None, None, :, None] + U * np.abs(ref) + 1e-30
    assert np.all(np.abs(p - ref) <= bound)


def test_pool_exact_when_partial_sums_are_representable():
    # identical rows with a short mantissa: every partial sum is exact, so the
    # mean of a block (any size) is the row itself
    row = (np.random.default_rng(2).integers(-64, 64, (1, 1, 1, 32)) / 8.0).astype(np.float32)
    x = np.repeat(row, 24, axis=2)
    for blk in (3, 4, 8, 12):
        p = oracle.pool_blocks(x, 24, blk)
        assert np.array_equal(p, np.repeat(row, 24 // blk, axis=2))
    # power-of-two blocks of small integers: the mean is exact
    xi = np.random.default_rng(3).integers(-50, 50, (1, 2, 64, 8)).astype(np.float32)
    p = oracle.pool_blocks(xi, 64, 16)
    assert np.array_equal(p, xi.reshape(1, 2, 4, 16, 8).astype(np.float64).mean(3).astype(np.float32))


def test_pool_sums_in_ascending_token_order():
    # With a block [1e8, 1, -1e8, 1] the ascending float32 sum is
    # ((1e8 + 1) - 1e8) + 1 = 1, a pairwise sum would give 0 or 2.
    x = np.array([1e8, 1.0, -1e8, 1.0], np.float32).reshape(1, 1, 4, 1)
    assert oracle.pool_blocks(x, 4, 4)[0, 0, 0, 0] == np.float32(0.25)


def test_logits_match_float64_matmul():
    B, H, nq, nk, D = 1, 2, 5, 7, 64
    qp = _rand((B, H, nq, D), 4)
    kp = _rand((B, H, nk, D), 5)
    n_k = np.array([16] * 6 + [3])
    for lc in (False, True):
        z = oracle.block_logits(qp, kp, n_k, lc)
        assert z.dtype == np.float32 and z.shape == (B, H, nq, nk)
        dot = np.einsum("bhid,bhjd->bhij", qp.astype(np.float64), kp.astype(np.float64))
        absdot = np.einsum("bhid,bhjd->bhij", np.abs(qp.astype(np.float64)), np.abs(kp.astype(np.float64)))
        ref = dot / math.sqrt(D) + (np.log(n_k)[None, None, None, :] if lc else 0.0)
        bound = (D + 3) * U * absdot / math.sqrt(D) + 4 * U * (np.abs(ref) + np.log(16))
        assert np.all(np.abs(z - ref) <= bound)


def test_logits_scale_and_sign_zero():
    assert oracle.score_scale(64) == np.float32(0.125)
    assert oracle.score_scale(128) == np.float32(1 / math.sqrt(128))
    # a negative subnormal dot product halved underflows to -0; stored as +0
    qp = np.zeros((1, 1, 1, 4), np.float32)
    kp = np.zeros((1, 1, 1, 4), np.float32)
    qp[..., 0] = -np.float32(1.4e-45)
    kp[..., 0] = 1.0
    z = oracle.block_logits(qp, kp, np.array([4]), False)
    assert z[0, 0, 0, 0] == 0 and not np.signbit(z[0, 0, 0, 0])


def test_logits_accumulate_in_ascending_channel_order():
    # products (1e8, 1, -1e8, 1) in channel order: float32 sequential sum is 1
    qp = np.array([1e8, 1.0, -1e8, 1.0], np.float32).reshape(1, 1, 1, 4)
    kp = np.ones((1, 1, 1, 4), np.float32)
    z = oracle.block_logits(qp, kp, np.array([4]), False)
    assert z[0, 0, 0, 0] == np.float32(1.0) * np.float32(0.5)


def test_log_cluster_term_only_shifts_short_blocks():
    # With equal block sizes the ln n_j term is a per-row constant, so the
    # ranking (hence the top-k mask) can change only through the short block.
    rng = np.random.default_rng(7)
    qp = rng.standard_normal((1, 1, 6, 32)).astype(np.float32)
    kp = rng.standard_normal((1, 1, 9, 32)).astype(np.float32)
    n_eq = np.full(9, 16)
    z0 = oracle.block_logits(qp, kp, n_eq, False)
    z1 = oracle.block_logits(qp, kp, n_eq, True)
    assert np.array_equal(oracle.select_topk(z0, 3), oracle.select_topk(z1, 3))
    n_short = n_eq.copy()
    n_short[-1] = 1
    z2 = oracle.block_logits(qp, kp, n_short, True)
    assert np.all(z2[..., -1] < z1[..., -1])          # ln 1 = 0 < ln 16
    assert np.array_equal(z2[..., :-1], z1[..., :-1])
