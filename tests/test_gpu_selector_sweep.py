"""Seeded random geometries through both selectors, against the oracle.

Each case draws a ragged geometry (up to 12 frames of 40x40 tokens, so rows
of up to about 1200 key blocks reach the 32-slot selection kernel), a
clustering selector (C <= 4 clusters, T <= 3 rounds) whose importance must
equal the oracle's bit for bit, and top-p over a random domain, p,
value-aware scores and overrides on that importance: masks, counts and
lists identical, head entropies within 1e-9.  A case whose entropy-median
split is closer than 1e-9 (relative) leaves the split-dependent domains'
masks uncompared: both sides may route such heads either way.
"""
import sys

import numpy as np
import pytest

import oracle
import oracle.domains as dm
from helpers import geometry_of, inputs_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(w, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if w.dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def _case(seed, large):
    rng = np.random.default_rng(seed)
    bq = int(rng.choice([32, 64]))
    bk = int(rng.choice([16, 32, 64]))
    D = int(rng.choice([64, 128]))
    fmax, lmin, lmax = (13, 8, 41) if large else (7, 1, 17)
    w = tiny(text_len=int(rng.integers(0, 200)), frames=int(rng.integers(1, fmax)), lh=int(rng.integers(lmin, lmax)),
             lw=int(rng.integers(lmin, lmax)), bq=bq, bk=bk, D=D, H=int(rng.integers(1, 6)), B=int(rng.integers(1, 3)),
             dtype=str(rng.choice(["bf16", "f32"])), mode="topk", topk=0, keep_ratio=0.2,
             log_cluster=bool(rng.integers(0, 2)), centroids=8, grid=(2, 4), align=int(max(bq, bk) * rng.integers(1, 3)))
    C = int(rng.integers(1, 5))
    T = int(rng.integers(0, 4))
    domain = str(rng.choice(["row", "head", "split", "all", "eg"]))
    p = float(rng.choice([0.5, 0.9, 0.97, 1.0]))
    return w, C, T, domain, p, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


@pytest.mark.parametrize("large", [False, True])
@pytest.mark.parametrize("k", range(12))
def test_selectors_random_geometry(k, large):
    w, C, T, domain, p, va, f0, tx = _case((8000 if large else 7000) + k, large)
    g = geometry_of(w)
    if C * g.nkb > 16384:
        C = 1
    print(f"[gpu] selector sweep #{k} large={large}: B={w.B} H={w.H} S={g.S} nkb={g.nkb} D={w.D} {w.dtype} "
          f"C={C} T={T} {domain} p={p} va={va} f0={f0} tx={tx}", flush=True)
    sys.stdout.flush()
    q, k_, v = inputs_of(w)
    gg = bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D, w.q_block, w.k_block,
                      w.seq_alloc)
    qd, kd, vd = _dev(w, q), _dev(w, k_), _dev(w, v)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    vp = bsa.bsa_pool_blocks(vd, gg, gg.k_block)
    P = bsa.bsa_cluster_importance(qd, kp, gg, C, T, w.log_cluster)
    torch.cuda.synchronize()
    oP = oracle.cluster_importance(q, oracle.pool_blocks(k_, g.S, g.k_block), g, C, T, w.log_cluster)
    assert np.array_equal(P.cpu().numpy(), oP)
    mask, cnt, idx, ent = bsa.bsa_select_top_p(P, gg, domain=domain, top_p=p, v_pooled=vp, value_aware=va,
                                               entropy_eps=1e-12, frame0_dense=f0, text_columns=tx)
    torch.cuda.synchronize()
    om, ocnt, oidx, oent = dm.select_top_p(P.cpu().numpy(), g, domain, p, vp=vp.cpu().numpy() if va else None,
                                           eps=1e-12, frame0_dense=f0, text_columns=tx)
    np.testing.assert_allclose(ent.cpu().numpy(), oent, rtol=1e-9, atol=1e-300)
    if domain in ("split", "eg") and g.H >= 2:
        srt = np.sort(oent, axis=1)
        if not (srt[:, g.H // 2] - srt[:, g.H // 2 - 1] > 1e-9 * np.abs(srt).max()).all():
            return
    assert np.array_equal(mask.cpu().numpy().astype(bool), om)
    c = cnt.cpu().numpy()
    assert np.array_equal(c, ocnt)
    ih = idx.cpu().numpy()
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.nqb):
                n = ocnt[b, h, i]
                assert np.array_equal(ih[b, h, i, :n], oidx[b, h, i, :n]), (b, h, i)
