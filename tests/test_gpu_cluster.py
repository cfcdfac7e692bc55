"""GPU parity of the intra-block clustering selector through the C ABI.

Bit-exact: the block importance (every rounding of the k-means, logits,
fixed-order exponentials and tree sums is specified), and the masks, counts
and lists selected from it (log-weights to 2.5e-7 relative, the hardware log).
The forward on those lists within max-abs 2e-2 / mean-abs 2e-3.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import geometry_of, inputs_of, params_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _geo(w):
    return bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D,
                        w.q_block, w.k_block, w.seq_alloc)


def _mp(w):
    return bsa.MaskParams(mode=w.mode, topk=w.topk, keep_ratio=w.keep_ratio,
                          frame0_dense=w.frame0_dense, text_columns=w.text_columns,
                          log_cluster=w.log_cluster, seed=w.sample_seed)


def _dev(w, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if w.dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


CASES = {
    # name: (workload, clusters, rounds)
    "ragged_bf16_k64_topk_c4": (tiny(text_len=45, frames=4, lh=10, lw=14, bq=64, bk=64, D=128, H=2,
                                     dtype="bf16", mode="topk", topk=0, keep_ratio=0.3,
                                     log_cluster=True, centroids=8, grid=(2, 4), align=64), 4, 3),
    "ragged_bf16_k16_sample_c3": (tiny(text_len=37, frames=5, lh=9, lw=13, bq=64, bk=16, D=128, H=2,
                                       dtype="bf16", mode="sample", topk=0, keep_ratio=0.15,
                                       sample_seed=7, centroids=8, grid=(2, 4), align=64), 3, 2),
    "ragged_f32_d64_q32_text_c8": (tiny(text_len=19, frames=3, lh=7, lw=9, bq=32, bk=16, D=64, H=2,
                                        dtype="f32", mode="topk", topk=5, text_columns=True,
                                        centroids=4, grid=(2, 2), align=32), 8, 4),
    "ragged_bf16_k16_topk_c4_long_rows": (tiny(text_len=30, frames=8, lh=20, lw=26, bq=64, bk=16, D=128,
                                               H=2, dtype="bf16", mode="topk", topk=0, keep_ratio=0.1,
                                               log_cluster=True, centroids=16, grid=(4, 4), align=64), 4, 3),
    "ragged_bf16_c1_t0": (tiny(text_len=0, frames=6, lh=10, lw=13, bq=64, bk=32, D=64, H=2,
                               dtype="bf16", mode="sample", topk=0, keep_ratio=0.3, sample_seed=99,
                               frame0_dense=False, centroids=8, grid=(2, 4), align=64), 1, 0),
}


def _run(w, C, T, q, k, v):
    g = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    kp = bsa.bsa_pool_blocks(kd, g, g.k_block)
    imp = torch.full((w.B, w.H, geometry_of(w).nqb, geometry_of(w).nkb), float("nan"), device=qd.device)
    bsa.bsa_cluster_importance(qd, kp, g, C, T, w.log_cluster, out=imp)
    mask, cnt, idx, logw = bsa.bsa_select_blocks(imp, g, _mp(w))
    out, lse = bsa.bsa_forward(qd, kd, vd, g, cnt, idx, logw, want_lse=True)
    torch.cuda.synchronize()
    return dict(kp=kp.cpu().numpy(), imp=imp.cpu().numpy(), mask=mask.cpu().numpy().astype(bool),
                cnt=cnt.cpu().numpy(), idx=idx.cpu().numpy(),
                logw=None if logw is None else logw.cpu().numpy(), out=out.float().cpu().numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_selector_every_row(name):
    w, C, T = CASES[name]
    g = geometry_of(w)
    _say(f"[gpu] cluster {name} S={g.S} nqb={g.nqb} nkb={g.nkb} C={C} T={T} mode={w.mode}")
    q, k, v = inputs_of(w, pad_value=np.nan)
    r = _run(w, C, T, q, k, v)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    assert np.array_equal(r["kp"], okp)
    oimp = oracle.cluster_importance(q, okp, g, C, T, w.log_cluster)
    bad = np.argwhere(r["imp"] != oimp)
    assert bad.size == 0, (name, bad[:5], r["imp"][tuple(bad[0])], oimp[tuple(bad[0])])
    p = params_of(w)
    om, ocnt, oidx, ologw = oracle.select_blocks(oimp, g, p)
    assert np.array_equal(r["mask"], om)
    assert np.array_equal(r["cnt"], ocnt)
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.nqb):
                c = ocnt[b, h, i]
                assert np.array_equal(r["idx"][b, h, i, :c], oidx[b, h, i, :c]), (b, h, i)
                if w.mode == "sample":
                    gw = r["logw"][b, h, i, :c].astype(np.float64)
                    ow = ologw[b, h, i, :c].astype(np.float64)
                    assert np.all(np.abs(gw - ow) <= 2.5e-7 * np.maximum(1.0, np.abs(ow))), (b, h, i)
    errs = []
    for b in range(g.B):
        for h in range(g.H):
            o, _ = oracle.attention_head(q[b, h], k[b, h], v[b, h], g, ocnt[b, h], oidx[b, h], ologw[b, h])
            err = np.abs(r["out"][b, h, :o.shape[0]].astype(np.float64) - o)
            assert err.max() <= 2e-2, (name, b, h, err.max())
            errs.append(err.ravel())
    allerr = np.concatenate(errs)
    _say(f"    importance bit-exact; out max|err| {allerr.max():.3e} mean|err| {allerr.mean():.3e}")
    assert allerr.mean() <= 2e-3


@pytest.mark.parametrize("name", ["wan_1p3b_keep10", "wan_1p3b_sampled_k16"])
def test_cluster_importance_full_size_sampled_rows(name):
    """Full-size geometries (Wan2.1-1.3B-like, 12 heads, 32760 tokens; 64- and
    16-key blocks), four clusters, three rounds: sampled rows against the oracle."""
    w = W.workload(name)
    g = geometry_of(w)
    _say(f"[gpu] cluster full-size {w.name} C=4 T=3")
    q, k, v = inputs_of(w)
    gg = _geo(w)
    qd, kd = _dev(w, q), _dev(w, k)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    imp = bsa.bsa_cluster_importance(qd, kp, gg, 4, 3, w.log_cluster)
    mask, cnt, idx, logw = bsa.bsa_select_blocks(imp, gg, _mp(w))
    torch.cuda.synchronize()
    imp_h = imp.cpu().numpy()
    rng = np.random.default_rng(3)
    rows = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, g.H, 10), rng.integers(0, g.nqb, 10))]
    rows += [(0, 0, 0), (0, g.H - 1, g.nqb - 1)]
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    oimp = oracle.cluster_importance(q, okp, g, 4, 3, w.log_cluster, rows=rows)
    for (b, h, i) in rows:
        assert np.array_equal(imp_h[b, h, i], oimp[b, h, i]), (b, h, i)
    om, ocnt, oidx, _ = oracle.select_blocks(oimp, g, params_of(w), rows=rows)
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    for (b, h, i) in rows:
        c = ocnt[b, h, i]
        assert cnt_h[b, h, i] == c and np.array_equal(idx_h[b, h, i, :c], oidx[b, h, i, :c]), (b, h, i)
    # every row sums to one within rounding (a property at any size)
    assert np.abs(imp_h.astype(np.float64).sum(-1) - 1.0).max() < 1e-5


LONG_ROWS = {
    # name: (workload, clusters, rounds); the row lengths take the register
    # tree of 8, 32 and 64 values per lane, the last at C * nkb = 16384
    "nkb1000_c4": (tiny(text_len=0, frames=4, lh=50, lw=80, bq=64, bk=16, D=64, H=1, dtype="bf16",
                        mode="topk", topk=0, keep_ratio=0.05, centroids=16, grid=(4, 4), align=64), 4, 3),
    "nkb3000_c4": (tiny(text_len=0, frames=6, lh=100, lw=80, bq=64, bk=16, D=64, H=1, dtype="bf16",
                        mode="topk", topk=0, keep_ratio=0.05, centroids=16, grid=(4, 4), align=64), 4, 2),
    "nkb8192_c2": (tiny(text_len=0, frames=8, lh=128, lw=128, bq=64, bk=16, D=64, H=1, dtype="bf16",
                        mode="topk", topk=0, keep_ratio=0.01, centroids=16, grid=(4, 4), align=64), 2, 2),
}


@pytest.mark.parametrize("name", list(LONG_ROWS))
def test_cluster_importance_long_rows(name):
    w, C, T = LONG_ROWS[name]
    g = geometry_of(w)
    _say(f"[gpu] cluster long rows {name} nkb={g.nkb} C={C} T={T}")
    q, k, v = inputs_of(w)
    gg = _geo(w)
    qd, kd = _dev(w, q), _dev(w, k)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    imp = bsa.bsa_cluster_importance(qd, kp, gg, C, T, w.log_cluster)
    torch.cuda.synchronize()
    imp_h = imp.cpu().numpy()
    rows = [(0, 0, i) for i in (0, 1, g.nqb // 3, g.nqb // 2, g.nqb - 2, g.nqb - 1)]
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    oimp = oracle.cluster_importance(q, okp, g, C, T, w.log_cluster, rows=rows)
    for (b, h, i) in rows:
        assert np.array_equal(imp_h[b, h, i], oimp[b, h, i]), (name, b, h, i)
    assert np.abs(imp_h.astype(np.float64).sum(-1) - 1.0).max() < 1e-5


@pytest.mark.parametrize("k", range(6))
def test_cluster_importance_random_geometries(k):
    """Seeded random geometries, cluster counts and rounds: the importance of
    every row bit-exact against the oracle."""
    rng = np.random.default_rng(300 + k)
    bq = int(rng.choice([32, 64]))
    bk = int(rng.choice([16, 32, 64]))
    D = int(rng.choice([64, 128]))
    w = tiny(text_len=int(rng.integers(0, 60)), frames=int(rng.integers(1, 5)), lh=int(rng.integers(3, 12)),
             lw=int(rng.integers(3, 14)), bq=bq, bk=bk, D=D, H=int(rng.integers(1, 4)), B=int(rng.integers(1, 3)),
             dtype=str(rng.choice(["bf16", "f32"])), mode="topk", topk=0, keep_ratio=0.2,
             log_cluster=bool(rng.integers(0, 2)), centroids=8, grid=(2, 4), align=max(bq, bk))
    C, T = int(rng.integers(1, 9)), int(rng.integers(0, 5))
    g = geometry_of(w)
    _say(f"[gpu] cluster random #{k}: S={g.S} D={D} bq={bq} bk={bk} B={w.B} H={w.H} C={C} T={T} {w.dtype}")
    q, kk, v = inputs_of(w)
    r = _run(w, C, T, q, kk, v)
    okp = oracle.pool_blocks(kk, g.S, g.k_block)
    oimp = oracle.cluster_importance(q, okp, g, C, T, w.log_cluster)
    assert np.array_equal(r["imp"], oimp)
