"""GPU parity of the structured mask producers through the C ABI.

Bit-exact: masks, counts and lists of every head class (full with and without
block-causal frames, sink, neighbor, dummy with and without the previous
frame) on ragged geometries whose frames straddle blocks, with text tokens,
dense frame-0 rows and text columns.  Frame attention scores within 1e-9
relative (float64 sums in another order); the head labelling then runs on
the host on the GPU's scores and is compared with the oracle's labelling of
the same scores.  The forward on structured lists is checked against the
oracle's attention.
"""
import sys

import numpy as np
import pytest

import oracle
import oracle.structured as st
import workloads as W
from helpers import geometry_of, inputs_of, tiny

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


def _dev(w, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if w.dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


# frames of 140 tokens over blocks of 64 / 16; 9 frames of 15 over blocks of 32 / 16;
# text spanning more than a block; one frame per block exactly
GEOS = {
    "straddle": tiny(text_len=40, frames=5, lh=10, lw=14, bq=64, bk=16, D=64, H=8, dtype="bf16", align=64),
    "ragged": tiny(text_len=5, frames=9, lh=3, lw=5, bq=32, bk=16, D=64, H=8, B=2, align=32),
    "aligned": tiny(text_len=0, frames=6, lh=4, lw=8, bq=32, bk=32, D=64, H=8, dtype="bf16", align=32),
}


def _classes(B, H, seed):
    rng = np.random.default_rng(seed)
    c = np.stack([rng.permutation(np.arange(H) % 4) for _ in range(B)]).astype(np.int32)
    return c


def _compare(w, cls, window, dummy_prev, causal, frame0, text):
    g = geometry_of(w)
    mask, cnt, idx = bsa.bsa_structured_lists(torch.from_numpy(cls).cuda(), _geo(w), window,
                                              dummy_prev=dummy_prev, block_causal=causal,
                                              frame0_dense=frame0, text_columns=text)
    torch.cuda.synchronize()
    om, ocnt, oidx = st.structured_lists(g, cls, window, dummy_prev, causal, frame0, text)
    assert np.array_equal(mask.cpu().numpy().astype(bool), om)
    c = cnt.cpu().numpy()
    assert np.array_equal(c, ocnt)
    ih = idx.cpu().numpy()
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.nqb):
                n = ocnt[b, h, i]
                assert np.array_equal(ih[b, h, i, :n], oidx[b, h, i, :n]), (b, h, i)
    return cnt, idx


@pytest.mark.parametrize("name", sorted(GEOS))
@pytest.mark.parametrize("window", [1, 3])
@pytest.mark.parametrize("dummy_prev", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_lists_every_class(name, window, dummy_prev, causal):
    w = GEOS[name]
    _say(f"[gpu] structured lists {name} L={window} prev={dummy_prev} causal={causal}")
    cls = _classes(w.B, w.H, window * 4 + 2 * dummy_prev + causal)
    _compare(w, cls, window, dummy_prev, causal, frame0=False, text=False)
    _compare(w, cls, window, dummy_prev, causal, frame0=True, text=True)


def test_lists_without_mask_match():
    w = GEOS["straddle"]
    _say("[gpu] structured lists without the mask output")
    cls = _classes(w.B, w.H, 7)
    g = _geo(w)
    m, c1, i1 = bsa.bsa_structured_lists(torch.from_numpy(cls).cuda(), g, 2, block_causal=True)
    none, c2, i2 = bsa.bsa_structured_lists(torch.from_numpy(cls).cuda(), g, 2, block_causal=True,
                                            want_mask=False)
    assert none is None
    assert torch.equal(c1, c2)
    for r in range(c1.numel()):
        n = int(c1.view(-1)[r])
        assert torch.equal(i1.view(-1, i1.shape[-1])[r, :n], i2.view(-1, i2.shape[-1])[r, :n])


@pytest.mark.parametrize("name", ["straddle", "ragged"])
@pytest.mark.parametrize("window", [1, 3])
def test_frame_scores_labels_and_forward(name, window):
    w = GEOS[name]
    _say(f"[gpu] frame scores + DHP + forward {name} L={window}")
    q, k, v = inputs_of(w)
    g = _geo(w)
    og = geometry_of(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    kp = bsa.bsa_pool_blocks(kd, g, g.k_block)
    P = bsa.bsa_cluster_importance(qd, kp, g, 1, 1, False)
    alpha = bsa.bsa_frame_scores(P, g, window)
    torch.cuda.synchronize()
    Ph = P.cpu().numpy()
    oal = st.frame_scores(Ph, og, window)
    ga = alpha.cpu().numpy()
    np.testing.assert_allclose(ga, oal, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(ga.sum(-1), 1.0, rtol=1e-9)    # every head has a scored row here
    n_dummy = w.H // 2
    cls = bsa.bsa_classify_heads(ga, n_dummy)
    assert np.array_equal(cls, st.classify_heads(ga, n_dummy))
    assert ((cls == st.DUMMY).sum(-1) == n_dummy).all()
    cnt, idx = _compare(w, cls, window, True, True, frame0=True, text=True)
    out, _ = bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, launch_order="frame_runs")
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    ch, ih = cnt.cpu().numpy(), idx.cpu().numpy()
    errs = []
    for b in range(og.B):
        for h in range(og.H):
            ref, _ = oracle.attention_head(q[b, h], k[b, h], v[b, h], og, ch[b, h], ih[b, h],
                                           np.zeros((og.nqb, og.nkb), np.float32))
            err = np.abs(o[b, h, :ref.shape[0]] - ref)
            assert err.max() <= 2e-2
            errs.append(err.ravel())
    assert np.concatenate(errs).mean() <= 2e-3


def test_lists_full_size():
    """The headline geometry (21 frames of 30x52 latents, 64-token blocks): one head
    of each class, every row, against the oracle."""
    base = W.workload("wan_1p3b_keep10")
    w = base.replace(H=4)
    _say("[gpu] structured lists full size, one head per class")
    cls = np.array([[st.FULL, st.SINK, st.NEIGHBOR, st.DUMMY]], dtype=np.int32)
    _compare(w, cls, 3, True, True, frame0=True, text=False)


@pytest.mark.parametrize("name", ["aligned", "straddle", "headline"])
def test_launch_orders_give_identical_outputs(name):
    """The launch order only moves work items between XCDs: outputs and LSE are
    bit-identical, for structured lists and for top-k lists (the aligned
    geometry has fewer other rows than XCDs, so some XCDs get none)."""
    w = W.workload("wan_1p3b_keep10") if name == "headline" else GEOS[name]
    _say(f"[gpu] launch orders {name}")
    q, k, v = inputs_of(w)
    g = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    cls = torch.from_numpy(_classes(w.B, w.H, 3)).cuda()
    _, c1, i1 = bsa.bsa_structured_lists(cls, g, 3, block_causal=True, frame0_dense=True, want_mask=False)
    p = bsa.MaskParams(mode="topk", topk=0, keep_ratio=0.1, frame0_dense=True, text_columns=False,
                       log_cluster=False, seed=0)
    qp = bsa.bsa_pool_blocks(qd, g, g.q_block)
    kp = bsa.bsa_pool_blocks(kd, g, g.k_block)
    _, c2, i2, _ = bsa.bsa_build_mask(qp, kp, g, p)
    for cnt, idx in ((c1, i1), (c2, i2)):
        o1, l1 = bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, want_lse=True)
        o2, l2 = bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, want_lse=True, launch_order="frame_runs")
        o3, l3 = bsa.bsa_forward_ex(qd, kd, vd, g, cnt, idx, None, want_lse=True)   # default order through _ex
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                           o3.view(torch.int16) if o3.dtype == torch.bfloat16 else o3)
        assert torch.equal(l1, l3)
        assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                           o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)
        assert torch.equal(l1, l2)


def _random_geometries(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        bq = int(rng.choice([32, 64]))
        bk = int(rng.choice([16, 32, 64]))
        out.append(tiny(text_len=int(rng.integers(0, 90)), frames=int(rng.integers(1, 8)),
                        lh=int(rng.integers(1, 12)), lw=int(rng.integers(1, 14)), bq=bq, bk=bk, D=64,
                        H=int(rng.integers(1, 6)), B=int(rng.integers(1, 3)), dtype="bf16", align=max(bq, bk)))
    return out


@pytest.mark.parametrize("k", range(12))
def test_lists_random_geometries(k):
    """Seeded random geometries (text, frames and latent sizes, block sizes),
    random classes and options: lists bit-exact against the oracle."""
    w = _random_geometries(2026, 12)[k]
    rng = np.random.default_rng(k)
    cls = rng.integers(0, 4, size=(w.B, w.H)).astype(np.int32)
    window = int(rng.integers(1, 5))
    prev, causal, f0, text = (bool(x) for x in rng.integers(0, 2, 4))
    _say(f"[gpu] structured random #{k}: text={w.text_len} frames={w.frames} {w.latent_h}x{w.latent_w} "
         f"bq={w.q_block} bk={w.k_block} B={w.B} H={w.H} L={window}")
    _compare(w, cls, window, prev, causal, f0, text)
