"""The whole path captured in one HIP graph.

No entry point allocates, frees, synchronizes or records a memset, so a
caller can capture pooling, a block selector and the forward on one stream
and replay them.  Each case here runs the path eagerly, captures it once,
then replays the graph three times: the outputs are overwritten with junk by
eager kernels before every replay, and new inputs are copied into the
captured input buffers before the third.  The key split of the frame-0 rows
(a forward plus a merge kernel, with its workspace) is captured the same way.  Every replay must reproduce, bit
for bit, the eager path on the same inputs (counts, the listed prefix of
every row, masks, log-weights, output and LSE).
"""
import sys

import numpy as np
import pytest

from helpers import inputs_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _workload(bk):
    return tiny(text_len=10, frames=4, lh=8, lw=12, bq=64, bk=bk, D=128, H=3, dtype="bf16", mode="topk", topk=0,
                keep_ratio=0.3, frame0_dense=True, centroids=8, grid=(2, 4), align=64)


def _geometry(w):
    return bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D, w.q_block, w.k_block,
                        w.seq_alloc)


def _device_inputs(w, seed):
    q, k, v = inputs_of(w.replace(data_seed=seed))
    return [torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda() for a in (q, k, v)]


def _path(case, g, q, k, v, head_class):
    """One pass of the path; returns (cnt, idx, logw or None, mask or None, out, lse or None)."""
    if case == "topk":
        qp = bsa.bsa_pool_blocks(q, g, g.q_block)
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        mask, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, g, bsa.MaskParams(keep_ratio=0.3, frame0_dense=True))
        out, lse = bsa.bsa_forward(q, k, v, g, cnt, idx, logw, want_lse=True)
    elif case == "split":
        qp = bsa.bsa_pool_blocks(q, g, g.q_block)
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        mask, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, g, bsa.MaskParams(keep_ratio=0.3, frame0_dense=True))
        out, lse = bsa.bsa_forward(q, k, v, g, cnt, idx, logw, want_lse=True, dense_split=3)
    elif case == "sample":
        qp = bsa.bsa_pool_blocks(q, g, g.q_block)
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        p = bsa.MaskParams(mode="sample", keep_ratio=0.3, frame0_dense=True, seed=11)
        mask, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, g, p)
        out, lse = bsa.bsa_forward(q, k, v, g, cnt, idx, logw, want_lse=True)
    elif case == "cluster":
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        imp = bsa.bsa_cluster_importance(q, kp, g, n_clusters=4, iters=3)
        mask, cnt, idx, logw = bsa.bsa_select_blocks(imp, g, bsa.MaskParams(keep_ratio=0.3, frame0_dense=True))
        out, lse = bsa.bsa_forward(q, k, v, g, cnt, idx, logw, want_lse=True)
    elif case == "top_p":
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        vp = bsa.bsa_pool_blocks(v, g, g.k_block)
        scores = bsa.bsa_cluster_importance(q, kp, g, n_clusters=1, iters=1)
        mask, cnt, idx, _ = bsa.bsa_select_top_p(scores, g, domain="eg", top_p=0.9, v_pooled=vp,
                                                 value_aware=True)
        logw = None
        out, lse = bsa.bsa_forward(q, k, v, g, cnt, idx, None, want_lse=True)
    else:  # structured
        mask, cnt, idx = bsa.bsa_structured_lists(head_class, g, window=2, block_causal=True, frame0_dense=True)
        logw = None
        out, lse = bsa.bsa_forward_ex(q, k, v, g, cnt, idx, None, want_lse=True, launch_order="frame_runs")
    return cnt, idx, logw, mask, out, lse


def _host(res):
    # bf16 has no numpy type: its bits are compared as int16
    return [None if t is None else (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
            for t in res]


def _same(got, want, where):
    cnt, idx, logw, mask, out, lse = got
    ecnt, eidx, elogw, emask, eout, else_ = want
    assert np.array_equal(cnt, ecnt), where
    rows = cnt.reshape(-1)
    gi, ei = idx.reshape(len(rows), -1), eidx.reshape(len(rows), -1)
    for r, n in enumerate(rows):
        assert np.array_equal(gi[r, :n], ei[r, :n]), (where, "idx row", r)
    if elogw is not None:
        gw, ew = logw.reshape(len(rows), -1), elogw.reshape(len(rows), -1)
        for r, n in enumerate(rows):
            assert np.array_equal(gw[r, :n].view(np.uint32), ew[r, :n].view(np.uint32)), (where, "logw row", r)
    if emask is not None:
        assert np.array_equal(mask, emask), where
    assert np.array_equal(out.view(np.int16), eout.view(np.int16)), where
    assert np.array_equal(lse.view(np.uint32), else_.view(np.uint32)), where


def _junk(res):
    for t in res:
        if t is None:
            continue
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


@pytest.mark.parametrize("case,bk", [("topk", 64), ("split", 64), ("sample", 16), ("cluster", 64), ("top_p", 64),
                                     ("structured", 64)])
def test_path_replays_from_one_graph(case, bk):
    w = _workload(bk)
    g = _geometry(w)
    print(f"[gpu] graph {case} bk={bk} H={w.H} S={w.text_len + w.frames * w.latent_h * w.latent_w}", flush=True)
    sys.stdout.flush()
    q, k, v = _device_inputs(w, 5)
    q2, k2, v2 = _device_inputs(w, 6)
    head_class = None
    if case == "structured":
        kp = bsa.bsa_pool_blocks(k, g, g.k_block)
        scores = bsa.bsa_cluster_importance(q, kp, g, n_clusters=1, iters=1)
        alpha = bsa.bsa_frame_scores(scores, g, window=2)
        cls = bsa.bsa_classify_heads(alpha, n_dummy=1)
        head_class = torch.from_numpy(cls).cuda()

    # eager results on both input sets
    want1 = _host(_path(case, g, q, k, v, head_class))
    want2 = _host(_path(case, g, q2, k2, v2, head_class))
    torch.cuda.synchronize()

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _path(case, g, q, k, v, head_class)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = _path(case, g, q, k, v, head_class)
    torch.cuda.synchronize()

    for r in range(3):
        _junk(res)
        if r == 2:
            q.copy_(q2)
            k.copy_(k2)
            v.copy_(v2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_host(res), want2 if r == 2 else want1, (case, "replay", r))
        # eager work between replays on the same inputs gives the same answer
        eager = _host(_path(case, g, q, k, v, head_class))
        torch.cuda.synchronize()
        _same(eager, want2 if r == 2 else want1, (case, "eager", r))
    del graph
