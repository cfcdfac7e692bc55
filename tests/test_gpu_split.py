"""Key split of the frame-0 rows (bsa_forward_split) against the oracle.

Each frame-0 row's list is split over several work items whose partial
softmax states a second kernel merges.  The merged rows must match the
oracle's attention (and LSE) within the usual tolerance; every other row
runs exactly as in bsa_forward and must equal its output bit for bit.  Cases
cover ragged sequences, 16/32/64-key blocks, 32/64-row query blocks, sampled
lists with log-weights, text columns, both launch orders, and splits with
more parts than a row has blocks (empty parts).
"""
import numpy as np
import pytest

import oracle
import test_gpu_parity as P
from helpers import geometry_of, inputs_of, params_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = {
    "k64_topk": (tiny(text_len=20, frames=5, lh=9, lw=14, bq=64, bk=64, D=128, H=2, dtype="bf16", mode="topk",
                      topk=0, keep_ratio=0.3, centroids=8, grid=(2, 4), align=64), (2, 3), "frame_position"),
    "k16_sample": (tiny(text_len=37, frames=5, lh=9, lw=13, bq=64, bk=16, D=128, H=2, dtype="bf16", mode="sample",
                        topk=0, keep_ratio=0.15, sample_seed=7, centroids=8, grid=(2, 4), align=64),
                   (2, 5), "frame_position"),
    "q32_k32_text_runs": (tiny(text_len=70, frames=4, lh=11, lw=15, bq=32, bk=32, D=128, H=2, dtype="bf16",
                               mode="topk", topk=0, keep_ratio=0.2, text_columns=True, centroids=8, grid=(2, 4),
                               align=32), (3,), "frame_runs"),
    "d64_f32": (tiny(text_len=19, frames=3, lh=7, lw=9, bq=32, bk=16, D=64, H=2, dtype="f32", mode="topk", topk=5,
                     text_columns=True, centroids=4, grid=(2, 2), align=32), (2,), "frame_position"),
    # frame-0 rows keep only their top 2 blocks: a 4-way split leaves parts empty
    "empty_parts": (tiny(text_len=0, frames=4, lh=8, lw=16, bq=64, bk=64, D=128, H=2, dtype="bf16", mode="topk",
                         topk=2, frame0_dense=False, centroids=8, grid=(2, 4), align=64), (4, 16), "frame_position"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_split_rows_match_the_oracle(name):
    w, splits, order = CASES[name]
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    if w.dtype == "bf16":    # the oracle sees the bf16 values the GPU gets
        q, k, v = (torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in (q, k, v))
    gg = P._geo(w)
    qd, kd, vd = P._dev(w, q), P._dev(w, k), P._dev(w, v)
    qp = bsa.bsa_pool_blocks(qd, gg, gg.q_block)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    _, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, gg, P._mp(w))
    base, base_lse = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, want_lse=True, launch_order=order)
    torch.cuda.synchronize()
    om, ocnt, oidx, ologw = oracle.build_mask(oracle.pool_blocks(q, g.S, g.q_block),
                                              oracle.pool_blocks(k, g.S, g.k_block), g, params_of(w))
    assert np.array_equal(cnt.cpu().numpy(), ocnt)
    d = bsa.bsa_derive(gg)
    f0 = np.zeros(g.nqb, dtype=bool)
    f0[d["frame0_first"]:d["frame0_last"] + 1] = True
    f0_rows = np.repeat(f0, g.q_block)[:g.seq_alloc]
    for split in splits:
        P._say(f"[gpu] split {name} x{split} order={order} B={w.B} H={w.H} S={w.S} bq={w.q_block} bk={w.k_block}")
        nbytes = bsa.bsa_forward_split_workspace_bytes(gg, split)
        nd = d["frame0_last"] - d["frame0_first"] + 1
        assert nbytes == w.B * w.H * nd * split * (w.q_block * w.D + 2 * w.q_block) * 4
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H, w.seq_alloc), float("nan"), device=qd.device)
        out, lse = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, out=out, lse=lse, launch_order=order,
                                   dense_split=split)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item(), "rows left unwritten"
        r = dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
        # every row against the oracle
        P._check_out(w, r, q, k, v, g, ocnt, oidx, ologw,
                     {(b, h): list(range(g.nqb)) for b in range(w.B) for h in range(w.H)})
        # rows outside frame 0 are the unsplit kernel's, bit for bit
        got = out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        ref = base.view(torch.int16 if base.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        assert np.array_equal(got[:, :, ~f0_rows], ref[:, :, ~f0_rows])
        assert np.array_equal(lse.cpu().numpy()[:, :, ~f0_rows].view(np.uint32),
                              base_lse.cpu().numpy()[:, :, ~f0_rows].view(np.uint32))


def test_split_of_one_is_the_plain_forward():
    w = CASES["k64_topk"][0]
    q, k, v = inputs_of(w)
    gg = P._geo(w)
    qd, kd, vd = P._dev(w, q), P._dev(w, k), P._dev(w, v)
    qp = bsa.bsa_pool_blocks(qd, gg, gg.q_block)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    _, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, gg, P._mp(w))
    P._say("[gpu] split x1 vs plain forward")
    a, la = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, want_lse=True)
    assert bsa.bsa_forward_split_workspace_bytes(gg, 1) == 0
    # through the C entry point with dense_split 1 and no workspace
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.seq_alloc), dtype=torch.float32, device=qd.device)
    L = bsa._lib.lib()
    opt = bsa._lib.bsa_forward_options(0)
    bsa._lib.check(L.bsa_forward_split(bsa._ptr(qd), bsa._ptr(kd), bsa._ptr(vd), 0, bsa.ctypes.byref(gg.c()),
                                       bsa._ptr(cnt), bsa._ptr(idx), None, 0.0, bsa._ptr(out), bsa._ptr(lse),
                                       bsa.ctypes.byref(opt), 1, None, 0, bsa._stream(None)))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), a.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), la.view(torch.int32))


@pytest.mark.parametrize("bk", [16, 64])
def test_split_parts_past_the_reference_bound(bk):
    """Each part of a split frame-0 row keeps its own first step's row max as
    the softmax reference; parts whose later blocks score far higher (+60 in
    log-weight) run again with the row max of every step, parts whose later
    blocks score far lower (-60) do not, and the merged rows match the oracle."""
    w = tiny(text_len=11, frames=4, lh=8, lw=16, bq=64, bk=bk, D=128, H=2, dtype="bf16", mode="topk",
             topk=0, keep_ratio=0.3, centroids=8, grid=(2, 4), align=64)
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    gg = P._geo(w)
    qd, kd, vd = P._dev(w, q), P._dev(w, k), P._dev(w, v)
    _, cnt, idx, _ = bsa.bsa_build_mask(bsa.bsa_pool_blocks(qd, gg, gg.q_block),
                                        bsa.bsa_pool_blocks(kd, gg, gg.k_block), gg, P._mp(w))
    c, ix = cnt.cpu().numpy(), idx.cpu().numpy()
    lw = np.zeros(ix.shape, np.float32)
    rng = np.random.default_rng(3)
    for h in range(g.H):
        for i in range(g.nqb):
            n = int(c[0, h, i])
            if n < 4:
                continue
            if (h + i) % 2 == 0:
                lw[0, h, i, int(rng.integers(n // 2, n))] = 60.0
            else:
                lw[0, h, i, n // 2:n] = -60.0
    lwd = torch.from_numpy(lw).cuda()
    for split in (1, 3):
        P._say(f"[gpu] split bound bk={bk} x{split}")
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H, w.seq_alloc), float("nan"), device=qd.device)
        out, lse = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, lwd, out=out, lse=lse, dense_split=split)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item() and not torch.isinf(out).any().item()
        r = dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
        P._check_out(w, r, q, k, v, g, c, ix, lw, {(0, h): list(range(g.nqb)) for h in range(g.H)})
