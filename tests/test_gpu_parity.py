"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: pooled means, block masks, counts and per-row lists (and the
sampling log-weights to 2 ulp, since ln is the GPU's own).  Attention output
within max-abs 2e-2 / mean-abs 2e-3 (bf16 in, float32 accumulate).  Small
workloads are compared on every row; the full-size workloads (launched
exactly as bench.py launches them) on sampled rows the oracle computes one by
one.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import geometry_of, inputs_of, params_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")

MAX_ABS, MEAN_ABS = 2e-2, 2e-3          # bf16 inputs: bf16 products, float32 accumulation


# bf16 LSE, absolute part: the row sum adds the same bf16-rounded P that the
# P.V product uses (so O / l stays consistent).  Each p is within half a bf16
# ulp, 2^-8 relative, so the sum of these positive terms is too, and its log
# within ln(1 + 2^-8) = 3.9e-3 nats of the exact one.  A row dominated by one
# p that is not exactly 1 (its max past the softmax reference) reaches that.
BF16_LSE_ATOL = 4e-3


def tolerances(w):
    """(max-abs, mean-abs, LSE atol) against the float64 oracle: the bf16
    bounds above for bf16 inputs; float32 inputs run float32 products and
    softmax, whose rounding (logits of magnitude <= 30 at 2^-24 relative,
    one-ulp exponentials) stays far below 1e-5.  The LSE also has a relative
    part (see _check_out)."""
    return (MAX_ABS, MEAN_ABS, BF16_LSE_ATOL) if w.dtype == "bf16" else (1e-5, 1e-6, 1e-5)


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


def run_gpu(w, q, k, v, want_lse=True):
    """The whole path on the GPU, through the C ABI."""
    _say(f"[gpu] {w.name} B={w.B} H={w.H} S={w.S} D={w.D} bq={w.q_block} bk={w.k_block} mode={w.mode}")
    g = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    qp, kp = bsa.bsa_pool_qk(qd, kd, g)          # one launch, as bench.py pools
    # the one-tensor entry point computes the same means, bit for bit
    assert torch.equal(bsa.bsa_pool_blocks(qd, g, g.q_block).view(torch.int32), qp.view(torch.int32))
    assert torch.equal(bsa.bsa_pool_blocks(kd, g, g.k_block).view(torch.int32), kp.view(torch.int32))
    mask, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, g, _mp(w))
    # NaN-filled outputs: every row (valid or pad) must be written by the kernel
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.H, w.seq_alloc), float("nan"), device=qd.device) if want_lse else None
    out, lse = bsa.bsa_forward(qd, kd, vd, g, cnt, idx, logw, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "forward left output rows unwritten"
    if lse is not None:
        assert not torch.isnan(lse).any().item(), "forward left LSE rows unwritten"
    r = dict(qp=qp.cpu().numpy(), kp=kp.cpu().numpy(), mask=mask.cpu().numpy().astype(bool),
             cnt=cnt.cpu().numpy(), idx=idx.cpu().numpy(),
             logw=None if logw is None else logw.cpu().numpy(),
             out=out.float().cpu().numpy(), lse=None if lse is None else lse.cpu().numpy())
    return r


def _check_lists(w, r, om, ocnt, oidx, ologw, rows):
    for (b, h, i) in rows:
        assert np.array_equal(r["mask"][b, h, i], om[b, h, i]), (w.name, b, h, i)
        c = ocnt[b, h, i]
        assert r["cnt"][b, h, i] == c, (w.name, b, h, i)
        assert np.array_equal(r["idx"][b, h, i, :c], oidx[b, h, i, :c]), (w.name, b, h, i)
        if w.mode == "sample":
            gw = r["logw"][b, h, i, :c].astype(np.float64)
            ow = ologw[b, h, i, :c].astype(np.float64)
            assert np.all(np.abs(gw - ow) <= 2.5e-7 * np.maximum(1.0, np.abs(ow))), (w.name, b, h, i)


def _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, qblocks_by_head):
    max_abs, mean_abs, lse_tol = tolerances(w)
    errs = []
    for (b, h), qbl in qblocks_by_head.items():
        o, l = oracle.attention_head(q[b, h], k[b, h], v[b, h], g, ocnt[b, h], oidx[b, h], ologw[b, h],
                                     q_blocks=qbl)
        rows = np.concatenate([np.arange(i * g.q_block, min((i + 1) * g.q_block, g.seq_alloc)) for i in qbl])
        got = r["out"][b, h, rows].astype(np.float64)
        assert np.isfinite(got).all()
        err = np.abs(got - o)
        errs.append(err)
        assert err.max() <= max_abs, (w.name, b, h, err.max())
        valid = rows < g.S
        gl = r["lse"][b, h, rows]
        assert np.all(np.isneginf(gl[~valid]))
        fin = np.isfinite(l[valid])
        assert np.array_equal(np.isfinite(gl[valid]), fin), (w.name, b, h)     # empty rows: -inf on both sides
        # the LSE carries the error of the logits themselves: bf16 products are
        # exact, but the bf16 matrix instructions' fp32 sums of them are not
        # sequential IEEE sums (measured: an LSE of 7.67 off by 2.9e-3 on a row
        # whose bf16-rounded P explain 6e-5 of it, and where the fp32 kernel on
        # the same inputs is within 5e-7), so the bound grows with |LSE|
        lse_rtol = 5e-4 if w.dtype == "bf16" else 1e-6
        assert np.all(np.abs(gl[valid][fin] - l[valid][fin]) <= lse_tol + lse_rtol * np.abs(l[valid][fin])), \
            (w.name, b, h)
        assert np.all(got[~valid] == 0)
    allerr = np.concatenate([e.ravel() for e in errs])
    _say(f"    out max|err| {allerr.max():.3e} mean|err| {allerr.mean():.3e} over {allerr.size} values")
    assert allerr.mean() <= mean_abs


SMALL = {
    "tiny_f32": W.workload("tiny_f32"),
    "small_bf16": W.workload("small_bf16"),
    "ragged_bf16_k16_sample": tiny(text_len=37, frames=5, lh=9, lw=13, bq=64, bk=16, D=128, H=3,
                                  dtype="bf16", mode="sample", topk=0, keep_ratio=0.15, sample_seed=7,
                                  centroids=8, grid=(2, 4), align=64),
    "ragged_bf16_k32_text_lc": tiny(text_len=70, frames=4, lh=11, lw=15, bq=64, bk=32, D=128, H=2,
                                   dtype="bf16", mode="topk", topk=0, keep_ratio=0.2, text_columns=True,
                                   log_cluster=True, centroids=8, grid=(2, 4), align=64),
    "ragged_f32_d64_q32_k16": tiny(text_len=19, frames=3, lh=7, lw=9, bq=32, bk=16, D=64, H=2,
                                  dtype="f32", mode="topk", topk=5, text_columns=True, centroids=4,
                                  grid=(2, 2), align=32),
    "ragged_bf16_q32_k64": tiny(text_len=45, frames=5, lh=12, lw=16, bq=32, bk=64, D=128, H=2,
                               dtype="bf16", mode="topk", topk=0, keep_ratio=0.4, centroids=8,
                               grid=(2, 4), align=64),
    "ragged_bf16_q32_k16_text": tiny(text_len=50, frames=4, lh=10, lw=14, bq=32, bk=16, D=128, H=2,
                                    dtype="bf16", mode="topk", topk=0, keep_ratio=0.25, text_columns=True,
                                    centroids=8, grid=(2, 4), align=32),
    "ragged_bf16_d64_q32_k32_sample": tiny(text_len=0, frames=6, lh=10, lw=12, bq=32, bk=32, D=64, H=2,
                                          dtype="bf16", mode="sample", topk=0, keep_ratio=0.3,
                                          sample_seed=11, centroids=8, grid=(2, 4), align=32),
    "ragged_bf16_d64_sample_k64": tiny(text_len=0, frames=6, lh=10, lw=13, bq=64, bk=64, D=64, H=2,
                                      dtype="bf16", mode="sample", topk=0, keep_ratio=0.3, sample_seed=99,
                                      frame0_dense=False, centroids=8, grid=(2, 4), align=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_every_row(name):
    w = SMALL[name]
    g = geometry_of(w)
    q, k, v = inputs_of(w, pad_value=np.nan)
    r = run_gpu(w, q, k, v)
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    assert np.array_equal(r["qp"], oqp) and np.array_equal(r["kp"], okp)
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w))
    rows = [(b, h, i) for b in range(g.B) for h in range(g.H) for i in range(g.nqb)]
    _check_lists(w, r, om, ocnt, oidx, ologw, rows)
    heads = [(b, h) for b in range(g.B) for h in range(g.H)]
    if g.S > 4096:   # every row of two heads, sampled rows of the others
        rng = np.random.default_rng(0)
        qbl = {bh: (list(range(g.nqb)) if n < 2 else sorted(set(rng.integers(0, g.nqb, 6).tolist()) | {0, g.nqb - 1}))
               for n, bh in enumerate(heads)}
    else:
        qbl = {bh: list(range(g.nqb)) for bh in heads}
    _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, qbl)


FULL = ["wan_1p3b_keep10", "wan_1p3b_sampled_k16", "hunyuan_keep08"]


# whole heads whose every row's mask, count, list (and log-weights) are
# compared at full size: all heads of the headline workload, four elsewhere
WHOLE_HEADS = {"wan_1p3b_keep10": None, "wan_1p3b_sampled_k16": 4, "hunyuan_keep08": 4}


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    """Full size: masks and lists of every row of whole heads (top-k mask first,
    frame-0 rows overwritten after), outputs on sampled rows."""
    w = W.workload(name)
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    r = run_gpu(w, q, k, v)
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    assert np.array_equal(r["qp"], oqp) and np.array_equal(r["kp"], okp)
    rng = np.random.default_rng(1)
    f0 = list(g.frame0_q_blocks())
    nh = WHOLE_HEADS[name]
    heads = list(range(g.H)) if nh is None else sorted(set([0, g.H - 1] + rng.choice(np.arange(1, g.H - 1), nh - 2,
                                                                                      replace=False).tolist()))
    every = [(0, h, i) for h in heads for i in range(g.nqb)]
    _say(f"    lists of every row of heads {heads} ({len(every)} rows)")
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w), rows=every)
    _check_lists(w, r, om, ocnt, oidx, ologw, every)
    # output rows: the first, last and a few random heads, a sample of their rows
    rows = []
    for h in sorted(set([0, g.H - 1] + rng.integers(0, g.H, 2).tolist())):
        picks = {f0[0], f0[-1], f0[-1] + 1, g.nqb - 1, g.nqb // 2} | set(rng.integers(0, g.nqb, 6).tolist())
        rows += [(0, h, i) for i in sorted(picks)]
    if any(h not in heads for (_, h, _) in rows):
        om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w), rows=rows + every)
        _check_lists(w, r, om, ocnt, oidx, ologw, rows)
    # every row non-empty, every list ascending (a property that holds at any size)
    assert (r["cnt"] >= 1).all()
    if w.mode == "topk":
        k_ = oracle.topk_count(g.nkb, w.topk, w.keep_ratio)
        sparse = np.ones(g.nqb, bool)
        sparse[f0] = False
        extra = len(g.text_k_blocks()) if w.text_columns else 0
        assert np.all(r["cnt"][:, :, sparse] >= k_) and np.all(r["cnt"][:, :, sparse] <= k_ + extra)
        assert np.all(r["cnt"][:, :, f0] == g.nkb)
    qbl = {}
    for (b, h, i) in rows[::2]:
        qbl.setdefault((b, h), []).append(i)
    _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, qbl)


def test_long_rows_top_k_radix_select():
    """Rows of more than 2048 key blocks take the LDS radix-select path of the mask kernel."""
    w = tiny(text_len=10, frames=2, lh=128, lw=130, bq=64, bk=16, D=64, H=1, dtype="bf16", mode="topk",
             topk=0, keep_ratio=0.02, text_columns=True, frame0_dense=False, centroids=16, grid=(4, 4),
             align=64)
    g = geometry_of(w)
    assert g.nkb > 2048
    q, k, v = inputs_of(w)
    r = run_gpu(w, q, k, v)
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    assert np.array_equal(r["qp"], oqp) and np.array_equal(r["kp"], okp)
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w))
    rows = [(0, 0, i) for i in range(g.nqb)]
    _check_lists(w, r, om, ocnt, oidx, ologw, rows)
    _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, {(0, 0): [0, 1, g.nqb // 2, g.nqb - 1]})


def test_forward_arbitrary_lists_weights_and_nan_pads():
    w = tiny(text_len=21, frames=4, lh=9, lw=11, bq=64, bk=16, D=128, H=3, dtype="bf16", align=64,
             centroids=4, grid=(2, 2))
    g = geometry_of(w)
    q, k, v = inputs_of(w, pad_value=np.nan)
    rng = np.random.default_rng(5)
    cnt = np.zeros((g.B, g.H, g.nqb), np.int32)
    idx = np.full((g.B, g.H, g.nqb, g.nkb), -1, np.int32)
    lw = np.zeros((g.B, g.H, g.nqb, g.nkb), np.float32)
    for h in range(g.H):
        for i in range(g.nqb):
            c = int(rng.integers(0, g.nkb + 1)) if (h, i) != (1, 2) else 0    # one empty row
            js = np.sort(rng.choice(g.nkb, c, replace=False))
            cnt[0, h, i] = c
            idx[0, h, i, :c] = js
            lw[0, h, i, :c] = rng.normal(0, 1.5, c).astype(np.float32)
    gg = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    out, lse = bsa.bsa_forward(qd, kd, vd, gg, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(lw).cuda(), want_lse=True)
    torch.cuda.synchronize()
    r = dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
    _check_out(w, r, q, k, v, g, cnt, idx, lw, {(0, h): list(range(g.nqb)) for h in range(g.H)})
    assert np.all(r["out"][0, 1, 2 * 64:3 * 64] == 0) and np.all(np.isneginf(r["lse"][0, 1, 2 * 64:3 * 64]))
    # an explicit softmax scale
    out2, _ = bsa.bsa_forward(qd, kd, vd, gg, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda(),
                              torch.from_numpy(lw).cuda(), softmax_scale=0.05)
    torch.cuda.synchronize()
    o, _ = oracle.attention_head(q[0, 0], k[0, 0], v[0, 0], g, cnt[0, 0], idx[0, 0], lw[0, 0], softmax_scale=0.05)
    assert np.abs(out2.float().cpu().numpy()[0, 0, :o.shape[0]] - o).max() <= tolerances(w)[0]


@pytest.mark.parametrize("bk", [16, 32, 64])
def test_forward_row_max_far_above_the_first_step(bk):
    """The 64-row forward keeps the first step's row max as the softmax
    reference; a row whose later blocks score far higher (here log-weights of
    +60 after a first step at 0: 2^86 times larger) runs again with the row max
    of every step.  Both kinds of rows, and rows whose later blocks score far
    lower (-60), agree with the oracle."""
    w = tiny(text_len=7, frames=3, lh=8, lw=12, bq=64, bk=bk, D=128, H=2, dtype="bf16", align=64,
             centroids=4, grid=(2, 2))
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    rng = np.random.default_rng(11)
    ne = 64 // bk                                   # list entries of the first 64-key step
    cnt = np.zeros((g.B, g.H, g.nqb), np.int32)
    idx = np.full((g.B, g.H, g.nqb, g.nkb), -1, np.int32)
    lw = np.zeros((g.B, g.H, g.nqb, g.nkb), np.float32)
    for h in range(g.H):
        for i in range(g.nqb):
            c = int(rng.integers(ne + 1, g.nkb + 1))
            js = np.sort(rng.choice(g.nkb, c, replace=False))
            cnt[0, h, i] = c
            idx[0, h, i, :c] = js
            kind = (h * g.nqb + i) % 3
            if kind == 0:
                lw[0, h, i, ne + int(rng.integers(0, c - ne))] = 60.0     # past the bound: the row runs again
            elif kind == 1:
                lw[0, h, i, ne:c] = -60.0                                  # later blocks vanish
    gg = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    out, lse = bsa.bsa_forward(qd, kd, vd, gg, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(lw).cuda(), want_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item() and not torch.isinf(out).any().item()
    r = dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
    _check_out(w, r, q, k, v, g, cnt, idx, lw, {(0, h): list(range(g.nqb)) for h in range(g.H)})


# seq_alloc past the last query block: rows no query block covers must still
# be written as 0 (LSE -inf), with and without the key split, by each kernel
TAIL = {
    "wide_bf16": tiny(text_len=9, frames=2, lh=5, lw=13, bq=64, bk=16, D=128, H=2, dtype="bf16", mode="topk",
                      keep_ratio=0.3, centroids=8, grid=(2, 4), align=256),
    "general_bf16_d64": tiny(text_len=3, frames=3, lh=5, lw=7, bq=32, bk=64, D=64, H=2, dtype="bf16",
                             mode="sample", keep_ratio=0.4, sample_seed=3, centroids=8, grid=(2, 4), align=192),
    # one frame: every query block (the last included) is a frame-0 block, split into parts
    "f32_one_frame": tiny(text_len=5, frames=1, lh=6, lw=7, bq=32, bk=32, D=64, H=2, dtype="f32", mode="topk", topk=1,
                          centroids=4, grid=(2, 2), align=160),
}


@pytest.mark.parametrize("name", list(TAIL))
def test_rows_past_the_last_block(name):
    w = TAIL[name]
    g = geometry_of(w)
    assert g.seq_alloc > g.nqb * g.q_block, "the case must leave rows past the last query block"
    q, k, v = inputs_of(w, pad_value=np.nan)
    r = run_gpu(w, q, k, v)                      # NaN-filled outputs: every row must be written
    tail = slice(g.nqb * g.q_block, g.seq_alloc)
    assert np.all(r["out"][:, :, tail] == 0) and np.all(np.isneginf(r["lse"][:, :, tail]))
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w))
    _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, {(b, h): list(range(g.nqb)) for b in range(g.B) for h in range(g.H)})
    # the key split of the frame-0 rows (here the frame-0 blocks include the last block or not)
    gg = _geo(w)
    qd, kd, vd = _dev(w, q), _dev(w, k), _dev(w, v)
    qp, kp = bsa.bsa_pool_qk(qd, kd, gg)
    _, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, gg, _mp(w))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.H, w.seq_alloc), float("nan"), device=qd.device)
    out, lse = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, out=out, lse=lse, dense_split=3)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert not np.isnan(o).any() and not torch.isnan(lse).any().item()
    assert np.all(o[:, :, tail] == 0) and np.all(np.isneginf(lse.cpu().numpy()[:, :, tail]))


def test_deterministic_reruns():
    w = SMALL["ragged_bf16_k16_sample"]
    q, k, v = inputs_of(w)
    a = run_gpu(w, q, k, v)
    b = run_gpu(w, q, k, v)
    for key in ("qp", "kp", "mask", "cnt", "out", "lse", "logw"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_max_key_blocks():
    """nkb = 8192, the limit of the top-k mask and the forward: the mask's LDS
    radix select, frame-0 rows listing all 8192 blocks, 16-token key blocks.
    Sampled rows (dense and sparse, first and last) against the oracle."""
    w = tiny(text_len=0, frames=8, lh=128, lw=128, bq=64, bk=16, D=64, H=1, dtype="bf16", mode="topk",
             topk=0, keep_ratio=0.01, frame0_dense=True, centroids=16, grid=(4, 4), align=64)
    g = geometry_of(w)
    assert g.nkb == 8192
    q, k, v = inputs_of(w)
    r = run_gpu(w, q, k, v)
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k, g.S, g.k_block)
    assert np.array_equal(r["qp"], oqp) and np.array_equal(r["kp"], okp)
    f0 = list(g.frame0_q_blocks())
    picks = [0, f0[-1], f0[-1] + 1, g.nqb // 2, g.nqb - 1]
    rows = [(0, 0, i) for i in picks]
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w), rows=rows)
    _check_lists(w, r, om, ocnt, oidx, ologw, rows)
    assert np.all(r["cnt"][0, 0, f0] == g.nkb)
    _check_out(w, r, q, k, v, g, ocnt, oidx, ologw, {(0, 0): picks})


@pytest.mark.parametrize("k", range(10))
def test_random_geometries_every_row(k):
    """Seeded random geometries, modes and options through the whole path:
    pooled means, masks and lists bit-exact, outputs within tolerance, every row."""
    rng = np.random.default_rng(500 + k)
    bq = int(rng.choice([32, 64]))
    bk = int(rng.choice([16, 32, 64]))
    D = int(rng.choice([64, 128]))
    mode = str(rng.choice(["topk", "sample"]))
    w = tiny(text_len=int(rng.integers(0, 80)), frames=int(rng.integers(1, 6)), lh=int(rng.integers(2, 12)),
             lw=int(rng.integers(2, 14)), bq=bq, bk=bk, D=D, H=int(rng.integers(1, 4)), B=int(rng.integers(1, 3)),
             dtype=str(rng.choice(["bf16", "f32"])), mode=mode, topk=int(rng.integers(0, 4)),
             keep_ratio=float(rng.uniform(0.05, 0.6)), frame0_dense=bool(rng.integers(0, 2)),
             text_columns=bool(rng.integers(0, 2)), log_cluster=bool(rng.integers(0, 2)),
             sample_seed=int(rng.integers(0, 1000)), centroids=8, grid=(2, 4), align=max(bq, bk))
    g = geometry_of(w)
    q, k_, v = inputs_of(w, pad_value=np.nan)
    r = run_gpu(w, q, k_, v)
    oqp = oracle.pool_blocks(q, g.S, g.q_block)
    okp = oracle.pool_blocks(k_, g.S, g.k_block)
    assert np.array_equal(r["qp"], oqp) and np.array_equal(r["kp"], okp)
    om, ocnt, oidx, ologw = oracle.build_mask(oqp, okp, g, params_of(w))
    rows = [(b, h, i) for b in range(g.B) for h in range(g.H) for i in range(g.nqb)]
    _check_lists(w, r, om, ocnt, oidx, ologw, rows)
    _check_out(w, r, q, k_, v, g, ocnt, oidx, ologw,
               {(b, h): list(range(g.nqb)) for b in range(g.B) for h in range(g.H)})
