"""The allocation-free key split (bsa_forward_split_static) against bsa_forward_split.

bsa_forward_split_static runs the same kernels as bsa_forward_split with the
partial softmax states in the library's own device scratch instead of a
caller-provided workspace, so its outputs must equal those of
bsa_forward_split bit for bit.  Two calls in a row, the second on a smaller
input, check that a call never depends on what the previous one left in the
shared scratch.
"""
import ctypes

import numpy as np
import pytest

import test_gpu_parity as P
from helpers import inputs_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (workload, dense_split): the second is smaller in heads, frames and split
CALLS = [
    (tiny(text_len=20, frames=6, lh=9, lw=14, bq=64, bk=64, D=128, H=3, dtype="bf16", mode="topk", topk=0,
          keep_ratio=0.3, centroids=8, grid=(2, 4), align=64), 3),
    (tiny(text_len=11, frames=3, lh=7, lw=10, bq=64, bk=16, D=128, H=1, dtype="bf16", mode="sample", topk=0,
          keep_ratio=0.2, sample_seed=5, centroids=8, grid=(2, 4), align=64), 2),
]


def _c_split(L, qd, kd, vd, gg, cnt, idx, logw, out, lse, split, static):
    opt = bsa._lib.bsa_forward_options(0)
    head = (bsa._ptr(qd), bsa._ptr(kd), bsa._ptr(vd), 0, ctypes.byref(gg.c()), bsa._ptr(cnt), bsa._ptr(idx),
            bsa._ptr(logw), 0.0, bsa._ptr(out), bsa._ptr(lse), ctypes.byref(opt), split)
    if static:
        return L.bsa_forward_split_static(*head, bsa._stream(None)), None
    nbytes = bsa.bsa_forward_split_workspace_bytes(gg, split)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=qd.device)
    return L.bsa_forward_split(*head, bsa._ptr(ws), ws.numel() * 4, bsa._stream(None)), ws


def test_static_split_equals_the_workspace_split_twice():
    L = bsa._lib.lib()
    for n, (w, split) in enumerate(CALLS):
        P._say(f"[gpu] static split call {n}: H={w.H} S={w.S} bk={w.k_block} mode={w.mode} split={split}")
        q, k, v = inputs_of(w)
        gg = P._geo(w)
        qd, kd, vd = P._dev(w, q), P._dev(w, k), P._dev(w, v)
        qp = bsa.bsa_pool_blocks(qd, gg, gg.q_block)
        kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
        _, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, gg, P._mp(w))
        assert 0 < bsa.bsa_forward_split_workspace_bytes(gg, split) <= bsa._lib.BSA_SPLIT_STATIC_MAX_BYTES
        res = []
        for static in (False, True):
            out = torch.full_like(qd, float("nan"))
            lse = torch.full((w.B, w.H, w.seq_alloc), float("nan"), dtype=torch.float32, device=qd.device)
            st, _ws = _c_split(L, qd, kd, vd, gg, cnt, idx, logw, out, lse, split, static)
            bsa._lib.check(st)
            torch.cuda.synchronize()
            res.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy().view(np.uint32)))
        assert not np.isnan(res[1][1].view(np.float32)).any(), "rows left unwritten"
        assert np.array_equal(res[0][0], res[1][0]), "outputs differ from bsa_forward_split"
        assert np.array_equal(res[0][1], res[1][1]), "LSE differs from bsa_forward_split"


def test_static_split_of_one_is_the_plain_forward():
    w, _ = CALLS[1]
    q, k, v = inputs_of(w)
    gg = P._geo(w)
    qd, kd, vd = P._dev(w, q), P._dev(w, k), P._dev(w, v)
    qp = bsa.bsa_pool_blocks(qd, gg, gg.q_block)
    kp = bsa.bsa_pool_blocks(kd, gg, gg.k_block)
    _, cnt, idx, logw = bsa.bsa_build_mask(qp, kp, gg, P._mp(w))
    P._say("[gpu] static split x1 vs plain forward")
    a, la = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, want_lse=True)
    b, lb = bsa.bsa_forward(qd, kd, vd, gg, cnt, idx, logw, want_lse=True, static_workspace=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
