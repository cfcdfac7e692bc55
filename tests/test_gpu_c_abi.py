"""The C ABI from a plain C client on the GPU.

tests/c_abi/bsa_example (built by build()) runs pooling, the top-k mask and
the forward (plain, and with the frame-0 rows' key lists split in two)
through include/bsa.h with only the HIP runtime's C API.  Its
counts, lists, output and LSE must equal, bit for bit, what the Python
binding gets from the same library on the same inputs; the lists are also
checked against the oracle.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from helpers import geometry_of, inputs_of, params_of, tiny

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_42_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "bsa_example")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_c_client_matches_the_binding(tmp_path):
    assert os.path.exists(EXE), "tests/c_abi/bsa_example is built by __graft_entry__.build()"
    w = tiny(text_len=10, frames=3, lh=8, lw=12, bq=64, bk=32, D=64, H=2, dtype="bf16", mode="topk", topk=0,
             keep_ratio=0.3, frame0_dense=True, centroids=8, grid=(2, 4), align=64)
    g = geometry_of(w)
    q, k, v = inputs_of(w)
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16) for a in (q, k, v))
    for name, t in (("q", qd), ("k", kd), ("v", vd)):
        t.view(torch.int16).numpy().tofile(str(tmp_path / f"{name}.bin"))
    args = [EXE, str(tmp_path), str(w.B), str(w.H), str(w.text_len), str(w.frames), str(w.latent_h),
            str(w.latent_w), str(w.D), str(w.q_block), str(w.k_block), str(w.seq_alloc), repr(w.keep_ratio)]
    print("[gpu] C client", " ".join(args[2:]), flush=True)
    sys.stdout.flush()
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    cnt = np.fromfile(str(tmp_path / "cnt.bin"), dtype=np.int32).reshape(w.B, w.H, g.nqb)
    idx = np.fromfile(str(tmp_path / "idx.bin"), dtype=np.int32).reshape(w.B, w.H, g.nqb, g.nkb)
    out = np.fromfile(str(tmp_path / "out.bin"), dtype=np.int16).reshape(w.B, w.H, w.seq_alloc, w.D)
    lse = np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).reshape(w.B, w.H, w.seq_alloc)

    # the same library through the binding
    gg = bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D, w.q_block, w.k_block,
                      w.seq_alloc)
    p = bsa.MaskParams(mode="topk", topk=0, keep_ratio=w.keep_ratio, frame0_dense=True)
    qc, kc, vc = qd.cuda(), kd.cuda(), vd.cuda()
    qp = bsa.bsa_pool_blocks(qc, gg, gg.q_block)
    kp = bsa.bsa_pool_blocks(kc, gg, gg.k_block)
    _, c2, i2, _ = bsa.bsa_build_mask(qp, kp, gg, p)
    o2, l2 = bsa.bsa_forward(qc, kc, vc, gg, c2, i2, None, want_lse=True)
    torch.cuda.synchronize()
    c2, i2 = c2.cpu().numpy(), i2.cpu().numpy()
    assert np.array_equal(cnt, c2)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(g.nqb):
                n = cnt[b, h, i]
                assert np.array_equal(idx[b, h, i, :n], i2[b, h, i, :n]), (b, h, i)
    assert np.array_equal(out, o2.view(torch.int16).cpu().numpy())
    assert np.array_equal(lse, l2.cpu().numpy())
    # the key-split forward: the binding's, bit for bit
    outs = np.fromfile(str(tmp_path / "out_split.bin"), dtype=np.int16).reshape(w.B, w.H, w.seq_alloc, w.D)
    lses = np.fromfile(str(tmp_path / "lse_split.bin"), dtype=np.float32).reshape(w.B, w.H, w.seq_alloc)
    o3, l3 = bsa.bsa_forward(qc, kc, vc, gg, torch.from_numpy(c2).cuda(), torch.from_numpy(i2).cuda(), None,
                             want_lse=True, dense_split=2)
    torch.cuda.synchronize()
    assert np.array_equal(outs, o3.view(torch.int16).cpu().numpy())
    assert np.array_equal(lses.view(np.uint32), l3.cpu().numpy().view(np.uint32))
    # and the lists are the oracle's
    _, ocnt, oidx, _ = oracle.build_mask(oracle.pool_blocks(q, g.S, g.q_block),
                                         oracle.pool_blocks(k, g.S, g.k_block), g, params_of(w))
    assert np.array_equal(cnt, ocnt)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(g.nqb):
                n = ocnt[b, h, i]
                assert np.array_equal(idx[b, h, i, :n], oidx[b, h, i, :n]), (b, h, i)
