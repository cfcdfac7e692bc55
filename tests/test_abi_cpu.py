"""The C ABI without a GPU: library loads, exports what include/bsa.h declares,
derives geometry like the pages' formulas, and rejects bad arguments before
any device work."""
import ctypes
import os
import re

import pytest

import oracle
import workloads as W
from helpers import geometry_of, params_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

bsa = pytest.importorskip("block_sparse_attention_42_amd")
from block_sparse_attention_42_amd import _lib  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbsa.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:bsa_status|const char\*|int32_t)\s+(bsa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"bsa_pool_blocks", "bsa_build_mask", "bsa_forward"}
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)
    assert L.bsa_abi_version() == 1


def _geo(w):
    return bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D,
                        w.q_block, w.k_block, w.seq_alloc)


def _mp(w):
    return bsa.MaskParams(mode=w.mode, topk=w.topk, keep_ratio=w.keep_ratio,
                          frame0_dense=w.frame0_dense, text_columns=w.text_columns,
                          log_cluster=w.log_cluster, seed=w.sample_seed)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_derive_matches_oracle_geometry(name):
    w = W.workload(name)
    d = bsa.bsa_derive(_geo(w), _mp(w))
    g = geometry_of(w)
    p = params_of(w)
    assert d["S"] == g.S and d["nqb"] == g.nqb and d["nkb"] == g.nkb
    f0 = g.frame0_q_blocks()
    assert (d["frame0_first"], d["frame0_last"]) == (f0.start, f0.stop - 1)
    tk = g.text_k_blocks()
    assert d["text_last"] == (tk.stop - 1 if len(tk) else -1)
    if w.mode == "topk":
        assert d["topk"] == oracle.topk_count(g.nkb, p.topk, p.keep_ratio)
    else:
        assert d["expected"] == float(oracle.reference.F32(p.keep_ratio * g.nkb))


def _status(fn, *args):
    return fn(*args)


def test_validation_rejects_before_launch():
    L = _lib.lib()
    w = W.workload("small_bf16")
    g = _geo(w).c()
    p = _mp(w).c()
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: every call below fails validation
    mis = ctypes.c_void_p(0x1004)
    st = L.bsa_pool_blocks(None, 0, ctypes.byref(g), 64, fake, None)
    assert st == _lib.BSA_ERR_INVALID_ARGUMENT and b"NULL" in L.bsa_last_error()
    assert L.bsa_pool_blocks(mis, 0, ctypes.byref(g), 64, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_pool_blocks(fake, 7, ctypes.byref(g), 64, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_pool_blocks(fake, 0, ctypes.byref(g), 48, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_pool_qk(fake, None, 0, ctypes.byref(g), fake, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_pool_qk(fake, fake, 0, ctypes.byref(g), mis, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_pool_qk(fake, fake, 3, ctypes.byref(g), fake, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    bad = _geo(w.replace(D=96)).c()
    assert L.bsa_pool_blocks(fake, 0, ctypes.byref(bad), 64, fake, None) == _lib.BSA_ERR_UNSUPPORTED
    bad = _geo(w.replace(q_block=128, align=128)).c()
    assert L.bsa_forward(fake, fake, fake, 0, ctypes.byref(bad), fake, fake, None, 0.0, fake, None, None) \
        == _lib.BSA_ERR_UNSUPPORTED
    small = _lib.bsa_geometry(1, 12, 0, 5, 30, 52, 128, 64, 64, 0, 7800)   # seq_alloc too small
    assert L.bsa_forward(fake, fake, fake, 0, ctypes.byref(small), fake, fake, None, 0.0, fake, None,
                         None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"seq_alloc" in L.bsa_last_error()
    # the key split: its range, and its workspace when frame-0 rows exist
    opt = _lib.bsa_forward_options(0)
    fwd_split = lambda split, ws, nbytes: L.bsa_forward_split(  # noqa: E731
        fake, fake, fake, 0, ctypes.byref(g), fake, fake, None, 0.0, fake, None, ctypes.byref(opt), split, ws,
        nbytes, None)
    need = ctypes.c_int64(0)
    assert L.bsa_forward_split_workspace_bytes(ctypes.byref(g), 2, ctypes.byref(need)) == _lib.BSA_OK
    assert need.value == 12 * 25 * 2 * (64 * 128 + 2 * 64) * 4      # small_bf16: 25 frame-0 query blocks
    for split in (0, 17):
        assert fwd_split(split, fake, need.value) == _lib.BSA_ERR_INVALID_ARGUMENT
        assert L.bsa_forward_split_workspace_bytes(ctypes.byref(g), split, ctypes.byref(need)) == \
            _lib.BSA_ERR_INVALID_ARGUMENT
    L.bsa_forward_split_workspace_bytes(ctypes.byref(g), 2, ctypes.byref(need))
    assert fwd_split(2, None, need.value) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert fwd_split(2, mis, need.value) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert fwd_split(2, fake, need.value - 1) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"workspace" in L.bsa_last_error()
    # the allocation-free split: validated like the split, then held to the library's scratch size
    fwd_static = lambda split, geo=g, qp=fake: L.bsa_forward_split_static(  # noqa: E731
        qp, fake, fake, 0, ctypes.byref(geo), fake, fake, None, 0.0, fake, None, ctypes.byref(opt), split, None)
    for split in (0, 17):
        assert fwd_static(split) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert fwd_static(2, qp=None) == _lib.BSA_ERR_INVALID_ARGUMENT
    hy = _geo(W.workload("hunyuan_keep08")).c()
    L.bsa_forward_split_workspace_bytes(ctypes.byref(hy), 16, ctypes.byref(need))
    assert need.value > _lib.BSA_SPLIT_STATIC_MAX_BYTES
    assert fwd_static(16, geo=hy) == _lib.BSA_ERR_UNSUPPORTED
    assert b"scratch" in L.bsa_last_error()
    # 4096 heads x 2^20 query blocks: more block rows than one launch counts
    huge = _lib.bsa_geometry(1, 4096, 1 << 26, 0, 0, 0, 128, 64, 64, 0, 1 << 26)
    assert L.bsa_pool_blocks(fake, 0, ctypes.byref(huge), 64, fake, None) == _lib.BSA_ERR_UNSUPPORTED
    assert b"block rows" in L.bsa_last_error()
    assert L.bsa_build_mask(fake, fake, ctypes.byref(huge), ctypes.byref(p), fake, fake, fake, None,
                            None) == _lib.BSA_ERR_UNSUPPORTED
    empty = _lib.bsa_geometry(1, 1, 0, 0, 4, 4, 64, 32, 32, 0, 64)
    assert L.bsa_derive(ctypes.byref(empty), None, ctypes.byref(_lib.bsa_derived())) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    # mask params
    for kw in ({"keep_ratio": 0.0}, {"keep_ratio": 1.5}, {"keep_ratio": float("nan")}):
        pp = _mp(w.replace(**kw)).c()
        assert L.bsa_build_mask(fake, fake, ctypes.byref(g), ctypes.byref(pp), fake, fake, fake, fake,
                                None) == _lib.BSA_ERR_INVALID_ARGUMENT
    ps = _mp(w.replace(mode="sample")).c()
    assert L.bsa_build_mask(fake, fake, ctypes.byref(g), ctypes.byref(ps), fake, fake, fake, None,
                            None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"log_w" in L.bsa_last_error()
    big = _geo(W.workload("hunyuan_keep08").replace(k_block=16)).c()
    ps = _mp(W.workload("hunyuan_keep08").replace(mode="sample", k_block=16)).c()
    assert L.bsa_build_mask(fake, fake, ctypes.byref(big), ctypes.byref(ps), fake, fake, fake, fake,
                            None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_forward(fake, fake, fake, 0, ctypes.byref(g), fake, fake, None,
                         ctypes.c_float(float("inf")), fake, None, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_status_string(2) == b"unsupported"
    # clustering selector
    for C, T in ((0, 3), (9, 3), (4, -1), (4, 17)):
        assert L.bsa_cluster_importance(fake, 0, fake, ctypes.byref(g), C, T, 0, fake, None) == \
            _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_cluster_importance(None, 0, fake, ctypes.byref(g), 4, 3, 0, fake, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_cluster_importance(fake, 0, fake, ctypes.byref(g), 4, 3, 0, mis, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    hy = _geo(W.workload("hunyuan_keep08").replace(k_block=16)).c()   # nkb 7441: 3 * 7441 > 16384
    assert L.bsa_cluster_importance(fake, 0, fake, ctypes.byref(hy), 3, 3, 0, fake, None) == \
        _lib.BSA_ERR_UNSUPPORTED
    ps = _mp(w.replace(mode="sample")).c()
    assert L.bsa_select_blocks(fake, ctypes.byref(g), ctypes.byref(ps), fake, fake, fake, None, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_select_blocks(None, ctypes.byref(g), ctypes.byref(p), fake, fake, fake, None, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    # top-p over competition domains
    nb = ctypes.c_int64()
    assert L.bsa_top_p_workspace_bytes(ctypes.byref(g), ctypes.byref(nb)) == _lib.BSA_OK and nb.value > 0

    def tp(**kw):
        base = dict(domain=4, value_aware=0, top_p=0.9, entropy_eps=1e-12, frame0_dense=0, text_columns=0,
                    reserved=0)
        base.update(kw)
        return _lib.bsa_topp_params(**base)

    def sel(t, vp=None, ws_bytes=None, geo=g):
        return L.bsa_select_top_p(fake, vp, ctypes.byref(geo), ctypes.byref(t), None, fake,
                                  nb.value if ws_bytes is None else ws_bytes, fake, fake, fake, None)
    for bad in (tp(domain=5), tp(domain=-1), tp(top_p=0.0), tp(top_p=1.5), tp(entropy_eps=0.0),
                tp(value_aware=1)):
        assert sel(bad) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert sel(tp(), ws_bytes=nb.value - 8) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"workspace" in L.bsa_last_error()
    big = _geo(W.workload("wan_1p3b_sampled_k16")).c()                  # nkb 2048: allowed
    assert L.bsa_top_p_workspace_bytes(ctypes.byref(big), ctypes.byref(nb)) == _lib.BSA_OK
    bigger = _geo(W.workload("hunyuan_keep08").replace(k_block=32)).c()   # nkb 3721 > 2048
    L.bsa_top_p_workspace_bytes(ctypes.byref(bigger), ctypes.byref(nb))
    assert sel(tp(), geo=bigger) == _lib.BSA_ERR_UNSUPPORTED
    # forward options
    bad_order = _lib.bsa_forward_options(7)
    assert L.bsa_forward_ex(fake, fake, fake, 0, ctypes.byref(g), fake, fake, None, 0.0, fake, None,
                            ctypes.byref(bad_order), None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"launch order" in L.bsa_last_error()
    # structured producers
    assert L.bsa_frame_scores(fake, ctypes.byref(g), 0, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_frame_scores(None, ctypes.byref(g), 2, fake, None) == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_frame_scores(fake, ctypes.byref(g), 2, mis, None) == _lib.BSA_ERR_INVALID_ARGUMENT

    def sp(**kw):
        base = dict(window=3, dummy_prev=0, block_causal=1, frame0_dense=0, text_columns=0, reserved=0)
        base.update(kw)
        return _lib.bsa_struct_params(**base)
    assert L.bsa_structured_lists(fake, ctypes.byref(g), ctypes.byref(sp(window=0)), None, fake, fake, None) \
        == _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_structured_lists(fake, ctypes.byref(g), None, None, fake, fake, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_structured_lists(None, ctypes.byref(g), ctypes.byref(sp()), None, fake, fake, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    assert L.bsa_structured_lists(fake, ctypes.byref(g), ctypes.byref(sp()), mis, fake, fake, None) == \
        _lib.BSA_ERR_INVALID_ARGUMENT


def test_python_binding_raises_on_missing_gpu_tensors():
    import torch
    w = W.workload("tiny_f32")
    x = torch.zeros((1, 2, 224, 64))
    with pytest.raises(ValueError):
        bsa.bsa_pool_blocks(x, _geo(w), 32)     # CPU tensor: refused, never computed on the CPU


def test_head_labelling_on_the_host_matches_the_oracle():
    """bsa_classify_heads is host-only: the page's worked example and random scores
    against the oracle's DHP."""
    import json
    import numpy as np
    import oracle.structured as st
    gd = json.load(open(os.path.join(ROOT, "tests", "golden", "dhp_example.json")))
    lh = gd["max_sink_neighbor"]
    alpha = np.zeros((1, len(lh), 3))
    for h, l in enumerate(lh):
        alpha[0, h] = [l, l / 2, 1 - l] if h % 2 else [l / 3, l, 1 - l]
    cls = bsa.bsa_classify_heads(alpha, gd["n_dummy"])
    assert sorted(np.nonzero(cls[0] == 3)[0].tolist()) == gd["dummy_heads"]
    rng = np.random.default_rng(0)
    for trial in range(50):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 20))
        a = rng.dirichlet([1, 1, 1], size=(B, H))
        a[..., :2] = np.round(a[..., :2] * 8) / 8                  # ties
        n = int(rng.integers(0, H + 1))
        assert np.array_equal(bsa.bsa_classify_heads(a, n), st.classify_heads(a, n))
    L = _lib.lib()
    bad = np.zeros((1, 2, 3))
    assert L.bsa_classify_heads(bad.ctypes.data, 1, 2, 3, np.zeros(2, np.int32).ctypes.data) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    bad[0, 1, 0] = np.nan
    assert L.bsa_classify_heads(bad.ctypes.data, 1, 2, 1, np.zeros(2, np.int32).ctypes.data) == \
        _lib.BSA_ERR_INVALID_ARGUMENT
    assert b"finite" in L.bsa_last_error()


def test_header_is_c99_and_a_c_client_links(tmp_path):
    """include/bsa.h compiles as C99 with warnings as errors, and a plain C
    client (tests/c_abi/bsa_example.c) links against libbsa.so; run without
    arguments it prints its usage and touches no device."""
    import subprocess
    import __graft_entry__ as ge
    out = str(tmp_path / "bsa_example")
    r = subprocess.run(ge.c_example_cmd(ge.C_EXAMPLE_SRC, out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([out], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_dense_split_suggestion():
    """The key split suggested for the frame-0 rows: their length over the
    launch's average blocks per SIMD, rounded, within 1..8, >= 16 blocks a part
    (host logic only: the SIMD count is given, the counts are a CPU tensor)."""
    import torch

    def counts(w, dense_len, other_len):
        g = _geo(w)
        d = bsa.bsa_derive(g)
        c = torch.full((w.B, w.H, d["nqb"]), other_len, dtype=torch.int32)
        c[:, :, d["frame0_first"]:d["frame0_last"] + 1] = dense_len
        return g, c

    small = W.workload("small_bf16")                  # 12 heads x 122 query blocks, 25 of them frame 0
    g, c = counts(small, 122, 31)
    assert bsa.suggest_dense_split(g, c, simds=1024) == 2        # 122 blocks against 71 per SIMD
    head = W.workload("wan_1p3b_keep10")              # 512-block frame-0 rows, 447 per SIMD
    g, c = counts(head, 512, 52)
    assert bsa.suggest_dense_split(g, c, simds=1024) == 1
    g, c = counts(head, 512, 4)                       # 512 against 173 per SIMD
    assert bsa.suggest_dense_split(g, c, simds=1024) == 3
    g, c = counts(head.replace(H=1), 512, 0)          # one head: 512 against 12.5, capped at 8
    assert bsa.suggest_dense_split(g, c, simds=1024) == 8
    g, c = counts(small.replace(H=1), 122, 0)         # 122 against 3: at least 16 blocks a part
    assert bsa.suggest_dense_split(g, c, simds=1024) == 7
    tiny = W.workload("tiny_f32")                     # 7-block rows: shorter than two 16-block parts
    g, c = counts(tiny, 7, 2)
    assert bsa.suggest_dense_split(g, c, simds=1024) == 1
    g = bsa.Geometry(1, 2, 64, 0, 0, 0, 64, 32, 32, 64)    # text only: no frame-0 rows
    assert bsa.suggest_dense_split(g, torch.full((1, 2, 2), 2, dtype=torch.int32), simds=1024) == 1


def test_validation_under_host_sanitizers(tmp_path):
    """Every validation path of the C ABI, plus the host-only bsa_derive and
    bsa_classify_heads, driven by a plain C program (tests/c_abi/bsa_validate.c)
    against abi.cpp rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code (device code is built as usual).  No call reaches a
    launch, so no GPU is needed; any sanitizer report fails the run."""
    import subprocess
    from block_sparse_attention_42_amd import build as B
    objs = [os.path.join(B.OBJ, s + ".o") for s in B.SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(B.HIPCC):
        pytest.skip("library objects not built")
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("no clang")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    host_san = [f for s in san[:2] for f in ("-Xarch_host", s)] + ["-fno-omit-frame-pointer", "-g"]
    inc = os.path.join(ROOT, "include")
    abi_o = str(tmp_path / "abi_san.o")
    cmd = [B.HIPCC, *B.COMMON, *B.EXTRA["abi.cpp"], *host_san, "-c", os.path.join(B.CSRC, "abi.cpp"), "-o", abi_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = subprocess.run(["nm", "-u", abi_o], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms, "host code not instrumented"
    drv_o = str(tmp_path / "validate.o")
    r = subprocess.run([clang, "-std=c99", "-Wall", "-Werror", "-O1", *san, "-I", inc, "-c",
                        os.path.join(ROOT, "tests", "c_abi", "bsa_validate.c"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "bsa_validate")
    r = subprocess.run([clang + "++", *san, drv_o, abi_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "all validation checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
