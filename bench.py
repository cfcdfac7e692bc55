"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = the whole path on one batch: pool Q and K (one launch), build the mask
(logits, per-row top-k or sampling, overrides, lists), sparse forward.
Inputs are resident in HBM before the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

`value` is the effective throughput of a whole step: forward FLOPs on the
executed blocks (4 * D * q_block * k_block per selected block) divided by
the step time.  The forward alone (the dominant kernel) is reported in
`roofline` and `fwd_*`, timed with HIP events on the launch stream:
`fwd_ms_per_call` is the median over the timed steps, `roofline.achieved`
uses the mean launch duration.  After the headline workload, `configs` holds
the same figures for the other workloads (tiny f32 clip, 5-frame clip,
sampled 16-key blocks, HunyuanVideo-sized clip with text), timed the same
way over fewer steps.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd ms/call + effective TFLOP/s (frac of MFMA peak) at 90% sparsity"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3     # MI355X dense float32 MFMA (the float32 forward)
PEAK_HBM_GBS = 8000.0
# fp32 vector lane-ops without packed math: 256 CUs x 4 SIMDs x 16 lanes per clock at 2.4 GHz
PEAK_VALU_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan_1p3b_keep10")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-qblocks", type=int, default=512)
    ap.add_argument("--cpu-sample-heads", type=int, default=3)
    ap.add_argument("--cluster-clusters", type=int, default=4,
                    help="also time the intra-block clustering selector with this many clusters (0: skip)")
    ap.add_argument("--cluster-iters", type=int, default=3)
    ap.add_argument("--no-top-p", action="store_true", help="skip the top-p domain selector timing")
    ap.add_argument("--no-structured", action="store_true", help="skip the structured-list producer timing")
    ap.add_argument("--no-graph", action="store_true", help="skip the timing of the step replayed from a HIP graph")
    ap.add_argument("--dense-split", default="auto",
                    help="key split of the frame-0 rows in the forward: a number 1..16, or auto "
                         "(suggest_dense_split from the lists, chosen before the timed steps)")
    ap.add_argument("--configs", default="all",
                    help="the other workloads measured after the headline: all, none, or a comma list")
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--config-warmup", type=int, default=5)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


# the sources (and their compile flags) that make each forward kernel: the
# digest a committed profile was taken under
FWD_SOURCES = {"fwd_wide_kernel": ("forward_wide.hip", "fwd_common.h"),
               "fwd_kernel": ("forward.hip", "fwd_common.h"),
               "fwd_f32_kernel": ("forward_f32.hip", "fwd_common.h")}


def fwd_kernel_of(w):
    """The forward kernel a workload runs: the float32 kernel for float32
    inputs; for bf16 the 64-key-step kernel at head_dim 128 with 64-row query
    blocks, the general kernel otherwise."""
    if w.dtype != "bf16":
        return "fwd_f32_kernel"
    wide = w.D == 128 and w.q_block == 64 and w.k_block in (16, 32, 64)
    return "fwd_wide_kernel" if wide else "fwd_kernel"


def code_digest(kernel):
    """sha256 of a forward kernel's HIP sources with `//` comments and blank
    lines removed, plus their compile flags (the code the counters measured)."""
    from block_sparse_attention_42_amd.build import COMMON, EXTRA
    out = []
    for name in FWD_SOURCES[kernel]:
        for line in open(os.path.join(ROOT, "block_sparse_attention_42_amd", "csrc", name), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                out.append(code)
        out.append(" ".join(COMMON + EXTRA.get(name, [])))
    return hashlib.sha256("\n".join(out).encode()).hexdigest()


def _profile_record(kind, kernel, name, field):
    """A figure from a committed rocprofv3 record (profiles/<kind>_<kernel>_<workload>.json),
    if the forward's code is unchanged since the counters were taken."""
    f = os.path.join(ROOT, "profiles", f"{kind}_{kernel}_{name}.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if rec.get("forward_code_sha256") != code_digest(kernel):
        return None
    return rec.get(field)


def cpu_baseline(w, q, k, v, nblocks, nheads):
    """The oracle, as it stands, on the first `nheads` heads: per head, pooling
    and the mask of every row, then token-expanded attention of `nblocks`
    query blocks (the frame-0 rows among them)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    g = oracle.Geometry(1, 1, w.text_len, w.frames, w.latent_h, w.latent_w, w.D, w.q_block, w.k_block,
                        w.seq_alloc)
    p = oracle.MaskParams(mode=w.mode, topk=w.topk, keep_ratio=w.keep_ratio, frame0_dense=w.frame0_dense,
                          text_columns=w.text_columns, log_cluster=w.log_cluster, seed=w.sample_seed)
    nheads = max(1, min(nheads, w.H))
    nblocks = max(1, min(nblocks, g.nqb))
    flops = sec = wall = sec_g = wall_g = 0.0
    for h in range(nheads):
        q1, k1, v1 = q[:1, h:h + 1], k[:1, h:h + 1], v[:1, h:h + 1]
        rng = np.random.default_rng(h)
        f0 = list(g.frame0_q_blocks())
        qbl = sorted(set(f0[:max(1, nblocks // 10)]) |
                     set(rng.choice(g.nqb, nblocks, replace=False).tolist()))[:nblocks]
        t0 = time.perf_counter()
        qp = oracle.pool_blocks(q1, g.S, g.q_block)
        kp = oracle.pool_blocks(k1, g.S, g.k_block)
        _, cnt, idx, logw = oracle.build_mask(qp, kp, g, p)
        t1 = time.perf_counter()
        oracle.attention_head(q1[0, 0], k1[0, 0], v1[0, 0], g, cnt[0, 0], idx[0, 0], logw[0, 0], q_blocks=qbl)
        t2 = time.perf_counter()
        # the same rows with the listed blocks' keys gathered first (cost follows the selected blocks)
        oracle.attention_head_gathered(q1[0, 0], k1[0, 0], v1[0, 0], g, cnt[0, 0], idx[0, 0], logw[0, 0],
                                       q_blocks=qbl)
        t3 = time.perf_counter()
        flops += 4.0 * w.D * w.q_block * w.k_block * float(cnt[0, 0, qbl].sum())
        # the sampled q-blocks' share of one head's mask work is charged to them
        sec += (t2 - t1) + (t1 - t0) * len(qbl) / g.nqb
        sec_g += (t3 - t2) + (t1 - t0) * len(qbl) / g.nqb
        wall += t2 - t0
        wall_g += t3 - t2
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"heads 0..{nheads - 1} of {w.name}: per head, pooling + mask of all {g.nqb} rows "
                      f"(charged pro rata) and float64 token-expanded attention of {nblocks} query blocks "
                      f"({wall:.1f} s wall)",
            "seconds": round(wall, 2),
            "block_skipping": {"value": flops / sec_g / 1e12, "unit": "TFLOP/s",
                               "kind": "oracle with the listed blocks' keys gathered (cost follows the selected "
                                       "blocks; a fairer CPU speed reference, not the parity oracle)",
                               "seconds": round(wall_g, 2)}}


def cluster_selector_timing(bsa, w, g, p, qd, kp, C, T, nqb, nkb, stream, ev, reps=20):
    """Intra-block clustering selector on the same inputs: importance, then selection.

    Not part of the timed step.  VALU work per query block (lane-ops):
    k-means (T+1) * n * C * D * 3 + T * n * C * D, logits C * nkb * D * 2;
    the exponentials and the mixture are counted as C * nkb * 30.  The
    k-means term counts all T rounds; the kernel stops once an assignment
    repeats, so the rate is an effective one.
    """
    import numpy as np
    import torch
    imp = torch.empty((w.B, w.H, nqb, nkb), dtype=torch.float32, device=qd.device)
    cnt = torch.empty((w.B, w.H, nqb), dtype=torch.int32, device=qd.device)
    idx = torch.empty((w.B, w.H, nqb, nkb), dtype=torch.int32, device=qd.device)
    logw = torch.empty((w.B, w.H, nqb, nkb), dtype=torch.float32, device=qd.device) if w.mode == "sample" else None
    for _ in range(3):
        bsa.bsa_cluster_importance(qd, kp, g, C, T, w.log_cluster, out=imp)
        bsa.bsa_select_blocks(imp, g, p, want_mask=False, out=(None, cnt, idx, logw))
    torch.cuda.synchronize()
    ti, ts = [], []
    for _ in range(reps):
        e = [ev() for _ in range(3)]
        e[0].record(stream)
        bsa.bsa_cluster_importance(qd, kp, g, C, T, w.log_cluster, out=imp)
        e[1].record(stream)
        bsa.bsa_select_blocks(imp, g, p, want_mask=False, out=(None, cnt, idx, logw))
        e[2].record(stream)
        ti.append(e)
    torch.cuda.synchronize()
    imp_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ti]))
    sel_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ti]))
    n = w.q_block
    ops_row = (T + 1) * n * C * w.D * 3 + T * n * C * w.D + C * nkb * w.D * 2 + C * nkb * 30
    lane_ops = float(w.B * w.H * nqb) * ops_row
    tops = lane_ops / (imp_ms * 1e-3) / 1e12
    return {"n_clusters": C, "iters": T, "importance_ms": round(imp_ms, 4), "select_ms": round(sel_ms, 4),
            "executed_blocks": int(cnt.sum().item()),
            "roofline": {"bound": "alu", "kernel": "importance_kernel", "achieved": round(tops, 2),
                         "peak": PEAK_VALU_TLANEOPS, "unit": "T lane-ops/s",
                         "frac": round(tops / PEAK_VALU_TLANEOPS, 4)}}


def top_p_timing(bsa, w, g, qd, kd, vd, kp, nqb, nkb, stream, ev, reps=20):
    """EG-Sparse routing (low-entropy heads pooled with value-aware scores, the
    rest per-row local), top-p 0.9, on P' of the same inputs (one cluster).

    Not part of the timed step.  Bytes counted: the scores read by the
    entropy and the selection passes (every head) and by the four radix
    passes (the pooled floor(H/2) heads), the pooled value rows read once for
    their norms, and the mask, counts and lists written once.
    """
    import ctypes
    import numpy as np
    import torch
    vp = bsa.bsa_pool_blocks(vd, g, g.k_block)
    P = bsa.bsa_cluster_importance(qd, kp, g, 1, 1, w.log_cluster)
    nbytes = ctypes.c_int64()
    bsa._lib.check(bsa._lib.lib().bsa_top_p_workspace_bytes(ctypes.byref(g.c()), ctypes.byref(nbytes)))
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=qd.device)
    for _ in range(3):
        bsa.bsa_select_top_p(P, g, "eg", 0.9, v_pooled=vp, value_aware=True, frame0_dense=w.frame0_dense,
                             workspace=ws)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e = [ev() for _ in range(2)]
        e[0].record(stream)
        mask, cnt, idx, ent = bsa.bsa_select_top_p(P, g, "eg", 0.9, v_pooled=vp, value_aware=True,
                                                   frame0_dense=w.frame0_dense, workspace=ws)
        e[1].record(stream)
        ts.append(e)
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in ts]))
    n = w.B * w.H * nqb * nkb
    kept = int(cnt.sum().item())
    pooled = (w.H // 2) / w.H
    byts = (2.0 + 4.0 * pooled) * n * 4 + w.B * w.H * nkb * w.D * 4 + n + 4.0 * kept + w.B * w.H * nqb * 4
    gbs = byts / (ms * 1e-3) / 1e9
    return {"domain": "eg", "value_aware": True, "top_p": 0.9, "select_ms": round(ms, 4),
            "executed_blocks": kept,
            "roofline": {"bound": "hbm", "kernel": "tp_* (selection passes)", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def structured_timing(bsa, w, g, qd, kd, vd, kp, nqb, nkb, stream, ev, window=3, reps=20):
    """Per-head frame contexts: frame scores of P' (one cluster), host-side head
    labelling with half the heads dummy heads, block-causal full heads, neighbor
    window 3; then the list producer and the forward on its lists (frame-run
    launch order, and the default order for comparison).

    Not part of the timed step.  Algorithmic bytes: the frame-score kernel reads
    the P' entries of the sink, neighbor and current runs of every scored row;
    the list producer writes the mask, counts and lists once.
    """
    import numpy as np
    import torch
    P = bsa.bsa_cluster_importance(qd, kp, g, 1, 1, w.log_cluster)
    alpha = bsa.bsa_frame_scores(P, g, window)
    cls = torch.from_numpy(bsa.bsa_classify_heads(alpha.cpu(), w.H // 2)).to(qd.device)
    out = torch.empty_like(qd)

    def lists():
        return bsa.bsa_structured_lists(cls, g, window, block_causal=True, frame0_dense=w.frame0_dense)
    for _ in range(3):
        bsa.bsa_frame_scores(P, g, window)
        _, cnt, idx = lists()
        bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, out=out, launch_order="frame_runs")
        bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, out=out)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e = [ev() for _ in range(5)]
        e[0].record(stream)
        bsa.bsa_frame_scores(P, g, window)
        e[1].record(stream)
        mask, cnt, idx = lists()
        e[2].record(stream)
        bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, out=out, launch_order="frame_runs")
        e[3].record(stream)
        bsa.bsa_forward(qd, kd, vd, g, cnt, idx, None, out=out)
        e[4].record(stream)
        ts.append(e)
    torch.cuda.synchronize()
    fs_ms, ls_ms, fw_ms, fp_ms = (float(np.median([e[k].elapsed_time(e[k + 1]) for e in ts])) for k in range(4))
    kept = int(cnt.sum().item())
    # P' entries the frame-score kernel reads (integer geometry of the frame runs)
    tpf = w.latent_h * w.latent_w

    def first_block(f):
        return -(-min(w.text_len + f * tpf, w.S) // w.k_block)
    read = 0
    for i in range(nqb):
        t = i * w.q_block
        f = -1 if t < w.text_len else (t - w.text_len) // tpf
        if f >= 1:
            read += first_block(1) - first_block(0) + first_block(f + 1) - first_block(max(1, f - window + 1))
    fs_bytes = 4.0 * read * w.B * w.H
    ls_bytes = w.B * w.H * nqb * (nkb + 4) + 4.0 * kept
    gbs = ls_bytes / (ls_ms * 1e-3) / 1e9
    tf = 4.0 * w.D * w.q_block * w.k_block * kept / (fw_ms * 1e-3) / 1e12
    counts = {c: int((cls.cpu() == i).sum()) for i, c in enumerate(("full", "sink", "neighbor", "dummy"))}
    return {"window": window, "heads": counts, "block_causal": True,
            "frame_scores_ms": round(fs_ms, 4), "frame_scores_gbs": round(fs_bytes / (fs_ms * 1e-3) / 1e9, 1),
            "lists_ms": round(ls_ms, 4), "executed_blocks": kept,
            "density": round(kept / (w.B * w.H * nqb * nkb), 4),
            "fwd_launch_order": "frame_runs", "fwd_ms": round(fw_ms, 4), "fwd_tflops": round(tf, 2),
            "fwd_ms_frame_position_order": round(fp_ms, 4),
            "roofline": {"bound": "hbm", "kernel": "struct_lists_kernel", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def graph_timing(torch, step, stream, ev, steps, out):
    """The same step captured once in a HIP graph and replayed: ms per replay,
    and whether a replay rewrites the eager step's output bit for bit."""
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                            ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref))
    s0, s1 = ev(), ev()
    s0.record(stream)
    for _ in range(steps):
        graph.replay()
    s1.record(stream)
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    del graph
    return {"ms_per_step": round(ms, 4), "replay_identical_to_eager": same}


class PathRun:
    """The hot path on one workload: inputs resident on the GPU, output
    buffers allocated once, the key split of the frame-0 rows chosen from the
    lists after warmup; `timed(steps)` times whole steps and each stage."""

    def __init__(self, bsa, torch, w, warmup, dense_split="auto", keep_host=False):
        import workloads as W
        self.bsa, self.torch, self.w = bsa, torch, w
        t_gen = time.perf_counter()
        q, k, v = W.generate(w)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = torch.device("cuda:0")
        self.qd, self.kd, self.vd = (torch.from_numpy(x).to(dt).to(dev) for x in (q, k, v))
        if keep_host:
            if w.dtype == "bf16":     # what the oracle sees: the bf16 values
                q, k, v = (t.float().cpu().numpy() for t in (self.qd, self.kd, self.vd))
            self.host = (q, k, v)
        del q, k, v
        self.input_gen_s = time.perf_counter() - t_gen
        self.g = g = bsa.Geometry(w.B, w.H, w.text_len, w.frames, w.latent_h, w.latent_w, w.D, w.q_block,
                                  w.k_block, w.seq_alloc)
        self.p = bsa.MaskParams(mode=w.mode, topk=w.topk, keep_ratio=w.keep_ratio, frame0_dense=w.frame0_dense,
                                text_columns=w.text_columns, log_cluster=w.log_cluster, seed=w.sample_seed)
        d = bsa.bsa_derive(g, self.p)
        self.nqb, self.nkb = nqb, nkb = d["nqb"], d["nkb"]
        self.qp = torch.empty((w.B, w.H, nqb, w.D), dtype=torch.float32, device=dev)
        self.kp = torch.empty((w.B, w.H, nkb, w.D), dtype=torch.float32, device=dev)
        self.mask = torch.empty((w.B, w.H, nqb, nkb), dtype=torch.uint8, device=dev)
        self.cnt = torch.empty((w.B, w.H, nqb), dtype=torch.int32, device=dev)
        self.idx = torch.empty((w.B, w.H, nqb, nkb), dtype=torch.int32, device=dev)
        self.logw = (torch.empty((w.B, w.H, nqb, nkb), dtype=torch.float32, device=dev)
                     if w.mode == "sample" else None)
        self.out = torch.empty_like(self.qd)
        self.stream = torch.cuda.current_stream()
        self.split, self.ws = 1, None
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        # the key split of the frame-0 rows: chosen from the lists, outside the timed region
        split = bsa.suggest_dense_split(g, self.cnt) if dense_split == "auto" else int(dense_split)
        if split != 1:
            self.split = split
            self.ws = torch.empty(max(bsa.bsa_forward_split_workspace_bytes(g, split), 16), dtype=torch.uint8,
                                  device=dev)
            for _ in range(2):
                self.step()
            torch.cuda.synchronize()
        self.blocks = int(self.cnt.sum().item())
        self.flops = 4.0 * w.D * w.q_block * w.k_block * self.blocks

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def step(self, times=None):
        bsa, g, s = self.bsa, self.g, self.stream
        e = [self.ev() for _ in range(4)] if times is not None else None
        if e: e[0].record(s)
        bsa.bsa_pool_qk(self.qd, self.kd, g, out=(self.qp, self.kp))
        if e: e[1].record(s)
        bsa.bsa_build_mask(self.qp, self.kp, g, self.p, out=(self.mask, self.cnt, self.idx, self.logw))
        if e: e[2].record(s)
        bsa.bsa_forward(self.qd, self.kd, self.vd, g, self.cnt, self.idx, self.logw, out=self.out,
                        dense_split=self.split, workspace=self.ws)
        if e:
            e[3].record(s)
            times.append(e)

    def timed(self, steps):
        """Whole steps bracketed by synchronize on both sides; per-stage HIP
        events on the launch stream."""
        import numpy as np
        torch, w = self.torch, self.w
        times = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s0 = self.ev()
        s0.record(self.stream)
        for _ in range(steps):
            self.step(times)
        s1 = self.ev()
        s1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = s0.elapsed_time(s1) / steps
        pool_ms = float(np.median([e[0].elapsed_time(e[1]) for e in times]))
        mask_ms = float(np.median([e[1].elapsed_time(e[2]) for e in times]))
        fwd_times = [e[2].elapsed_time(e[3]) for e in times]
        nqb, nkb, esz = self.nqb, self.nkb, (2 if w.dtype == "bf16" else 4)
        pool_bytes = 2 * w.B * w.H * w.S * w.D * esz + w.B * w.H * (nqb + nkb) * w.D * 4
        # mask: the logits are D non-fused multiplies and D adds each (the VALU-bound part); its bytes are
        # the pooled summaries in, and the mask, counts, listed indices (and log-weights) out
        mask_lane_ops = 2.0 * w.B * w.H * nqb * nkb * w.D
        mask_bytes = (w.B * w.H * (nqb + nkb) * w.D * 4 + w.B * w.H * nqb * nkb + w.B * w.H * nqb * 4
                      + self.blocks * 4 * (2 if self.logw is not None else 1))
        return {"step_ms": step_ms, "wall": wall, "pool_ms": pool_ms, "mask_ms": mask_ms,
                "fwd_ms": float(np.median(fwd_times)),          # ms per forward call: the median
                "fwd_ms_mean": float(np.mean(fwd_times)),       # the average launch duration, for the roofline
                "pool_bytes": pool_bytes, "mask_bytes": mask_bytes, "mask_lane_ops": mask_lane_ops}

    def summary(self, m):
        """Per-workload figures: forward, pooling and mask times and their roofline fractions."""
        w = self.w
        kernel = fwd_kernel_of(w)
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
        tf = self.flops / (m["fwd_ms"] * 1e-3) / 1e12
        tf_avg = self.flops / (m["fwd_ms_mean"] * 1e-3) / 1e12
        pool_gbs = m["pool_bytes"] / (m["pool_ms"] * 1e-3) / 1e9
        mask_tops = m["mask_lane_ops"] / (m["mask_ms"] * 1e-3) / 1e12
        return {"B": w.B, "H": w.H, "head_dim": w.D, "seq_len": w.S, "q_block": w.q_block, "k_block": w.k_block,
                "selection": w.mode, "keep_ratio": w.keep_ratio, "topk": w.topk, "dtype": w.dtype,
                "text_columns": w.text_columns, "dense_split": self.split,
                "ms_per_step": round(m["step_ms"], 4),
                "step_tflops": round(self.flops / (m["step_ms"] * 1e-3) / 1e12, 2),
                "fwd_kernel": kernel, "fwd_ms": round(m["fwd_ms"], 4), "fwd_ms_mean": round(m["fwd_ms_mean"], 4),
                "fwd_tflops": round(tf, 2), "fwd_frac": round(tf_avg / peak, 4), "fwd_peak_tflops": peak,
                "fwd_hbm_bytes": _profile_record("traffic", kernel, w.name, "hbm_bytes_per_launch"),
                "pool_ms": round(m["pool_ms"], 4), "pool_gbs": round(pool_gbs, 1),
                "pool_frac": round(pool_gbs / PEAK_HBM_GBS, 4),
                "mask_ms": round(m["mask_ms"], 4), "mask_valu_frac": round(mask_tops / PEAK_VALU_TLANEOPS, 4),
                "executed_blocks": self.blocks, "density": round(self.blocks / (w.B * w.H * self.nqb * self.nkb), 4)}


HEADLINE = "wan_1p3b_keep10"
OTHER_WORKLOADS = ("tiny_f32", "small_bf16", "wan_1p3b_sampled_k16", "hunyuan_keep08")


def main():
    a = _args()
    if a.calibrate_copy_mib:
        import torch
        n = a.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU: the path has no multi-GPU part "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_42_amd as bsa
    import workloads as W

    w = W.workload(a.workload)
    run = PathRun(bsa, torch, w, a.warmup, a.dense_split, keep_host=not a.no_cpu_baseline)
    m = run.timed(a.steps)
    summ = run.summary(m)
    kernel = summ["fwd_kernel"]
    g, nqb, nkb = run.g, run.nqb, run.nkb
    fwd_tflops_avg = run.flops / (m["fwd_ms_mean"] * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(run.flops / (m["step_ms"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(m["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded clustered Q/K, V ~ N(0,1); stands in for Wan2.1 activations)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "head_dim": w.D, "seq_len": w.S,
                   "seq_alloc": w.seq_alloc, "q_block": w.q_block, "k_block": w.k_block,
                   "selection": w.mode, "keep_ratio": w.keep_ratio, "frame0_dense": w.frame0_dense,
                   "text_columns": w.text_columns, "dense_split": run.split},
        "fwd_ms_per_call": summ["fwd_ms"],
        "fwd_ms_mean": summ["fwd_ms_mean"],
        "fwd_tflops": summ["fwd_tflops"],
        "fwd_frac_of_bf16_peak": round(summ["fwd_tflops"] / PEAK_BF16_TFLOPS, 4),
        "pool_ms": summ["pool_ms"],
        "pool_gbs": summ["pool_gbs"],
        "pool_hbm": {"bound": "hbm", "achieved": summ["pool_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": summ["pool_frac"]},
        "mask_ms": summ["mask_ms"],
        "mask_gbs": round(m["mask_bytes"] / (m["mask_ms"] * 1e-3) / 1e9, 1),
        "mask_valu": {"bound": "alu",
                      "achieved": round(m["mask_lane_ops"] / (m["mask_ms"] * 1e-3) / 1e12, 2),
                      "peak": round(PEAK_VALU_TLANEOPS, 2), "unit": "T lane-ops/s",
                      "frac": summ["mask_valu_frac"]},
        "executed_blocks": run.blocks,
        "density": summ["density"],
        "wall_s_timed": round(m["wall"], 3),
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(fwd_tflops_avg, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops_avg / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profile_record("traffic", kernel, w.name, "hbm_bytes_per_launch"),
                     "mfma_busy": _profile_record("sq", kernel, w.name, "mfma_busy_frac"),
                     "clock_ghz": _profile_record("sq", kernel, w.name, "clock_ghz")},
    }
    qd, kd, vd, kp, stream, ev = run.qd, run.kd, run.vd, run.kp, run.stream, run.ev
    if not a.no_graph:
        res["graph_step"] = graph_timing(torch, run.step, stream, ev, a.steps, run.out)
    if a.cluster_clusters > 0 and a.cluster_clusters * nkb <= 16384:
        res["cluster_selector"] = cluster_selector_timing(bsa, w, g, run.p, qd, kp, a.cluster_clusters,
                                                          a.cluster_iters, nqb, nkb, stream, ev)
    if not a.no_top_p and nkb <= 2048:
        res["top_p_selector"] = top_p_timing(bsa, w, g, qd, kd, vd, kp, nqb, nkb, stream, ev)
    if not a.no_structured:
        res["structured_lists"] = structured_timing(bsa, w, g, qd, kd, vd, kp, nqb, nkb, stream, ev)
    if not a.no_cpu_baseline:
        q, k, v = run.host
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, a.cpu_sample_qblocks, a.cpu_sample_heads)
        del run.host, q, k, v
    res["input_gen_s"] = round(run.input_gen_s, 1)
    del run, qd, kd, vd, kp
    torch.cuda.empty_cache()
    # the other workloads: the same step, fewer steps, figures only
    names = [] if a.configs == "none" else (
        [n for n in OTHER_WORKLOADS if n != w.name] if a.configs == "all" else a.configs.split(","))
    if names:
        res["configs"] = {w.name: summ}
        for name in names:
            r = PathRun(bsa, torch, W.workload(name), a.config_warmup)
            res["configs"][name] = r.summary(r.timed(a.config_steps))
            del r
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
