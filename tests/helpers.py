"""Test-side glue: turn a workload into oracle arguments (no method arithmetic)."""
import numpy as np

import oracle
import workloads as W


def geometry_of(w: W.Workload) -> oracle.Geometry:
    return oracle.Geometry(B=w.B, H=w.H, text_len=w.text_len, frames=w.frames,
                           latent_h=w.latent_h, latent_w=w.latent_w, head_dim=w.D,
                           q_block=w.q_block, k_block=w.k_block, seq_alloc=w.seq_alloc)


def params_of(w: W.Workload) -> oracle.MaskParams:
    return oracle.MaskParams(mode=w.mode, topk=w.topk, keep_ratio=w.keep_ratio,
                             frame0_dense=w.frame0_dense, text_columns=w.text_columns,
                             log_cluster=w.log_cluster, seed=w.sample_seed)


def inputs_of(w: W.Workload, heads=None, pad_value=0.0):
    """Q, K, V float32 arrays holding exactly the values the GPU sees."""
    q, k, v = W.generate(w, heads=heads, pad_value=pad_value)
    if w.dtype == "bf16":
        q, k, v = (W.bf16_round(a) for a in (q, k, v))
    return q, k, v


def tiny(text_len=5, frames=2, lh=3, lw=5, bq=8, bk=8, D=16, H=2, B=1, **kw):
    """A small ragged workload (S not a multiple of the block sizes)."""
    base = W.workload("tiny_f32")
    align = kw.pop("align", max(bq, bk))
    M = kw.pop("centroids", 4)
    grid = kw.pop("grid", (2, 2) if M == 4 else (1, M))
    return base.replace(name="tiny_ragged", B=B, H=H, D=D, text_len=text_len, frames=frames,
                        latent_h=lh, latent_w=lw, q_block=bq, k_block=bk, align=align,
                        centroids=M, grid=grid, **kw)
