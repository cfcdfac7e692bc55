"""Seeded synthetic inputs for block-sparse video attention.

This module only draws random tensors and names workload shapes.  It holds
none of the method's arithmetic (no pooling, scoring, selection or
attention), so both the CPU oracle's tests and the GPU path can take their
inputs from it without sharing any computation.

The workloads stand in for the video-DiT activations the pages measure on
(Wan2.1 and HunyuanVideo, AB-Attention page, TL;DR): tokens are packed as
``[text] + [frame0] + [frame1] + ...`` (frame-0 dense-rows page, section 1),
and Q/K are drawn around per-head centroids that are constant over
spatially contiguous patches of each frame, so that nearby query blocks
prefer the same key blocks, as clustered video attention does.  The recipe
is fixed here so that every run, on any machine, sees the same bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "seq_len", "seq_alloc", "bf16_round"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, selection policy and input recipe of one synthetic workload."""

    name: str
    B: int
    H: int
    D: int
    dtype: str               # "f32" or "bf16": storage type of Q, K, V and O
    text_len: int
    frames: int
    latent_h: int
    latent_w: int
    q_block: int
    k_block: int
    mode: str                # "topk" or "sample"
    topk: int                # explicit k (>0) or 0 to derive it from keep_ratio
    keep_ratio: float
    frame0_dense: bool
    text_columns: bool
    log_cluster: bool
    sample_seed: int         # key of the counter-based sampling generator
    data_seed: int           # seed of numpy's default_rng for the tensors
    centroids: int           # centroids per head
    grid: tuple              # (gh, gw) patch grid over latent_h x latent_w
    drift: float             # std of the per-frame random walk of centroids
    noise: float = 0.5       # std of the per-token noise around the centroid
    align: int = 64          # seq_alloc is S rounded up to this multiple

    @property
    def S(self) -> int:
        return seq_len(self)

    @property
    def seq_alloc(self) -> int:
        return seq_alloc(self)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def seq_len(w: Workload) -> int:
    return w.text_len + w.frames * w.latent_h * w.latent_w


def seq_alloc(w: Workload) -> int:
    a = max(w.align, w.q_block, w.k_block)
    return -(-seq_len(w) // a) * a


# The five workloads.  Names say what they are; sizes are the ones the
# block-sparse video-DiT setting uses (Wan2.1-1.3B-like: 12 heads of 128,
# 21 latent frames of 30x52; HunyuanVideo-like: 24 heads, 256 text tokens +
# 33 frames of 45x80).
WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", B=1, H=2, D=64, dtype="f32", text_len=32, frames=3,
        latent_h=8, latent_w=8, q_block=32, k_block=32, mode="topk", topk=2,
        keep_ratio=0.0, frame0_dense=True, text_columns=False, log_cluster=False,
        sample_seed=0, data_seed=0, centroids=16, grid=(4, 4), drift=0.0, align=32),
    "small_bf16": Workload(
        name="small_bf16", B=1, H=12, D=128, dtype="bf16", text_len=0, frames=5,
        latent_h=30, latent_w=52, q_block=64, k_block=64, mode="topk", topk=0,
        keep_ratio=0.25, frame0_dense=True, text_columns=False, log_cluster=False,
        sample_seed=1, data_seed=1, centroids=64, grid=(8, 8), drift=0.0),
    "wan_1p3b_keep10": Workload(
        name="wan_1p3b_keep10", B=1, H=12, D=128, dtype="bf16", text_len=0, frames=21,
        latent_h=30, latent_w=52, q_block=64, k_block=64, mode="topk", topk=0,
        keep_ratio=0.10, frame0_dense=True, text_columns=False, log_cluster=False,
        sample_seed=2, data_seed=2, centroids=128, grid=(8, 16), drift=0.1),
    "wan_1p3b_sampled_k16": Workload(
        name="wan_1p3b_sampled_k16", B=1, H=12, D=128, dtype="bf16", text_len=0,
        frames=21, latent_h=30, latent_w=52, q_block=64, k_block=16, mode="sample",
        topk=0, keep_ratio=0.10, frame0_dense=True, text_columns=False,
        log_cluster=False, sample_seed=3, data_seed=2, centroids=128, grid=(8, 16),
        drift=0.1),
    "hunyuan_keep08": Workload(
        name="hunyuan_keep08", B=1, H=24, D=128, dtype="bf16", text_len=256, frames=33,
        latent_h=45, latent_w=80, q_block=64, k_block=64, mode="topk", topk=0,
        keep_ratio=0.08, frame0_dense=True, text_columns=True, log_cluster=False,
        sample_seed=4, data_seed=4, centroids=256, grid=(16, 16), drift=0.0),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _patch_of_pixel(w: Workload) -> np.ndarray:
    """Centroid index of every pixel of one frame (row-major lh x lw)."""
    gh, gw = w.grid
    assert gh * gw == w.centroids
    y = np.arange(w.latent_h)[:, None]
    x = np.arange(w.latent_w)[None, :]
    return ((y * gh) // w.latent_h) * gw + (x * gw) // w.latent_w


def generate(w: Workload, heads: Optional[range] = None, pad_value: float = 0.0):
    """Draw Q, K, V as float32 numpy arrays of shape [B, H, seq_alloc, D].

    Per (b, h), in this order, from ``numpy.random.default_rng([data_seed, b, h])``:
    centroids ``M x D`` ~ N(0, 1); if ``drift`` > 0, ``frames-1`` steps of a
    random walk ``drift * N(0, 1)``; text Q and text K ~ N(0, 1); per-token
    Q noise and K noise ~ ``noise * N(0, 1)`` for the visual tokens; V ~
    N(0, 1) for all tokens.  Visual token (f, y, x) gets the centroid of its
    patch (the same patch map in every frame) in frame f.  Rows >= S hold
    ``pad_value``.  ``heads`` restricts the output to a sub-range of heads;
    every head has its own generator, so a head's values never depend on
    which heads were asked for.

    The caller casts to bfloat16 when ``w.dtype == "bf16"`` (round to
    nearest even, e.g. ``torch.Tensor.to(torch.bfloat16)``).
    """
    S, Sa, D = w.S, w.seq_alloc, w.D
    hs = range(w.H) if heads is None else heads
    npix = w.latent_h * w.latent_w
    patch = _patch_of_pixel(w).reshape(-1)
    nvis = w.frames * npix
    out = [np.full((w.B, len(hs), Sa, D), pad_value, dtype=np.float32) for _ in range(3)]
    for b in range(w.B):
        for h in hs:
            rng = np.random.default_rng([w.data_seed, b, h])
            cent = rng.standard_normal((w.centroids, D), dtype=np.float32)
            if w.drift > 0 and w.frames > 1:
                steps = rng.standard_normal((w.frames - 1, w.centroids, D), dtype=np.float32)
            else:
                steps = None
            tq = rng.standard_normal((w.text_len, D), dtype=np.float32)
            tk = rng.standard_normal((w.text_len, D), dtype=np.float32)
            nq = rng.standard_normal((nvis, D), dtype=np.float32)
            nk = rng.standard_normal((nvis, D), dtype=np.float32)
            v = rng.standard_normal((S, D), dtype=np.float32)
            hi = hs.index(h)
            # centroid of every frame: c^(0) = cent, c^(f) = c^(f-1) + drift*step
            if steps is not None:
                per_frame = np.concatenate(
                    [cent[None], cent[None] + np.cumsum(w.drift * steps, axis=0, dtype=np.float32)], axis=0)
            else:
                per_frame = np.broadcast_to(cent[None], (w.frames, w.centroids, D))
            base = per_frame[:, patch, :].reshape(nvis, D)
            q = out[0][b, hi]
            k = out[1][b, hi]
            q[:w.text_len] = tq
            k[:w.text_len] = tk
            q[w.text_len:S] = base + np.float32(w.noise) * nq
            k[w.text_len:S] = base + np.float32(w.noise) * nk
            out[2][b, hi, :S] = v
    return out[0], out[1], out[2]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even), returned as float32.

    Plain bit arithmetic on the float32 encoding; NaN stays NaN.  Used so the
    oracle sees exactly the values a bfloat16 tensor holds without needing
    torch.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = r.astype(np.uint32)
    nan = np.isnan(x)
    r[nan] = (u[nan].astype(np.uint32) | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return r.view(np.float32)
