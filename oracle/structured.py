"""Structured mask producers over the same forward: CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module; the library never imports, links or runs it.

Sources:
* "Efficient Autoregressive Video Diffusion with Dummy Head" (Dummy-Head
  page): per-head frame attention scores [a_sink, a_neighbor, a_current]
  (its Step 0); Dynamic Head Programming, the greedy labelling that makes
  the N heads of smallest max(a_sink, a_neighbor) dummy heads and the rest
  sink or neighbor heads by the larger of the two (its Step 1 and the
  8-head worked example); Heterogeneous Memory Allocation, the per-class
  context: sink heads see the sink frame and the current frame, neighbor
  heads a window of the last L frames (current included), dummy heads the
  current frame, or frames i-1 and i when packed (its Steps 2 and 3).
* The block-causal frame mask of "Purpose of the block-causal mask ..."
  (block-causal page): a frame attends to itself and earlier frames.
* "Attention matrix view: make only frame-0 query rows dense" (frame-0
  page): token packing [text] + [frame 0] + [frame 1] + ... (sec. 1);
  optional dense frame-0 rows (sec. 4) and text blocks (sec. 7).

Readings (the pages describe autoregressive generation with a KV cache;
here the same contexts become block lists of one bidirectional sequence):
* Token t belongs to frame -1 (text) if t < text_len, else to frame
  (t - text_len) // (latent_h * latent_w).  A block covers the frames of its
  valid tokens, an interval.  The sink frame is frame 0.
* A query block's context is the union, over the frames f of its tokens, of
  its head class's frames for f; text is in every context (the prompt), and
  a query block holding text tokens sees everything.  A key block is listed
  iff it covers a frame of that context.  Classes: full (every frame; with
  block-causal on, frames <= f), sink ({0, f}), neighbor ({f-L+1 .. f},
  clipped at 0), dummy ({f}, or {f-1, f} with the previous frame on).
* Frame scores of a head: for every query block whose first token is in a
  frame f >= 1, the P' mass on key blocks whose first token is in frame 0
  (sink), in frames f-L+1 .. f-1 above 0 (neighbor) and in frame f
  (current), normalized to sum 1; the mean over those blocks (float64).
  Text key blocks count in none of the three.
* DHP ties: lower head index first; a head with a_sink == a_neighbor is a
  neighbor head.
"""
from __future__ import annotations

import numpy as np

from .reference import Geometry

FULL, SINK, NEIGHBOR, DUMMY = 0, 1, 2, 3


def token_frame(g: Geometry, t: int) -> int:
    if t < g.text_len:
        return -1
    return (t - g.text_len) // (g.latent_h * g.latent_w)


def block_frame_range(g: Geometry, block: int, i: int):
    """(first, last) frame of the valid tokens of block i of size ``block``."""
    lo = i * block
    hi = min(lo + block, g.S) - 1
    return token_frame(g, lo), token_frame(g, hi)


def context_frames(cls: int, f: int, L: int, dummy_prev: bool, causal: bool, n_frames: int) -> set:
    """Frames (and -1 for text) a query token of frame f sees under head class ``cls``."""
    everything = set(range(-1, n_frames))
    if f < 0:
        return everything
    if cls == FULL:
        return set(range(-1, f + 1)) if causal else everything
    if cls == SINK:
        return {-1, 0, f}
    if cls == NEIGHBOR:
        return {-1} | set(range(max(0, f - L + 1), f + 1))
    if cls == DUMMY:
        return {-1, f} | ({f - 1} if (dummy_prev and f >= 1) else set())
    raise ValueError(cls)


def structured_lists(g: Geometry, classes: np.ndarray, L: int, dummy_prev: bool = False,
                     block_causal: bool = False, frame0_dense: bool = False, text_columns: bool = False):
    """Mask, counts and ascending lists [B,H,nqb,nkb] of the per-head structured contexts."""
    classes = np.asarray(classes)
    B, H = classes.shape
    mask = np.zeros((B, H, g.nqb, g.nkb), dtype=bool)
    qr = [block_frame_range(g, g.q_block, i) for i in range(g.nqb)]
    kr = [block_frame_range(g, g.k_block, j) for j in range(g.nkb)]
    for b in range(B):
        for h in range(H):
            for i, (q0, q1) in enumerate(qr):
                ctx = set()
                for f in range(q0, q1 + 1):
                    ctx |= context_frames(int(classes[b, h]), f, L, dummy_prev, block_causal, g.frames)
                for j, (k0, k1) in enumerate(kr):
                    if any(f in ctx for f in range(k0, k1 + 1)):
                        mask[b, h, i, j] = True
    for i in (g.frame0_q_blocks() if frame0_dense else []):
        mask[:, :, i, :] = True
    for j in (g.text_k_blocks() if text_columns else []):
        mask[:, :, :, j] = True
    cnt = mask.sum(-1).astype(np.int32)
    idx = np.full(mask.shape, -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(g.nqb):
                js = np.nonzero(mask[b, h, i])[0]
                idx[b, h, i, :len(js)] = js
    return mask, cnt, idx


def frame_scores(P: np.ndarray, g: Geometry, L: int) -> np.ndarray:
    """[B, H, 3] = mean over query blocks of a frame f >= 1 of the normalized
    (sink, neighbor, current) P' mass (float64)."""
    P = np.asarray(P, dtype=np.float64)
    B, H, nqb, nkb = P.shape
    kf = np.array([token_frame(g, j * g.k_block) for j in range(nkb)])
    out = np.zeros((B, H, 3))
    rows = [i for i in range(nqb) if token_frame(g, i * g.q_block) >= 1]
    for i in rows:
        f = token_frame(g, i * g.q_block)
        sink = kf == 0
        nb = (kf >= max(1, f - L + 1)) & (kf <= f - 1)
        cur = kf == f
        a = np.stack([P[:, :, i][..., sink].sum(-1), P[:, :, i][..., nb].sum(-1), P[:, :, i][..., cur].sum(-1)], -1)
        s = a.sum(-1, keepdims=True)
        out += np.where(s > 0, a / np.where(s > 0, s, 1.0), 0.0)
    return out / max(1, len(rows))


def classify_heads(alpha: np.ndarray, n_dummy: int) -> np.ndarray:
    """DHP: per batch element, the n_dummy heads of smallest max(a_sink, a_neighbor)
    (lower head first among equals) are dummy heads; the others are sink heads if
    a_sink > a_neighbor, else neighbor heads."""
    alpha = np.asarray(alpha, dtype=np.float64)
    B, H, _ = alpha.shape
    cls = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        lh = [max(alpha[b, h, 0], alpha[b, h, 1]) for h in range(H)]
        order = sorted(range(H), key=lambda h: (lh[h], h))
        dummy = set(order[:n_dummy])
        for h in range(H):
            cls[b, h] = DUMMY if h in dummy else (SINK if alpha[b, h, 0] > alpha[b, h, 1] else NEIGHBOR)
    return cls
