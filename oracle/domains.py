"""Top-p selection over competition domains: CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module; the library never imports, links or runs it.

Source: "Competition Domains Matter ... (EG-Sparse)" (EG-Sparse page).
* Scores: P' of each (head, query block, key block), the cluster-size-weighted
  softmax of its Eq. 2 (here the rows of an importance matrix, e.g.
  ``cluster_select.cluster_importance`` with one cluster).
* Per-head entropy (its Eq. 3): H_h = (1/C_q) sum_i sum_j -P' log(P' + eps).
* The domain hierarchy of its Section 3.3: per-row local, per-head global,
  grouped cross-head (low- and high-entropy heads, split at the median, each
  a pool), all-head global; its deployed method routes only the low-entropy
  heads to a shared pool and keeps per-row local selection for the rest.
* Top-p: a domain keeps the top-p portion of its scores' mass.
* The minimum one-key-per-row safeguard for the expanded domains.
* The value-aware score of the cross-head pool: P' times the norm of the
  key cluster's value centroid.

Readings (the pages fix none of these details):
* Mass is counted in fixed point: m(s) = floor(s * 2^32) + 1 per block, an
  integer, so a pool's mass is exact in any summation order (the +1 keeps
  every block's mass positive; it moves a pool's total by 2^-32 per block).
  target = ceil(p * total) in double.  The kept set of a domain is every
  block whose score is at least T, the largest score with
  mass(score >= T) >= target; blocks equal to T are all kept.
* The median split: in each batch element, the floor(H/2) heads of lowest
  entropy (lower head index first among equals) are the low-entropy heads.
* Entropy uses eps as given, natural log, float64.
* The value norm of key block j: ``acc = 0; for d ascending:
  acc = fl32(acc + fl32(v̄_d * v̄_d))``, ``fl32(sqrt(acc))``; the value-aware
  score is fl32(P' * norm).  Value-aware scores are used only in pooled
  domains (the page replaces P' in the cross-head pool).
* The safeguard keeps, in a pooled domain, the first block of largest score
  of a row left empty.  Frame-0 rows and text columns are applied after, as
  in ``reference.build_mask``.
"""
from __future__ import annotations

import math

import numpy as np

from .reference import F32, Geometry

DOMAINS = ("row", "head", "split", "all", "eg")
FIX_SCALE = 2.0 ** 32


def order_keys(s: np.ndarray) -> np.ndarray:
    """uint32 keys ordered as the non-negative float32 scores."""
    u = np.asarray(s, dtype=F32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def fixed_mass(s: np.ndarray) -> np.ndarray:
    """m(s) = floor(s * 2^32) + 1 as uint64 (s >= 0, float32; the product is exact in float64)."""
    return (np.floor(np.asarray(s, dtype=F32).astype(np.float64) * FIX_SCALE) + 1).astype(np.uint64)


def top_p_threshold(scores: np.ndarray, p: float) -> int:
    """Key T of the largest score with mass(score >= T) >= ceil(p * mass(all))."""
    s = np.asarray(scores, dtype=F32).ravel()
    keys = order_keys(s)
    mass = fixed_mass(s)
    total = int(mass.sum(dtype=np.uint64))
    target = int(math.ceil(p * float(total)))
    uk, inv = np.unique(keys, return_inverse=True)           # ascending unique keys
    group = np.zeros(uk.shape[0], dtype=object)
    np.add.at(group, inv, mass.astype(object))
    acc = 0
    for g in range(uk.shape[0] - 1, -1, -1):                 # descending keys
        acc += int(group[g])
        if acc >= target:
            return int(uk[g])
    return int(uk[0])


def value_norms(vp: np.ndarray) -> np.ndarray:
    """fl32 norm of every pooled value row [..., nkb, D], channels in ascending order."""
    vp = np.asarray(vp, dtype=F32)
    acc = np.zeros(vp.shape[:-1], dtype=F32)
    for d in range(vp.shape[-1]):
        acc = acc + vp[..., d] * vp[..., d]
    return np.sqrt(acc).astype(F32)


def head_entropy(P: np.ndarray, eps: float) -> np.ndarray:
    """H[b, h] = (1/nqb) sum_i sum_j -P log(P + eps), float64."""
    P = np.asarray(P, dtype=np.float64)
    return (-(P * np.log(P + float(F32(eps))))).sum(axis=(-1, -2)) / P.shape[-2]


def head_pools(H_bh: np.ndarray, domain: str) -> np.ndarray:
    """Pool id of every (b, h): -1 = per-row local; pools are numbered per batch element."""
    B, H = H_bh.shape
    pool = np.full((B, H), -1, dtype=np.int64)
    for b in range(B):
        order = sorted(range(H), key=lambda h: (H_bh[b, h], h))
        low = set(order[:H // 2])
        for h in range(H):
            if domain == "row":
                pool[b, h] = -1
            elif domain == "head":
                pool[b, h] = b * H + h
            elif domain == "all":
                pool[b, h] = b
            elif domain == "split":
                pool[b, h] = 2 * b + (0 if h in low else 1)
            elif domain == "eg":
                pool[b, h] = b if h in low else -1
            else:
                raise ValueError(domain)
    return pool


def select_top_p(P: np.ndarray, g: Geometry, domain: str, p: float, vp=None, eps: float = 1e-12,
                 frame0_dense: bool = False, text_columns: bool = False):
    """Top-p block mask over competition domains and its compacted lists.

    ``P``: [B, H, nqb, nkb] float32 scores (P').  ``vp``: pooled values
    [B, H, nkb, D] for value-aware scores in pooled domains, or None.
    Returns (mask bool, cnt int32, idx int32, entropy float64 [B, H]).
    """
    P = np.asarray(P, dtype=F32)
    B, H, nqb, nkb = P.shape
    ent = head_entropy(P, eps)
    pool = head_pools(ent, domain)
    score = P.copy()
    if vp is not None:
        vn = value_norms(vp)                                   # [B, H, nkb]
        for b in range(B):
            for h in range(H):
                if pool[b, h] >= 0:
                    score[b, h] = (P[b, h] * vn[b, h][None, :]).astype(F32)
    mask = np.zeros((B, H, nqb, nkb), dtype=bool)
    # per-row local
    for b in range(B):
        for h in range(H):
            if pool[b, h] < 0:
                for i in range(nqb):
                    T = top_p_threshold(score[b, h, i], p)
                    mask[b, h, i] = order_keys(score[b, h, i]) >= T
    # pooled domains
    for pid in sorted(set(pool[pool >= 0].tolist())):
        members = [(b, h) for b in range(B) for h in range(H) if pool[b, h] == pid]
        T = top_p_threshold(np.concatenate([score[b, h].ravel() for (b, h) in members]), p)
        for (b, h) in members:
            mask[b, h] = order_keys(score[b, h]) >= T
            for i in range(nqb):
                if not mask[b, h, i].any():                     # one-key-per-row safeguard
                    mask[b, h, i, int(np.argmax(score[b, h, i]))] = True
    dense = set(g.frame0_q_blocks()) if frame0_dense else set()
    text = list(g.text_k_blocks()) if text_columns else []
    for i in dense:
        mask[:, :, i, :] = True
    for j in text:
        mask[:, :, :, j] = True
    cnt = mask.sum(-1).astype(np.int32)
    idx = np.full((B, H, nqb, nkb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                js = np.nonzero(mask[b, h, i])[0]
                idx[b, h, i, :len(js)] = js
    return mask, cnt, idx, ent
