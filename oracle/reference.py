"""Plain CPU oracle of block-sparse video attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module.  It shares no code with the HIP library: it is
written from the pages and from the plain definitions below, slowly and in
the order the pages state the steps.

Sources (page title; section):

* "Attention matrix view: make only frame-0 query rows dense" (frame-0 page):
  section 1 token packing ``[text] + [frame0] + ...``; section 2 frame-0
  rows use every K/V token; section 4 block-level override formula; section
  6 top-k mask first, frame-0 rows overwritten after; section 7 always keep
  text blocks.
* "Competition Domains Matter ... (EG-Sparse)" (EG-Sparse page): centroid
  setup with the cluster-size-weighted softmax (its Eq. 2, whose body is
  lost in the text: read here as ``P'_ij ∝ n_j exp(q_i·k_j / sqrt(d))``);
  the minimum one-key-per-row safeguard.
* "AB-Attention: accurate block-sparse attention for video diffusion"
  (AB-Attention page): TL;DR and flowchart -- exact attention on selected
  blocks, blocks sampled in proportion to importance and reweighted by the
  inverse inclusion probability, small blocks gathered into full tiles.

Precision.  Every step whose floating-point result decides an integer (the
block mask, the selected lists, a Bernoulli draw) is computed in float32 with
each operation's rounding and order written out, because the GPU takes the
same decisions in float32 and the two must agree bit for bit.  The
attention output (compared under a tolerance) is computed in float64.

Pins.  Every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (closed forms from the pages, library routines,
brute force, invariants).  No function is "parity unpinned".
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# Geometry (frame-0 page, sections 1 and 4; section 7 for text blocks)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Geometry:
    B: int
    H: int
    text_len: int
    frames: int
    latent_h: int
    latent_w: int
    head_dim: int
    q_block: int
    k_block: int
    seq_alloc: int

    @property
    def S(self) -> int:
        # sequence = [text tokens] + [frame0 tokens] + ... (frame-0 page, sec. 1)
        return self.text_len + self.frames * self.latent_h * self.latent_w

    @property
    def nqb(self) -> int:
        return -(-self.S // self.q_block)

    @property
    def nkb(self) -> int:
        return -(-self.S // self.k_block)

    def q_block_tokens(self) -> np.ndarray:
        """Valid tokens of each query block (the last one may be short)."""
        i = np.arange(self.nqb)
        return np.minimum(self.q_block, self.S - i * self.q_block)

    def k_block_tokens(self) -> np.ndarray:
        """n_j: valid tokens of each key block (the cluster size of block j)."""
        j = np.arange(self.nkb)
        return np.minimum(self.k_block, self.S - j * self.k_block)

    def frame0_q_blocks(self) -> range:
        """Query blocks overlapping frame 0 (frame-0 page, section 4 formula)."""
        if self.frames == 0 or self.latent_h * self.latent_w == 0:
            return range(0)
        visual_start = self.text_len
        tokens_per_frame = self.latent_h * self.latent_w
        frame0_q_start = visual_start
        frame0_q_end = visual_start + tokens_per_frame
        first_q_block = frame0_q_start // self.q_block
        last_q_block = (frame0_q_end - 1) // self.q_block
        return range(first_q_block, last_q_block + 1)

    def text_k_blocks(self) -> range:
        """Key blocks overlapping the text tokens [0, text_len) (frame-0 page, sec. 7)."""
        if self.text_len <= 0:
            return range(0)
        return range(0, (self.text_len - 1) // self.k_block + 1)


# ---------------------------------------------------------------------------
# Block summaries: mean of the valid tokens of each block (AB-Attention page,
# TL;DR "coarse summaries"; EG-Sparse page, centroids of clusters of n tokens)
# ---------------------------------------------------------------------------

def pool_blocks(x: np.ndarray, S: int, block: int) -> np.ndarray:
    """Mean of each block's valid rows, float32, fixed order.

    ``x``: [B, H, seq_alloc, D] (float32 values; bfloat16 inputs widened
    exactly).  For block i with n_i = min(block, S - i*block) valid rows and
    every channel d: ``acc = 0; for t in rows of the block, ascending:
    acc = fl32(acc + x[t, d])``; then ``fl32(acc / n_i)``.  Rows >= S are
    never read.
    """
    x = np.asarray(x, dtype=F32)
    B, H, _, D = x.shape
    nb = -(-S // block)
    out = np.empty((B, H, nb, D), dtype=F32)
    for i in range(nb):
        lo = i * block
        n = min(block, S - lo)
        acc = np.zeros((B, H, D), dtype=F32)
        for t in range(lo, lo + n):
            acc = acc + x[:, :, t, :]          # float32 + float32 -> float32
        out[:, :, i, :] = acc / F32(n)        # one IEEE division
    return out


# ---------------------------------------------------------------------------
# Block logits (EG-Sparse page, Eq. 2: P' is a softmax over key clusters of
# the centroid dot products scaled by 1/sqrt(d), weighted by cluster size)
# ---------------------------------------------------------------------------

def score_scale(D: int) -> np.float32:
    """1/sqrt(D) evaluated in double and rounded once to float32."""
    return F32(1.0 / math.sqrt(float(D)))


def log_cluster_table(n_max: int) -> np.ndarray:
    """fp32(ln n) for n = 0..n_max (entry 0 unused), evaluated in double."""
    t = np.zeros(n_max + 1, dtype=F32)
    for n in range(1, n_max + 1):
        t[n] = F32(math.log(n))
    return t


def block_logits(qp: np.ndarray, kp: np.ndarray, n_k: np.ndarray,
                 log_cluster: bool) -> np.ndarray:
    """z[b,h,i,j] = (q̄_i·k̄_j)/sqrt(D) (+ ln n_j), float32 with written-out order.

    ``acc = 0; for d = 0..D-1: acc = fl32(acc + fl32(q̄_d * k̄_d))`` (no fused
    multiply-add), ``z = fl32(acc * fp32(1/sqrt(D)))``, then, with the
    cluster-size term on, ``z = fl32(z + fp32(ln n_j))``.  A zero result is
    stored as +0.  The softmax itself is monotone along a row, so ranking z
    ranks P'; it is only evaluated where probabilities are needed
    (importance sampling).
    """
    qp = np.asarray(qp, dtype=F32)
    kp = np.asarray(kp, dtype=F32)
    B, H, nqb, D = qp.shape
    nkb = kp.shape[2]
    acc = np.zeros((B, H, nqb, nkb), dtype=F32)
    for d in range(D):
        prod = qp[:, :, :, d][:, :, :, None] * kp[:, :, :, d][:, :, None, :]
        acc = acc + prod
    z = acc * score_scale(D)
    if log_cluster:
        table = log_cluster_table(int(n_k.max()))
        z = z + table[np.asarray(n_k)][None, None, None, :]
    z[z == 0] = F32(0.0)
    return z.astype(F32)


# ---------------------------------------------------------------------------
# Per-row top-k (frame-0 page, section 6: the sparse top-k mask is built
# first, with the same ratio for every frame)
# ---------------------------------------------------------------------------

def topk_count(nkb: int, topk: int, keep_ratio: float) -> int:
    """k = topk if given, else ceil(keep_ratio * nkb) in double, clamped to [1, nkb]."""
    if topk > 0:
        return min(topk, nkb)
    return max(1, min(nkb, math.ceil(keep_ratio * nkb)))


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """Boolean mask of the k largest entries of each row of z (last axis).

    Order: larger z first; equal z -> lower block index first.
    """
    order = np.argsort(-z, axis=-1, kind="stable")
    sel = np.zeros(z.shape, dtype=bool)
    np.put_along_axis(sel, order[..., :k], True, axis=-1)
    return sel


# ---------------------------------------------------------------------------
# Importance sampling (AB-Attention page, TL;DR item 2 and flowchart: blocks
# sampled with probability by importance, reweighted by the inverse
# inclusion probability)
# ---------------------------------------------------------------------------

# e^t for t <= 0 by Cody and Waite's argument reduction (W. J. Cody and
# W. Waite, "Software Manual for the Elementary Functions", 1980): t = n*ln2
# + x with n = round(t*log2 e) and ln2 split in a high part with trailing
# zero bits (so n*ln2_hi is exact) and a low part; e^x for |x| <= ln2/2 by
# the degree-7 Taylor polynomial in Horner form; the result r * 2^n.  Every
# operation is one float32 rounding, no fused multiply-add.
EXP_LOG2E = F32(1.4426950408889634)
EXP_LN2_HI = F32(0.693145751953125)          # 0x3F317200: 15 significant bits
EXP_LN2_LO = F32(0.6931471805599453 - 0.693145751953125)
EXP_TAYLOR = [F32(1.0 / math.factorial(k)) for k in range(8)]   # 1/k!, k = 0..7
EXP_FLUSH = F32(-125.0)


def exp_spec(t: np.ndarray) -> np.ndarray:
    """float32 e^t for t <= 0 (t*log2 e < -125 gives 0)."""
    t = np.asarray(t, dtype=F32)
    y = t * EXP_LOG2E
    flush = y < EXP_FLUSH
    t = np.where(flush, F32(0.0), t).astype(F32)      # flushed lanes: result forced to 0 below
    y = np.where(flush, F32(0.0), y).astype(F32)
    n = np.floor(y + F32(0.5)).astype(F32)
    x = t - n * EXP_LN2_HI
    x = x - n * EXP_LN2_LO
    r = np.full(t.shape, EXP_TAYLOR[7], dtype=F32)
    for kk in range(6, -1, -1):
        r = r * x
        r = r + EXP_TAYLOR[kk]
    out = np.ldexp(r, n.astype(np.int32)).astype(F32)
    return np.where(flush, F32(0.0), out).astype(F32)


# Philox4x64-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
# "Parallel random numbers: as easy as 1, 2, 3", SC 2011): a counter-based
# generator; ten rounds of two 64x64->128-bit multiplies on a 4-word
# counter, with a 2-word key bumped by Weyl constants between rounds.
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """One Philox4x64-10 block: 4 output words for a 4-word counter, 2-word key."""
    x0, x1, x2, x3 = (int(c) & _MASK64 for c in counter)
    k0, k1 = (int(c) & _MASK64 for c in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & _MASK64
            k1 = (k1 + PHILOX_W1) & _MASK64
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> 64, p0 & _MASK64
        hi1, lo1 = p1 >> 64, p1 & _MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def sample_uniforms(seed: int, row_id: int, nkb: int) -> np.ndarray:
    """u_j in [0, 1) with 24-bit resolution for one mask row.

    Block j of row ``row_id = (b*H + h)*nqb + i`` takes word ``j % 4`` of
    Philox4x64-10 at counter ``(row_id, j // 4, 0, 0)`` with key ``(seed, 0)``;
    ``u = (word >> 40) * 2^-24``.
    """
    u = np.empty(nkb, dtype=F32)
    for g in range(-(-nkb // 4)):
        words = philox4x64_10((row_id, g, 0, 0), (seed, 0))
        for w in range(4):
            j = 4 * g + w
            if j < nkb:
                u[j] = F32((words[w] >> 40) * 2.0 ** -24)
    return u


def fold_sum(x: np.ndarray) -> np.float32:
    """float32 sum of a row in a fixed tree order.

    Pad with zeros to the next power of two n, then repeatedly add the upper
    half onto the lower half (``x[k] = fl32(x[k] + x[k + n/2])``) until one
    value remains.
    """
    x = np.asarray(x, dtype=F32)
    n = 1
    while n < x.shape[-1]:
        n *= 2
    a = np.zeros(x.shape[:-1] + (n,), dtype=F32)
    a[..., :x.shape[-1]] = x
    while n > 1:
        n //= 2
        a = a[..., :n] + a[..., n:2 * n]
    return a[..., 0]


def inclusion_probabilities(z_row: np.ndarray, expected: np.float32):
    """Inclusion probabilities pi_j proportional to softmax(z), capped at 1.

    pi_j = min(1, c * e_j) with e_j = exp_spec(z_j - max z) and c chosen so
    that sum_j pi_j = E (``expected``).  Water-filling: the set C of capped
    blocks starts empty; repeat ``sigma = fold_sum(e_j for j not in C)``,
    ``c = fl32((E - |C|) / sigma)`` (0 if the numerator or sigma is <= 0),
    ``C += {j : fl32(c * e_j) >= 1}`` until C stops growing.  If E >= nkb
    every pi is 1.  Returns (pi, e), float32.
    """
    z_row = np.asarray(z_row, dtype=F32)
    nkb = z_row.shape[0]
    m = z_row.max()
    e = exp_spec(z_row - m)
    if float(expected) >= nkb:
        return np.ones(nkb, dtype=F32), e
    capped = np.zeros(nkb, dtype=bool)
    while True:
        sigma = fold_sum(np.where(capped, F32(0.0), e))
        num = F32(expected) - F32(capped.sum())
        c = F32(num / sigma) if (num > 0 and sigma > 0) else F32(0.0)
        grown = capped | (c * e >= F32(1.0))
        if np.array_equal(grown, capped):
            break
        capped = grown
    pi = np.where(capped, F32(1.0), c * e).astype(F32)
    return pi, e


def select_sample(z_row: np.ndarray, expected: np.float32, seed: int, row_id: int):
    """One importance-sampled mask row: (selected bool, log-weight float32 by j).

    Block j is kept iff u_j < pi_j (Poisson sampling: each block at most once,
    inclusion probability exactly pi_j).  A kept block's additive log-weight
    is -ln pi_j, so its keys enter the softmax with weight 1/pi_j, the
    inverse inclusion probability.  If nothing is kept, the block with the
    largest z (lowest index among equals) is kept with weight 0 (EG-Sparse
    page, minimum one-key-per-row safeguard).
    """
    pi, _ = inclusion_probabilities(z_row, expected)
    u = sample_uniforms(seed, row_id, z_row.shape[0])
    sel = u < pi
    logw = np.zeros(z_row.shape[0], dtype=F32)
    if not sel.any():
        j = int(np.argmax(z_row))          # first maximum = lowest index
        sel[j] = True
        return sel, logw
    w = -np.log(pi[sel].astype(np.float64))
    logw[sel] = w.astype(F32)
    logw[sel & (pi >= F32(1.0))] = F32(0.0)
    return sel, logw


# ---------------------------------------------------------------------------
# Whole mask: selection, then overrides, then the compacted per-row lists
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MaskParams:
    mode: str = "topk"           # "topk" | "sample"
    topk: int = 0
    keep_ratio: float = 0.1
    frame0_dense: bool = True
    text_columns: bool = False
    log_cluster: bool = False
    seed: int = 0


def build_mask(qp: np.ndarray, kp: np.ndarray, g: Geometry, p: MaskParams,
               rows=None):
    """Block mask and compacted per-row lists.

    Returns ``mask`` bool [B,H,nqb,nkb], ``cnt`` int32 [B,H,nqb], ``idx``
    int32 [B,H,nqb,nkb] (ascending selected j in the first cnt slots, -1
    after), ``logw`` float32 [B,H,nqb,nkb] (log-weight of list slot p, 0
    after cnt).  ``rows``, if given, is a list of (b, h, i) to compute; other
    rows are left empty (cnt 0).

    Steps, in the pages' order: sparse selection on every row (top-k or
    sampling); then query blocks overlapping frame 0 select every key block
    with weight 0 (frame-0 page, sections 4 and 6); then, with text columns
    on, every row also keeps the key blocks overlapping the text with
    weight 0 (frame-0 page, section 7), without reducing its top-k budget.
    """
    B, H, nqb, nkb = g.B, g.H, g.nqb, g.nkb
    mask = np.zeros((B, H, nqb, nkb), dtype=bool)
    wj = np.zeros((B, H, nqb, nkb), dtype=F32)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nqb)]
    rows = list(rows)
    dense_rows = set(g.frame0_q_blocks()) if p.frame0_dense else set()
    text_cols = list(g.text_k_blocks()) if p.text_columns else []
    n_k = g.k_block_tokens()

    # block logits only for the requested rows, grouped by (b, h)
    by_head = {}
    for (b, h, i) in rows:
        by_head.setdefault((b, h), []).append(i)
    k = topk_count(nkb, p.topk, p.keep_ratio)
    expected = F32(p.keep_ratio * nkb)
    for (b, h), ilist in by_head.items():
        ii = np.array(sorted(set(ilist)))
        z = block_logits(qp[b:b + 1, h:h + 1, ii], kp[b:b + 1, h:h + 1], n_k, p.log_cluster)[0, 0]
        for r, i in enumerate(ii):
            if i in dense_rows:
                mask[b, h, i, :] = True
                continue
            if p.mode == "topk":
                mask[b, h, i] = select_topk(z[r], k)
            elif p.mode == "sample":
                row_id = (b * H + h) * nqb + int(i)
                sel, lw = select_sample(z[r], expected, p.seed, row_id)
                mask[b, h, i] = sel
                wj[b, h, i] = lw
            else:
                raise ValueError(p.mode)
            for j in text_cols:
                mask[b, h, i, j] = True
                wj[b, h, i, j] = F32(0.0)

    cnt = np.zeros((B, H, nqb), dtype=np.int32)
    idx = np.full((B, H, nqb, nkb), -1, dtype=np.int32)
    logw = np.zeros((B, H, nqb, nkb), dtype=F32)
    for (b, h, i) in rows:
        js = np.nonzero(mask[b, h, i])[0]
        cnt[b, h, i] = len(js)
        idx[b, h, i, :len(js)] = js
        logw[b, h, i, :len(js)] = wj[b, h, i, js]
    return mask, cnt, idx, logw


# ---------------------------------------------------------------------------
# Attention on the selected blocks, expanded to tokens (frame-0 page, section
# 2 token-level definition; AB-Attention page, reweighted attention)
# ---------------------------------------------------------------------------

def forward_scale(D: int, softmax_scale: float = 0.0) -> float:
    """The softmax scale the forward uses: the given one, else fp32(1/sqrt(D))."""
    return float(F32(softmax_scale)) if softmax_scale else float(score_scale(D))


def attention_head(q, k, v, g: Geometry, cnt_h, idx_h, logw_h,
                   q_blocks=None, softmax_scale: float = 0.0):
    """Masked softmax attention of one (b, h), float64, expanded to tokens.

    ``q, k, v``: [seq_alloc, D] values.  ``cnt_h, idx_h, logw_h``: the
    row lists of this head.  For each query token t of query block i, every
    key token u with block j = u // k_block in row i's list and u < S gets
    logit ``(q_t·k_u) * scale + logw_ij``; every other key is excluded (-inf).
    ``O_t = softmax(logits) @ V``, ``LSE_t = ln sum exp(logits)``.  Rows t >= S
    and rows with an empty list give O = 0, LSE = -inf.  Returns O
    [n, D] and LSE [n] for the tokens of ``q_blocks`` (default: all).
    """
    S, bq, bk = g.S, g.q_block, g.k_block
    scale = forward_scale(g.head_dim, softmax_scale)
    if q_blocks is None:
        q_blocks = range(g.nqb)
    K = np.asarray(k[:S], dtype=np.float64)
    V = np.asarray(v[:S], dtype=np.float64)
    key_block = np.arange(S) // bk
    outs, lses = [], []
    for i in q_blocks:
        lo, hi = i * bq, min((i + 1) * bq, g.seq_alloc)
        Q = np.asarray(q[lo:hi], dtype=np.float64)
        O = np.zeros((hi - lo, g.head_dim))
        L = np.full(hi - lo, -np.inf)
        c = int(cnt_h[i])
        if c > 0:
            bias_j = np.full(g.nkb, -np.inf)
            bias_j[idx_h[i, :c]] = np.asarray(logw_h[i, :c], dtype=np.float64)
            bias = bias_j[key_block]                      # block mask expanded to tokens
            logits = (Q @ K.T) * scale + bias[None, :]
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            s = e.sum(axis=1, keepdims=True)
            O = (e / s) @ V
            L = (m + np.log(s))[:, 0]
            valid = np.arange(lo, hi) < S
            O[~valid] = 0.0
            L[~valid] = -np.inf
        outs.append(O)
        lses.append(L)
    return np.concatenate(outs, axis=0), np.concatenate(lses)


def attention_head_gathered(q, k, v, g: Geometry, cnt_h, idx_h, logw_h,
                            q_blocks=None, softmax_scale: float = 0.0):
    """attention_head with the key tokens of each row's listed blocks gathered
    first, so its cost follows the selected blocks rather than the whole
    sequence (AB-Attention page, TL;DR: attention is computed only on the
    selected blocks).  The excluded keys of attention_head contribute exp(-inf)
    = 0 there, so both give the same float64 softmax up to summation order.
    Used as a CPU speed reference; the parity oracle is attention_head."""
    S, bq, bk = g.S, g.q_block, g.k_block
    scale = forward_scale(g.head_dim, softmax_scale)
    if q_blocks is None:
        q_blocks = range(g.nqb)
    K = np.asarray(k[:S], dtype=np.float64)
    V = np.asarray(v[:S], dtype=np.float64)
    outs, lses = [], []
    for i in q_blocks:
        lo, hi = i * bq, min((i + 1) * bq, g.seq_alloc)
        O = np.zeros((hi - lo, g.head_dim))
        L = np.full(hi - lo, -np.inf)
        c = int(cnt_h[i])
        if c > 0:
            blocks = np.asarray(idx_h[i, :c])
            toks = (blocks[:, None] * bk + np.arange(bk)[None, :]).ravel()
            bias = np.repeat(np.asarray(logw_h[i, :c], dtype=np.float64), bk)
            keep = toks < S
            toks, bias = toks[keep], bias[keep]
            Q = np.asarray(q[lo:hi], dtype=np.float64)
            logits = (Q @ K[toks].T) * scale + bias[None, :]
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            s = e.sum(axis=1, keepdims=True)
            O = (e / s) @ V[toks]
            L = (m + np.log(s))[:, 0]
            valid = np.arange(lo, hi) < S
            O[~valid] = 0.0
            L[~valid] = -np.inf
        outs.append(O)
        lses.append(L)
    return np.concatenate(outs, axis=0), np.concatenate(lses)


def attention(q, k, v, g: Geometry, cnt, idx, logw, softmax_scale: float = 0.0):
    """attention_head over every (b, h): O [B,H,seq_alloc,D], LSE [B,H,seq_alloc]."""
    O = np.zeros((g.B, g.H, g.seq_alloc, g.head_dim))
    L = np.full((g.B, g.H, g.seq_alloc), -np.inf)
    for b in range(g.B):
        for h in range(g.H):
            o, l = attention_head(q[b, h], k[b, h], v[b, h], g, cnt[b, h], idx[b, h],
                                  logw[b, h], softmax_scale=softmax_scale)
            n = o.shape[0]
            O[b, h, :n] = o
            L[b, h, :n] = l
    return O, L
