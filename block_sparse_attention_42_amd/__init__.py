"""Block-sparse self-attention for video diffusion transformers on MI355X (gfx950).

Thin Python binding of ``libbsa.so`` (C ABI in ``include/bsa.h``).  The
functions keep the C names and only marshal arguments: they check tensor
shapes, dtypes and devices, allocate outputs with PyTorch when none are
given, and pass raw device pointers plus the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback.

    g = Geometry(B, H, text_len, frames, latent_h, latent_w, head_dim,
                 q_block, k_block, seq_alloc)
    qp, kp = bsa_pool_qk(q, k, g)      # or bsa_pool_blocks(q, g, g.q_block), ...(k, g, g.k_block)
    mask, cnt, idx, logw = bsa_build_mask(qp, kp, g, MaskParams(keep_ratio=0.1))
    out, lse = bsa_forward(q, k, v, g, cnt, idx, logw)

Other list producers for the same forward: bsa_cluster_importance +
bsa_select_blocks (intra-block clustering), bsa_select_top_p (top-p over
competition domains), bsa_frame_scores + bsa_classify_heads +
bsa_structured_lists (per-head frame contexts; run the forward with
launch_order="frame_runs" on these lists).
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import BsaError

__all__ = ["Geometry", "MaskParams", "BsaError", "bsa_derive", "bsa_pool_blocks", "bsa_pool_qk",
           "bsa_build_mask", "bsa_forward", "bsa_forward_ex", "bsa_cluster_importance", "bsa_select_blocks",
           "bsa_select_top_p", "DOMAINS", "HEAD_CLASSES", "LAUNCH_ORDERS", "bsa_frame_scores", "bsa_classify_heads",
           "bsa_structured_lists", "library_path"]


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

    def c(self) -> _lib.bsa_geometry:
        return _lib.bsa_geometry(self.B, self.H, self.text_len, self.frames, self.latent_h,
                                 self.latent_w, self.head_dim, self.q_block, self.k_block, 0,
                                 self.seq_alloc)


@dataclasses.dataclass(frozen=True)
class MaskParams:
    mode: str = "topk"            # "topk" or "sample"
    topk: int = 0
    keep_ratio: float = 0.1
    frame0_dense: bool = True
    text_columns: bool = False
    log_cluster: bool = False
    seed: int = 0

    def c(self) -> _lib.bsa_mask_params:
        mode = {"topk": _lib.BSA_SELECT_TOPK, "sample": _lib.BSA_SELECT_SAMPLE}[self.mode]
        return _lib.bsa_mask_params(mode, self.topk, float(self.keep_ratio), int(self.frame0_dense),
                                    int(self.text_columns), int(self.log_cluster), 0,
                                    int(self.seed) & (2 ** 64 - 1))


def library_path() -> str:
    return _lib.LIB_PATH


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BSA_DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.BSA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def bsa_derive(g: Geometry, p: Optional[MaskParams] = None) -> dict:
    """S, nqb, nkb, frame-0 query blocks, last text key block, k and E (host only)."""
    out = _lib.bsa_derived()
    pc = p.c() if p is not None else None
    _lib.check(_lib.lib().bsa_derive(ctypes.byref(g.c()), ctypes.byref(pc) if pc is not None else None,
                                     ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in _lib.bsa_derived._fields_ if f != "reserved"}


def bsa_pool_blocks(x: torch.Tensor, g: Geometry, block: int, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Per-block mean of the valid rows of x [B,H,seq_alloc,D] -> float32 [B,H,ceil(S/block),D]."""
    d = bsa_derive(g)
    nb = -(-d["S"] // block)
    _need(x, "x", (g.B, g.H, g.seq_alloc, g.head_dim))
    if out is None:
        out = torch.empty((g.B, g.H, nb, g.head_dim), dtype=torch.float32, device=x.device)
    _need(out, "out", (g.B, g.H, nb, g.head_dim), torch.float32, x.device)
    _lib.check(_lib.lib().bsa_pool_blocks(_ptr(x), _dtype_code(x), ctypes.byref(g.c()), block,
                                          _ptr(out), _stream(stream)))
    return out


def bsa_pool_qk(q: torch.Tensor, k: torch.Tensor, g: Geometry, out=None, stream=None):
    """bsa_pool_blocks of q with q_block and of k with k_block in one launch -> (q_pooled, k_pooled)."""
    d = bsa_derive(g)
    _need(q, "q", (g.B, g.H, g.seq_alloc, g.head_dim))
    _need(k, "k", (g.B, g.H, g.seq_alloc, g.head_dim), q.dtype, q.device)
    if out is None:
        out = (torch.empty((g.B, g.H, d["nqb"], g.head_dim), dtype=torch.float32, device=q.device),
               torch.empty((g.B, g.H, d["nkb"], g.head_dim), dtype=torch.float32, device=q.device))
    qp, kp = out
    _need(qp, "q_pooled", (g.B, g.H, d["nqb"], g.head_dim), torch.float32, q.device)
    _need(kp, "k_pooled", (g.B, g.H, d["nkb"], g.head_dim), torch.float32, q.device)
    _lib.check(_lib.lib().bsa_pool_qk(_ptr(q), _ptr(k), _dtype_code(q), ctypes.byref(g.c()), _ptr(qp), _ptr(kp),
                                      _stream(stream)))
    return qp, kp


def bsa_build_mask(q_pooled: torch.Tensor, k_pooled: torch.Tensor, g: Geometry, p: MaskParams,
                   want_mask: bool = True, want_logw: Optional[bool] = None, out=None, stream=None):
    """Block logits -> selection -> overrides -> compacted lists.

    Returns (mask u8 [B,H,nqb,nkb] or None, kv_cnt i32 [B,H,nqb],
    kv_idx i32 [B,H,nqb,nkb], log_w f32 [B,H,nqb,nkb] or None).  ``out`` may
    hold preallocated (mask, cnt, idx, logw) tensors.
    """
    d = bsa_derive(g, p)
    nqb, nkb = d["nqb"], d["nkb"]
    dev = q_pooled.device
    _need(q_pooled, "q_pooled", (g.B, g.H, nqb, g.head_dim), torch.float32)
    _need(k_pooled, "k_pooled", (g.B, g.H, nkb, g.head_dim), torch.float32, dev)
    if want_logw is None:
        want_logw = p.mode == "sample"
    if out is None:
        mask = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=dev) if want_mask else None
        cnt = torch.empty((g.B, g.H, nqb), dtype=torch.int32, device=dev)
        idx = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.int32, device=dev)
        logw = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.float32, device=dev) if want_logw else None
    else:
        mask, cnt, idx, logw = out
    if mask is not None:
        _need(mask, "mask", (g.B, g.H, nqb, nkb), torch.uint8, dev)
    _need(cnt, "kv_cnt", (g.B, g.H, nqb), torch.int32, dev)
    _need(idx, "kv_idx", (g.B, g.H, nqb, nkb), torch.int32, dev)
    if logw is not None:
        _need(logw, "log_w", (g.B, g.H, nqb, nkb), torch.float32, dev)
    _lib.check(_lib.lib().bsa_build_mask(_ptr(q_pooled), _ptr(k_pooled), ctypes.byref(g.c()),
                                         ctypes.byref(p.c()), _ptr(mask), _ptr(cnt), _ptr(idx),
                                         _ptr(logw), _stream(stream)))
    return mask, cnt, idx, logw


def bsa_cluster_importance(q: torch.Tensor, k_pooled: torch.Tensor, g: Geometry, n_clusters: int = 4,
                           iters: int = 3, log_cluster: bool = False, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Block importance [B,H,nqb,nkb] float32 from k-means representatives of each query block."""
    d = bsa_derive(g)
    nqb, nkb = d["nqb"], d["nkb"]
    _need(q, "q", (g.B, g.H, g.seq_alloc, g.head_dim))
    _need(k_pooled, "k_pooled", (g.B, g.H, nkb, g.head_dim), torch.float32, q.device)
    if out is None:
        out = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.float32, device=q.device)
    _need(out, "importance", (g.B, g.H, nqb, nkb), torch.float32, q.device)
    _lib.check(_lib.lib().bsa_cluster_importance(_ptr(q), _dtype_code(q), _ptr(k_pooled), ctypes.byref(g.c()),
                                                 int(n_clusters), int(iters), 1 if log_cluster else 0,
                                                 _ptr(out), _stream(stream)))
    return out


def bsa_select_blocks(importance: torch.Tensor, g: Geometry, p: MaskParams, want_mask: bool = True,
                      want_logw: Optional[bool] = None, out=None, stream=None):
    """Selection from an importance matrix -> (mask, kv_cnt, kv_idx, log_w) as bsa_build_mask."""
    d = bsa_derive(g, p)
    nqb, nkb = d["nqb"], d["nkb"]
    dev = importance.device
    _need(importance, "importance", (g.B, g.H, nqb, nkb), torch.float32)
    if want_logw is None:
        want_logw = p.mode == "sample"
    if out is None:
        mask = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=dev) if want_mask else None
        cnt = torch.empty((g.B, g.H, nqb), dtype=torch.int32, device=dev)
        idx = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.int32, device=dev)
        logw = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.float32, device=dev) if want_logw else None
    else:
        mask, cnt, idx, logw = out
    if mask is not None:
        _need(mask, "mask", (g.B, g.H, nqb, nkb), torch.uint8, dev)
    _need(cnt, "kv_cnt", (g.B, g.H, nqb), torch.int32, dev)
    _need(idx, "kv_idx", (g.B, g.H, nqb, nkb), torch.int32, dev)
    if logw is not None:
        _need(logw, "log_w", (g.B, g.H, nqb, nkb), torch.float32, dev)
    _lib.check(_lib.lib().bsa_select_blocks(_ptr(importance), ctypes.byref(g.c()), ctypes.byref(p.c()),
                                            _ptr(mask), _ptr(cnt), _ptr(idx), _ptr(logw), _stream(stream)))
    return mask, cnt, idx, logw


DOMAINS = {"row": 0, "head": 1, "split": 2, "all": 3, "eg": 4}


def bsa_select_top_p(scores: torch.Tensor, g: Geometry, domain: str = "eg", top_p: float = 0.9,
                     v_pooled: Optional[torch.Tensor] = None, value_aware: bool = False,
                     entropy_eps: float = 1e-12, frame0_dense: bool = False, text_columns: bool = False,
                     workspace: Optional[torch.Tensor] = None, want_mask: bool = True, stream=None):
    """Top-p over competition domains -> (mask u8 or None, kv_cnt, kv_idx, head entropy f64 [B,H])."""
    d = bsa_derive(g)
    nqb, nkb = d["nqb"], d["nkb"]
    dev = scores.device
    _need(scores, "scores", (g.B, g.H, nqb, nkb), torch.float32)
    if value_aware:
        _need(v_pooled, "v_pooled", (g.B, g.H, nkb, g.head_dim), torch.float32, dev)
    nbytes = ctypes.c_int64()
    _lib.check(_lib.lib().bsa_top_p_workspace_bytes(ctypes.byref(g.c()), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    mask = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=dev) if want_mask else None
    cnt = torch.empty((g.B, g.H, nqb), dtype=torch.int32, device=dev)
    idx = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.int32, device=dev)
    ent = torch.empty((g.B, g.H), dtype=torch.float64, device=dev)
    tp = _lib.bsa_topp_params(DOMAINS[domain], 1 if value_aware else 0, float(top_p), float(entropy_eps),
                              1 if frame0_dense else 0, 1 if text_columns else 0, 0)
    _lib.check(_lib.lib().bsa_select_top_p(_ptr(scores), _ptr(v_pooled) if value_aware else None,
                                           ctypes.byref(g.c()), ctypes.byref(tp), _ptr(ent), _ptr(workspace),
                                           workspace.numel(), _ptr(mask), _ptr(cnt), _ptr(idx),
                                           _stream(stream)))
    return mask, cnt, idx, ent


HEAD_CLASSES = {"full": 0, "sink": 1, "neighbor": 2, "dummy": 3}
LAUNCH_ORDERS = {"frame_position": 0, "frame_runs": 1}


def bsa_frame_scores(scores: torch.Tensor, g: Geometry, window: int, stream=None) -> torch.Tensor:
    """Frame attention scores [B,H,3] float64 (sink, neighbor, current) from P' [B,H,nqb,nkb]."""
    d = bsa_derive(g)
    _need(scores, "scores", (g.B, g.H, d["nqb"], d["nkb"]), torch.float32)
    alpha = torch.empty((g.B, g.H, 3), dtype=torch.float64, device=scores.device)
    _lib.check(_lib.lib().bsa_frame_scores(_ptr(scores), ctypes.byref(g.c()), int(window), _ptr(alpha),
                                           _stream(stream)))
    return alpha


def bsa_classify_heads(alpha, n_dummy: int):
    """Host-side head labelling (numpy or CPU tensor alpha [B,H,3]) -> numpy int32 [B,H]."""
    import numpy as np
    a = np.ascontiguousarray(alpha.cpu().numpy() if isinstance(alpha, torch.Tensor) else alpha, dtype=np.float64)
    B, H, _ = a.shape
    out = np.empty((B, H), dtype=np.int32)
    _lib.check(_lib.lib().bsa_classify_heads(a.ctypes.data, B, H, int(n_dummy), out.ctypes.data))
    return out


def bsa_structured_lists(head_class: torch.Tensor, g: Geometry, window: int, dummy_prev: bool = False,
                         block_causal: bool = False, frame0_dense: bool = False, text_columns: bool = False,
                         want_mask: bool = True, stream=None):
    """Per-head frame-context lists -> (mask u8 or None, kv_cnt i32, kv_idx i32)."""
    d = bsa_derive(g)
    nqb, nkb = d["nqb"], d["nkb"]
    dev = head_class.device
    _need(head_class, "head_class", (g.B, g.H), torch.int32)
    mask = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=dev) if want_mask else None
    cnt = torch.empty((g.B, g.H, nqb), dtype=torch.int32, device=dev)
    idx = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.int32, device=dev)
    sp = _lib.bsa_struct_params(int(window), 1 if dummy_prev else 0, 1 if block_causal else 0,
                                1 if frame0_dense else 0, 1 if text_columns else 0, 0)
    _lib.check(_lib.lib().bsa_structured_lists(_ptr(head_class), ctypes.byref(g.c()), ctypes.byref(sp), _ptr(mask),
                                               _ptr(cnt), _ptr(idx), _stream(stream)))
    return mask, cnt, idx


def bsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Geometry,
                kv_cnt: torch.Tensor, kv_idx: torch.Tensor, log_w: Optional[torch.Tensor] = None,
                softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = False, launch_order: str = "frame_position",
                stream=None, _ex: bool = False, dense_split: int = 1, workspace: Optional[torch.Tensor] = None,
                static_workspace: bool = False):
    """Attention of every query block over its listed key blocks.  Returns (out, lse or None).

    ``launch_order`` ("frame_position" or "frame_runs", see LAUNCH_ORDERS) only
    changes which work items run together; "frame_runs" calls bsa_forward_ex.
    ``dense_split`` > 1 splits each frame-0 row's list over that many work
    items and merges their partial states (bsa_forward_split, with
    ``workspace`` or a new one of bsa_forward_split_workspace_bytes bytes);
    see suggest_dense_split.  ``static_workspace`` runs the split through
    bsa_forward_split_static instead: its partial states go to the library's
    own device scratch (BSA_SPLIT_STATIC_MAX_BYTES per GPU), so the call
    allocates nothing beyond ``out`` and ``lse`` when they are not given."""
    if launch_order not in LAUNCH_ORDERS:
        raise ValueError(f"launch_order {launch_order!r} not in {sorted(LAUNCH_ORDERS)}")
    d = bsa_derive(g)
    nqb, nkb = d["nqb"], d["nkb"]
    shape = (g.B, g.H, g.seq_alloc, g.head_dim)
    _need(q, "q", shape)
    dev = q.device
    _need(k, "k", shape, q.dtype, dev)
    _need(v, "v", shape, q.dtype, dev)
    _need(kv_cnt, "kv_cnt", (g.B, g.H, nqb), torch.int32, dev)
    _need(kv_idx, "kv_idx", (g.B, g.H, nqb, nkb), torch.int32, dev)
    if log_w is not None:
        _need(log_w, "log_w", (g.B, g.H, nqb, nkb), torch.float32, dev)
    if out is None:
        out = torch.empty(shape, dtype=q.dtype, device=dev)
    _need(out, "out", shape, q.dtype, dev)
    if lse is None and want_lse:
        lse = torch.empty((g.B, g.H, g.seq_alloc), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (g.B, g.H, g.seq_alloc), torch.float32, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), ctypes.byref(g.c()), _ptr(kv_cnt), _ptr(kv_idx),
            _ptr(log_w), ctypes.c_float(softmax_scale), _ptr(out), _ptr(lse))
    if static_workspace:
        if workspace is not None:
            raise ValueError("static_workspace and workspace exclude each other")
        opt = _lib.bsa_forward_options(LAUNCH_ORDERS[launch_order])
        _lib.check(_lib.lib().bsa_forward_split_static(*args, ctypes.byref(opt), int(dense_split), _stream(stream)))
    elif dense_split != 1:
        nbytes = bsa_forward_split_workspace_bytes(g, dense_split)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
        opt = _lib.bsa_forward_options(LAUNCH_ORDERS[launch_order])
        _lib.check(_lib.lib().bsa_forward_split(*args, ctypes.byref(opt), int(dense_split), _ptr(workspace),
                                                workspace.numel(), _stream(stream)))
    elif launch_order == "frame_position" and not _ex:
        _lib.check(_lib.lib().bsa_forward(*args, _stream(stream)))
    else:
        opt = _lib.bsa_forward_options(LAUNCH_ORDERS[launch_order])
        _lib.check(_lib.lib().bsa_forward_ex(*args, ctypes.byref(opt), _stream(stream)))
    return out, lse


def bsa_forward_split_workspace_bytes(g: Geometry, dense_split: int) -> int:
    """Bytes of workspace bsa_forward_split needs (0 when nothing is split)."""
    nbytes = ctypes.c_int64(0)
    _lib.check(_lib.lib().bsa_forward_split_workspace_bytes(ctypes.byref(g.c()), int(dense_split),
                                                            ctypes.byref(nbytes)))
    return nbytes.value


def suggest_dense_split(g: Geometry, kv_cnt: torch.Tensor, simds: Optional[int] = None) -> int:
    """A key split for the frame-0 rows from the lists' lengths (reads kv_cnt back: a synchronization).

    A frame-0 row is walked by one wave; when it holds more blocks than the
    launch's average per SIMD it becomes the launch's critical path.  The
    split is that ratio, rounded, within 1..8, with at least 16 blocks a part
    (shorter parts save less than the merge launch costs; measured on MI355X:
    2 parts take the 122-block rows of a 5-frame Wan-like clip from 0.244 to
    0.220 ms, while 7-block rows get slower)."""
    d = bsa_derive(g)
    if d["frame0_first"] < 0:
        return 1
    if simds is None:
        simds = 4 * torch.cuda.get_device_properties(kv_cnt.device).multi_processor_count
    cnt = kv_cnt.reshape(g.B * g.H, -1)
    dense = cnt[:, d["frame0_first"]:d["frame0_last"] + 1]
    longest = int(dense.max().item())
    per_simd = float(cnt.sum().item()) / simds
    if per_simd <= 0:
        return 1
    return int(max(1, min(8, longest // 16, round(longest / per_simd))))


def bsa_forward_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Geometry,
                   kv_cnt: torch.Tensor, kv_idx: torch.Tensor, log_w: Optional[torch.Tensor] = None,
                   softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                   launch_order: str = "frame_position", stream=None):
    """bsa_forward through the C entry point bsa_forward_ex (options: the launch order)."""
    return bsa_forward(q, k, v, g, kv_cnt, kv_idx, log_w, softmax_scale, out, lse, want_lse, launch_order, stream,
                       _ex=True)
