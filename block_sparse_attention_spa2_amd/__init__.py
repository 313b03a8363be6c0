"""SpargeAttention2 hot path on AMD MI355X: hybrid Top-k U Top-p block-mask prediction and
block-sparse attention forward/backward, as hand-written gfx950 kernels behind a C ABI
(include/spa2.h).

This module only marshals torch tensors (device memory, the current stream) into the C
ABI calls of the same names; every step of the computation runs in libspa2.so. There is
no CPU fallback: without the built library, the calls raise.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import Spa2Error  # noqa: F401

__all__ = ["BlockMask", "pool", "mask", "select", "mask_lists", "fwd", "bwd", "bwd_noalloc",
           "bwd_prep", "bwd_dkdv", "bwd_dq", "bwd_dq_rowterm", "error_terms",
           "mask_workspace_size", "bwd_workspace_size", "bwd_workspace", "row_term", "num_blocks",
           "Spa2Error"]


def num_blocks(n: int, b: int) -> int:
    return -(-n // b)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _desc(x: torch.Tensor, bq: int, bkv: int) -> _lib.Desc:
    if x.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor")
    B, H, N, D = x.shape
    return _lib.Desc(B, H, N, D, bq, bkv, _dtype_code(x))


def _expect(name: str, t: torch.Tensor, shape, dtype) -> None:
    """Host-side check that a tensor matches what the kernels index (shape, dtype)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _check_bm(bm: "BlockMask", q: torch.Tensor) -> None:
    B, H, N, _ = q.shape
    tm, tn = num_blocks(N, bm.bq), num_blocks(N, bm.bkv)
    _expect("mask", bm.mask, (B, H, tm, tn), torch.uint8)
    _expect("row_cnt", bm.row_cnt, (B, H, tm), torch.int32)
    _expect("row_idx", bm.row_idx, (B, H, tm, tn), torch.int32)
    _expect("col_cnt", bm.col_cnt, (B, H, tn), torch.int32)
    _expect("col_idx", bm.col_idx, (B, H, tn, tm), torch.int32)
    if bm.row_order is not None:
        _expect("row_order", bm.row_order, (B, H, tm), torch.int32)
    if bm.col_order is not None:
        _expect("col_order", bm.col_order, (B, H, tn), torch.int32)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


@dataclass
class BlockMask:
    """Block mask M-bar and its compacted lists (device tensors), see spa2_blockmask."""
    mask: torch.Tensor      # uint8 [B, H, Tm, Tn]
    row_cnt: torch.Tensor   # int32 [B, H, Tm]
    row_idx: torch.Tensor   # int32 [B, H, Tm, Tn]
    col_cnt: torch.Tensor   # int32 [B, H, Tn]
    col_idx: torch.Tensor   # int32 [B, H, Tn, Tm]
    bq: int
    bkv: int
    row_order: torch.Tensor | None = None  # int32 [B, H, Tm], scheduling order (optional)
    col_order: torch.Tensor | None = None  # int32 [B, H, Tn]

    @staticmethod
    def empty(B: int, H: int, N: int, bq: int, bkv: int, device) -> "BlockMask":
        tm, tn = num_blocks(N, bq), num_blocks(N, bkv)
        kw = dict(device=device)
        return BlockMask(
            mask=torch.empty((B, H, tm, tn), dtype=torch.uint8, **kw),
            row_cnt=torch.empty((B, H, tm), dtype=torch.int32, **kw),
            row_idx=torch.empty((B, H, tm, tn), dtype=torch.int32, **kw),
            col_cnt=torch.empty((B, H, tn), dtype=torch.int32, **kw),
            col_idx=torch.empty((B, H, tn, tm), dtype=torch.int32, **kw),
            bq=bq, bkv=bkv,
            row_order=torch.empty((B, H, tm), dtype=torch.int32, **kw),
            col_order=torch.empty((B, H, tn), dtype=torch.int32, **kw))

    def c(self) -> _lib.BlockMaskC:
        return _lib.BlockMaskC(_ptr(self.mask), _ptr(self.row_cnt), _ptr(self.row_idx),
                               _ptr(self.col_cnt), _ptr(self.col_idx),
                               _ptr(self.row_order), _ptr(self.col_order))

    def kept_fraction(self) -> float:
        return float(self.mask.float().mean())


def mask_workspace_size(q: torch.Tensor, bq: int = 128, bkv: int = 64) -> int:
    n = C.c_size_t(0)
    _lib.check("spa2_mask_workspace_size",
               _lib.lib().spa2_mask_workspace_size(C.byref(_desc(q, bq, bkv)), C.byref(n)))
    return int(n.value)


def bwd_workspace_size(q: torch.Tensor, bq: int = 128, bkv: int = 64) -> int:
    n = C.c_size_t(0)
    _lib.check("spa2_bwd_workspace_size",
               _lib.lib().spa2_bwd_workspace_size(C.byref(_desc(q, bq, bkv)), C.byref(n)))
    return int(n.value)


def bwd_workspace(q: torch.Tensor, bq: int = 128, bkv: int = 64) -> torch.Tensor:
    """A backward workspace (uint8, bwd_workspace_size bytes) on q's device."""
    return torch.empty(bwd_workspace_size(q, bq, bkv), dtype=torch.uint8, device=q.device)


def row_term(workspace: torch.Tensor, q: torch.Tensor) -> torch.Tensor:
    """The row term rowsum(dO * O) held at the start of a backward workspace: a float32
    [B, H, N] view of its first B*H*N*4 bytes."""
    B, H, N = q.shape[:3]
    if workspace.dtype != torch.uint8 or workspace.numel() < B * H * N * 4:
        raise ValueError("workspace: too small for the row term (uint8)")
    return workspace[:B * H * N * 4].view(torch.float32).view(B, H, N)


def _expect_ws(workspace: torch.Tensor, q: torch.Tensor, bq: int, bkv: int) -> None:
    need = bwd_workspace_size(q, bq, bkv)
    if workspace.dtype != torch.uint8 or workspace.numel() < need or workspace.device != q.device:
        raise ValueError(f"workspace: need {need} bytes (uint8) on {q.device}")


def pool(q: torch.Tensor, k: torch.Tensor, bq: int = 128, bkv: int = 64):
    """Block means (float64): qbar [B, H, Tm, D], kbar [B, H, Tn, D]."""
    B, H, N, D = q.shape
    _expect("k", k, q.shape, q.dtype)
    qbar = torch.empty((B, H, num_blocks(N, bq), D), dtype=torch.float64, device=q.device)
    kbar = torch.empty((B, H, num_blocks(N, bkv), D), dtype=torch.float64, device=q.device)
    _lib.check("spa2_pool", _lib.lib().spa2_pool(C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k),
                                                 _ptr(qbar), _ptr(kbar), _stream(q)))
    return qbar, kbar


def mask(q: torch.Tensor, k: torch.Tensor, k_frac: float, p_frac: float, bq: int = 128,
         bkv: int = 64, *, return_pbar: bool = False, out: BlockMask | None = None,
         workspace: torch.Tensor | None = None):
    """Hybrid Top-k U Top-p block mask from Q and K (pool -> P-bar -> select)."""
    B, H, N, D = q.shape
    _expect("k", k, q.shape, q.dtype)
    bm = out if out is not None else BlockMask.empty(B, H, N, bq, bkv, q.device)
    _check_bm(bm, q)
    ws_bytes = mask_workspace_size(q, bq, bkv)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.numel() < ws_bytes:
        raise ValueError(f"workspace: need {ws_bytes} bytes (uint8)")
    pbar = None
    if return_pbar:
        pbar = torch.empty((B, H, num_blocks(N, bq), num_blocks(N, bkv)), dtype=torch.float64,
                           device=q.device)
    _lib.check("spa2_mask", _lib.lib().spa2_mask(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), float(k_frac), float(p_frac),
        C.byref(bm.c()), _ptr(pbar), _ptr(workspace), workspace.numel(), _stream(q)))
    return (bm, pbar) if return_pbar else bm


def select(pbar: torch.Tensor, k_frac: float, p_frac: float, like: torch.Tensor, bq: int = 128,
           bkv: int = 64) -> BlockMask:
    """Hybrid selection on a given P-bar (float64 [B, H, Tm, Tn]) for inputs shaped like `like`."""
    B, H, N, D = like.shape
    _expect("pbar", pbar, (B, H, num_blocks(N, bq), num_blocks(N, bkv)), torch.float64)
    bm = BlockMask.empty(B, H, N, bq, bkv, pbar.device)
    _lib.check("spa2_select", _lib.lib().spa2_select(
        C.byref(_desc(like, bq, bkv)), _ptr(pbar), float(k_frac), float(p_frac),
        C.byref(bm.c()), _stream(pbar)))
    return bm


def mask_lists(mask_u8: torch.Tensor, like: torch.Tensor, bq: int = 128, bkv: int = 64) -> BlockMask:
    """Row and column lists for a caller-made uint8 mask [B, H, Tm, Tn]."""
    B, H, N, D = like.shape
    bm = BlockMask.empty(B, H, N, bq, bkv, mask_u8.device)
    _expect("mask", mask_u8, bm.mask.shape, torch.uint8)
    bm.mask.copy_(mask_u8)
    _lib.check("spa2_mask_lists", _lib.lib().spa2_mask_lists(
        C.byref(_desc(like, bq, bkv)), C.byref(bm.c()), _stream(mask_u8)))
    return bm


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bm: BlockMask | None,
        bq: int = 128, bkv: int = 64, *, out: tuple | None = None,
        o_f32: torch.Tensor | None = None):
    """Block-sparse attention forward -> (O, LSE). bm = None runs dense attention.

    o_f32: optional float32 [B, H, N, D] tensor that receives O before rounding; pass it
    on to bwd() so that the backward's row term uses the unrounded O."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
    B, H, N, D = q.shape
    _expect("k", k, q.shape, q.dtype)
    _expect("v", v, q.shape, q.dtype)
    if bm is not None:
        _check_bm(bm, q)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    _expect("o", o, q.shape, q.dtype)
    _expect("lse", lse, (B, H, N), torch.float32)
    if o_f32 is not None:
        _expect("o_f32", o_f32, q.shape, torch.float32)
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_fwd", _lib.lib().spa2_fwd(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), bmc, _ptr(o), _ptr(lse),
        _ptr(o_f32), _stream(q)))
    return o, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        do: torch.Tensor, bm: BlockMask | None, bq: int = 128, bkv: int = 64, *,
        out: tuple | None = None, workspace: torch.Tensor | None = None,
        o_f32: torch.Tensor | None = None):
    """Backward of fwd with the mask fixed -> (dQ, dK, dV). o_f32: the forward's unrounded
    O (optional, preferred for the row term rowsum(dO * O))."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _expect(name, t, q.shape, q.dtype)
    _expect("lse", lse, q.shape[:3], torch.float32)
    if o_f32 is not None:
        _expect("o_f32", o_f32, q.shape, torch.float32)
    if bm is not None:
        _check_bm(bm, q)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, q.shape, q.dtype)
    ws_bytes = bwd_workspace_size(q, bq, bkv)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.numel() < ws_bytes:
        raise ValueError(f"workspace: need {ws_bytes} bytes (uint8)")
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_bwd", _lib.lib().spa2_bwd(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_f32), _ptr(lse),
        _ptr(do), bmc, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
        _stream(q)))
    return dq, dk, dv


def bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                lse: torch.Tensor, do: torch.Tensor, bm: BlockMask | None, out: tuple,
                bq: int = 128, bkv: int = 64, *, o_f32: torch.Tensor | None = None):
    """bwd() through spa2_bwd_noalloc: no workspace (the library's built-in scratch holds
    the row term), outputs given by the caller in `out` = (dQ, dK, dV). Calls that overlap
    on one GPU share that scratch and must be serialised."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _expect(name, t, q.shape, q.dtype)
    _expect("lse", lse, q.shape[:3], torch.float32)
    if o_f32 is not None:
        _expect("o_f32", o_f32, q.shape, torch.float32)
    if bm is not None:
        _check_bm(bm, q)
    dq, dk, dv = out
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, q.shape, q.dtype)
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_bwd_noalloc", _lib.lib().spa2_bwd_noalloc(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_f32), _ptr(lse),
        _ptr(do), bmc, _ptr(dq), _ptr(dk), _ptr(dv), _stream(q)))
    return dq, dk, dv


def bwd_prep(o: torch.Tensor, do: torch.Tensor, dvec: torch.Tensor, bq: int = 128,
             bkv: int = 64, *, o_f32: torch.Tensor | None = None) -> torch.Tensor:
    """dvec [B, H, N] float32 = rowsum(dO * O), O = o_f32 if given (first kernel of bwd)."""
    _expect("do", do, o.shape, o.dtype)
    _expect("dvec", dvec, o.shape[:3], torch.float32)
    if o_f32 is not None:
        _expect("o_f32", o_f32, o.shape, torch.float32)
    _lib.check("spa2_bwd_prep", _lib.lib().spa2_bwd_prep(
        C.byref(_desc(o, bq, bkv)), _ptr(o), _ptr(o_f32), _ptr(do), _ptr(dvec), _stream(o)))
    return dvec


def bwd_dkdv(q, k, v, lse, do, dvec, bm: BlockMask | None, dk, dv, bq: int = 128, bkv: int = 64):
    """dK, dV pass of bwd, reading the row term dvec (float32 [B, H, N], e.g.
    row_term(workspace, q))."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
        _check_bm(bm, q)
    for name, t in (("k", k), ("v", v), ("do", do), ("dk", dk), ("dv", dv)):
        _expect(name, t, q.shape, q.dtype)
    _expect("lse", lse, q.shape[:3], torch.float32)
    _expect("dvec", dvec, q.shape[:3], torch.float32)
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_bwd_dkdv", _lib.lib().spa2_bwd_dkdv(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dvec),
        bmc, _ptr(dk), _ptr(dv), _stream(q)))
    return dk, dv


def bwd_dq(q, k, v, lse, do, workspace, bm: BlockMask | None, dq, bq: int = 128,
           bkv: int = 64):
    """dQ pass of bwd, reading the row term from the start of `workspace` (a backward
    workspace, see bwd_workspace / row_term); it writes the workspace's mean keys."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
        _check_bm(bm, q)
    for name, t in (("k", k), ("v", v), ("do", do), ("dq", dq)):
        _expect(name, t, q.shape, q.dtype)
    _expect("lse", lse, q.shape[:3], torch.float32)
    _expect_ws(workspace, q, bq, bkv)
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_bwd_dq", _lib.lib().spa2_bwd_dq(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(do),
        _ptr(workspace), workspace.numel(), bmc, _ptr(dq), _stream(q)))
    return dq


def bwd_dq_rowterm(q, k, v, o, lse, do, workspace, bm: BlockMask | None, dq, bq: int = 128,
                   bkv: int = 64, *, o_f32: torch.Tensor | None = None):
    """dQ pass that also writes the row term rowsum(dO * O) (O = o_f32 if given) at the
    start of `workspace` (row_term(workspace, q) views it); bwd runs it before the dK/dV
    pass, which reads the row term."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
        _check_bm(bm, q)
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq)):
        _expect(name, t, q.shape, q.dtype)
    if o_f32 is not None:
        _expect("o_f32", o_f32, q.shape, torch.float32)
    _expect("lse", lse, q.shape[:3], torch.float32)
    _expect_ws(workspace, q, bq, bkv)
    bmc = C.byref(bm.c()) if bm is not None else None
    _lib.check("spa2_bwd_dq_rowterm", _lib.lib().spa2_bwd_dq_rowterm(
        C.byref(_desc(q, bq, bkv)), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_f32), _ptr(lse),
        _ptr(do), bmc, _ptr(workspace), workspace.numel(), _ptr(dq), _stream(q)))
    return dq


def error_terms(o_sparse: torch.Tensor, lse_sparse: torch.Tensor, o_dense: torch.Tensor,
                lse_dense: torch.Tensor, bq: int = 128, bkv: int = 64, *, with_tau: bool = False):
    """Error decomposition of a sparse forward against the dense one, per head: float64
    [B, H, 4] = sums of |O_dense|, |O_dense - O_sparse|, |dropped-mass term|,
    |renormalisation term|; O in float32 (the o_f32 outputs of fwd). With with_tau, also
    the per-row kept dense mass tau [B, H, N] (float32)."""
    B, H = o_sparse.shape[:2]
    for name, t in (("o_sparse", o_sparse), ("o_dense", o_dense)):
        _expect(name, t, o_sparse.shape, torch.float32)
    for name, t in (("lse_sparse", lse_sparse), ("lse_dense", lse_dense)):
        _expect(name, t, o_sparse.shape[:3], torch.float32)
    terms = torch.empty((B, H, 4), dtype=torch.float64, device=o_sparse.device)
    tau = torch.empty(o_sparse.shape[:3], dtype=torch.float32, device=o_sparse.device) if with_tau else None
    _lib.check("spa2_error_terms", _lib.lib().spa2_error_terms(
        C.byref(_desc(o_sparse, bq, bkv)), _ptr(o_sparse), _ptr(lse_sparse), _ptr(o_dense),
        _ptr(lse_dense), _ptr(terms), _ptr(tau), _stream(o_sparse)))
    return (terms, tau) if with_tau else terms
