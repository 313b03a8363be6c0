"""Helpers shared by the GPU parity tests: upload stored inputs, compare against the
oracle, classify mask mismatches. Inputs always come from gen/, expected values always
from oracle/; nothing here feeds GPU results into the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gen import synth

# tolerances: floating-point outputs (bf16 relative L2 and fp32 max-abs), LSE absolute
TOL = {"bf16": dict(rel_l2=2e-2, lse=1e-3), "f32": dict(max_abs=1e-4, lse=1e-4)}


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy().astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def _segments(shape, block):
    """Row segments of a [..., N, D] array: every block of `block` rows (the last one
    partial) of every leading index (head)."""
    n = shape[-2]
    lead = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    for hh in range(lead):
        for lo in range(0, n, block):
            yield hh, lo, min(n, lo + block)


def _check_one(name, got, ref, dtype):
    tol = TOL[dtype]
    stats = dict(max_abs=float(np.abs(got - ref).max()) if got.size else 0.0,
                 rel_l2=rel_l2(got, ref))
    if not np.any(ref):
        assert stats["max_abs"] <= TOL["f32"]["max_abs"], f"{name} (zero reference): {stats}"
        return stats
    if dtype == "bf16":
        assert stats["rel_l2"] <= tol["rel_l2"], f"{name}: {stats}"
    else:
        assert stats["max_abs"] <= tol["max_abs"], f"{name}: {stats}"
    return stats


def check_close(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, block=None) -> dict:
    """bf16: relative L2 bar; fp32: max-abs bar. A reference that is exactly zero (e.g. the
    gradients of a row whose single kept key takes all the weight) has no relative scale
    and is held to the fp32 max-abs bar instead.

    The bar holds for the whole tensor and, when `block` is given, for every block on its
    own, so that one wrong row or block cannot hide in a whole-tensor norm:
      block = int:  rows per block along axis -2 of a [..., N, D] array (the query block
                    size for O and dQ, the key block size for dK and dV), per head;
      block = list: explicit row-index arrays into axis 0 of a 2-D array (sampled blocks).
    The returned stats carry the worst block's relative L2 as `block_rel_l2`."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    stats = _check_one(name, got, ref, dtype)
    if block is None:
        return stats
    worst = 0.0
    if isinstance(block, int):
        g = got.reshape(-1, *got.shape[-2:])
        r = ref.reshape(-1, *ref.shape[-2:])
        segs = ((f"{name}[head {hh} rows {lo}:{hi}]", g[hh, lo:hi], r[hh, lo:hi])
                for hh, lo, hi in _segments(got.shape, block))
    else:
        segs = ((f"{name}[rows {int(ix[0])}..{int(ix[-1])}]", got[ix], ref[ix])
                for ix in block if len(ix))
    for nm, gb, rb in segs:
        st = _check_one(nm, gb, rb, dtype)
        if np.any(rb):
            worst = max(worst, st["rel_l2"])
    stats["block_rel_l2"] = worst
    return stats


def check_lse(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), "LSE: -inf rows differ"
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= TOL[dtype]["lse"], f"LSE max-abs {err}"
    return err


def oracle_masks(inp: synth.Inputs, bq: int, bkv: int, k: float, p: float):
    """Oracle mask [B, H, Tm, Tn] plus per-head info (P-bar, pooled vectors, row selections)."""
    B, H = inp.q.shape[:2]
    masks, infos = [], []
    for b in range(B):
        for h in range(H):
            m, info = oracle.block_mask_head(inp.head_f64("q", b, h), inp.head_f64("k", b, h),
                                             bq, bkv, k, p, with_info=True)
            masks.append(m)
            infos.append(info)
    tm, tn = masks[0].shape
    return np.stack(masks).reshape(B, H, tm, tn), infos


def classify_mask(gpu: np.ndarray, ref: np.ndarray, infos) -> dict:
    """Mismatched block pairs split into p-band (excused), k-band and other."""
    B, H, tm, tn = ref.shape
    g = gpu.reshape(B * H, tm, tn).astype(bool)
    r = ref.reshape(B * H, tm, tn)
    out = dict(p_band=0, k_band=0, other=0, p_band_blocks=0)
    for hh in range(B * H):
        for i in range(tm):
            sel = infos[hh]["rows"][i]
            out["p_band_blocks"] += len(sel["p_band"])
            diff = np.flatnonzero(g[hh, i] != r[hh, i])
            for j in diff:
                if j in set(sel["p_band"]):
                    out["p_band"] += 1
                elif j in set(sel["k_band"]):
                    out["k_band"] += 1
                else:
                    out["other"] += 1
    return out


def lists_from_mask(m: np.ndarray):
    """Expected row/column lists of a bool mask (ascending)."""
    B, H, tm, tn = m.shape
    row_cnt = m.sum(axis=3).astype(np.int32)
    col_cnt = m.sum(axis=2).astype(np.int32)
    return row_cnt, col_cnt
