"""Automatic Top-p calibration to a target block sparsity.

The pages name the hand tuning of k% and p% as a weakness of the method and suggest
choosing them automatically (paper.rainbus.top summary, "局限与改进"). This module does the
plain version of that: for a fixed k%, it finds a p whose hybrid mask keeps a target
fraction of block pairs, over all heads at once or head by head.

P-bar is computed once on the GPU (spa2_mask); each probe is one spa2_select on it. The
kept count is a non-decreasing step function of p (a larger p only extends each row's
Top-p prefix), so bisection finds the step whose count is nearest the target, and the
returned p is the midpoint of that step's flat interval: no row's exclusive prefix mass
lies near it, so rounding differences in P-bar cannot change the mask. The host side is
only the bisection; the selection itself runs in the library.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import torch

from . import mask, select


@dataclass
class Calibration:
    p: float            # midpoint of the chosen step's flat interval
    kept_pairs: int     # kept block pairs at p
    pairs: int          # all block pairs of the calibrated heads
    interval: tuple     # (lo, hi): every p in [lo, hi) keeps exactly kept_pairs
    k: float

    @property
    def kept_fraction(self) -> float:
        return self.kept_pairs / self.pairs


def _first(count: Callable[[float], int], pred: Callable[[int], bool], lo: float, hi: float,
           steps: int) -> float:
    """Smallest p in (lo, hi] with pred(count(p)), to (hi - lo) 2^-steps; pred must be
    monotone (false then true) in p."""
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if pred(count(mid)):
            hi = mid
        else:
            lo = mid
    return hi


def calibrate_count(count: Callable[[float], int], target: float, steps: int = 48):
    """The step of a non-decreasing step function count(p) on [0, 1] nearest to `target`:
    returns (p, count, (lo, hi)) with p the midpoint of the step's flat interval. The step
    at or above the target wins ties."""
    b1 = _first(count, lambda c: c >= target, 0.0, 1.0, steps)
    c_hi = count(b1)
    eps = 2.0 ** -steps
    c_lo = count(max(b1 - eps, 0.0))
    if c_lo < c_hi and abs(c_lo - target) < abs(c_hi - target):
        b0 = _first(count, lambda c: c >= c_lo, 0.0, b1, steps)
        lo, hi, c = b0, b1, c_lo
    else:
        b2 = _first(count, lambda c: c > c_hi, b1, 1.0, steps)
        lo, hi, c = b1, b2, c_hi
    return 0.5 * (lo + hi), c, (lo, hi)


def calibrate(q: torch.Tensor, k: torch.Tensor, k_frac: float, target_fraction: float,
              bq: int = 128, bkv: int = 64, *, per_head: bool = False, steps: int = 48):
    """p such that the hybrid mask at (k_frac, p) keeps `target_fraction` of the block pairs
    (the nearest achievable count). per_head=True calibrates every (batch, head) on its own
    and returns a list of Calibration in (b, h) order; otherwise one Calibration for all."""
    if not 0.0 < target_fraction <= 1.0:
        raise ValueError("target_fraction must lie in (0, 1]")
    B, H = q.shape[:2]
    _, pbar = mask(q, k, k_frac, 1.0, bq, bkv, return_pbar=True)
    groups = [(slice(b, b + 1), slice(h, h + 1)) for b in range(B) for h in range(H)] \
        if per_head else [(slice(0, B), slice(0, H))]
    out = []
    for sb, sh in groups:
        pb = pbar[sb, sh]
        like = q[sb, sh]
        pairs = pb.numel()

        def count(p, pb=pb, like=like):
            return int(select(pb, k_frac, p, like, bq, bkv).row_cnt.sum().item())

        p, c, (lo, hi) = calibrate_count(count, target_fraction * pairs, steps)
        out.append(Calibration(p=p, kept_pairs=c, pairs=pairs, interval=(lo, hi), k=k_frac))
    return out if per_head else out[0]
