"""Tune Top-p for the Wan-shaped workloads so that 5.0% of block pairs are kept.

Runs the float64 oracle only (pooling, P-bar and per-row selection) on the workload's
seeded inputs, at the workload's fixed k. The kept count is a non-decreasing step
function of p; the script bisects for the step nearest the target and then stores the
midpoint of that step's flat interval, so that no row's prefix sum lies close to p.
Writes tests/golden/calibrated_p.json.

Usage: python tests/golden/make_calibration.py [workload ...]
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))

import oracle  # noqa: E402
from gen import configs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "calibrated_p.json")


def kept_count(pbars, k, p):
    total = 0
    for pb in pbars:
        for i in range(pb.shape[0]):
            total += len(oracle.select_row(pb[i], k, p)["kept"])
    return total


def bisect_first(pbars, k, pred, lo=0.0, hi=1.0, steps=48):
    """Smallest p in (lo, hi] with pred(kept_count(p)) true, to 2^-steps."""
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if pred(kept_count(pbars, k, mid)):
            hi = mid
        else:
            lo = mid
    return hi


def calibrate(name: str) -> dict:
    w = configs.WORKLOADS[name]
    inp = configs.make_inputs(name, with_do=False)
    pbars = []
    for b in range(w["B"]):
        for h in range(w["H"]):
            qbar = oracle.pool_blocks(inp.head_f64("q", b, h), w["BQ"])
            kbar = oracle.pool_blocks(inp.head_f64("k", b, h), w["BKV"])
            pbars.append(oracle.pooled_probs(qbar, kbar))
    pairs = sum(pb.size for pb in pbars)
    target = w["target_kept"] * pairs
    k = w["k"]
    # boundary where the count first reaches the target
    b1 = bisect_first(pbars, k, lambda c: c >= target)
    c_hi = kept_count(pbars, k, b1)
    c_lo = kept_count(pbars, k, b1 - 1e-12)
    if abs(c_lo - target) < abs(c_hi - target):
        # the step below: [b0, b1)
        b0 = bisect_first(pbars, k, lambda c: c >= c_lo, 0.0, b1)
        lo_edge, hi_edge, count = b0, b1, c_lo
    else:
        b2 = bisect_first(pbars, k, lambda c: c > c_hi, b1, 1.0)
        lo_edge, hi_edge, count = b1, b2, c_hi
    p = 0.5 * (lo_edge + hi_edge)
    assert kept_count(pbars, k, p) == count
    return dict(p=p, k=k, kept_pairs=int(count), pairs=int(pairs),
                kept_fraction=count / pairs, interval=[lo_edge, hi_edge],
                margin=0.5 * (hi_edge - lo_edge))


def main(names):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in names:
        res = calibrate(name)
        print(name, res, flush=True)
        data[name] = res
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or ["wan13b_480p", "wan14b_720p"])
