"""Named synthetic workloads (shapes, block sizes, k/p, generator recipe, seed).

The Top-p fraction of the two Wan-shaped workloads is tuned so that 5.0% of block pairs
are kept (95% block sparsity). The tuned values are stored in
tests/golden/calibrated_p.json, written by tests/golden/make_calibration.py, which runs
the float64 oracle's mask only (bisection on p at fixed k).
"""
from __future__ import annotations

import json
import os

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
_CALIB = os.path.join(_HERE, "..", "tests", "golden", "calibrated_p.json")

WORKLOADS = {
    # tiny fp32 parity case: 16 x 16 block grid, sink on key block 0
    "tiny_fp32": dict(B=1, H=2, N=1024, D=64, BQ=64, BKV=64, dtype="f32", k=0.20, p=0.60,
                      gen="sink", n_sink=1, sink_scale=3.0, seed=1),
    # mid bf16: 8 x 32 x 32 latent grid, smooth low-rank positional Q/K, two sink blocks
    "mid_bf16": dict(B=1, H=12, N=8192, grid=(8, 32, 32), D=128, BQ=128, BKV=64,
                     dtype="bf16", k=0.05, p=0.50, gen="fourier", n_sink=2, sink_scale=3.0,
                     seed=2),
    # Wan2.1-1.3B-shaped 480p: 21 x 30 x 52 latent tokens, 256 x 512 block grid
    "wan13b_480p": dict(B=1, H=12, N=32760, grid=(21, 30, 52), D=128, BQ=128, BKV=64,
                        dtype="bf16", k=0.02, p="calibrated", gen="sink", n_sink=1,
                        sink_scale=3.0, seed=3, target_kept=0.05),
    # Wan2.1-14B-shaped 720p: 21 x 45 x 80 latent tokens, 591 x 1182 block grid
    "wan14b_720p": dict(B=1, H=40, N=75600, grid=(21, 45, 80), D=128, BQ=128, BKV=64,
                        dtype="bf16", k=0.02, p="calibrated", gen="sink", n_sink=1,
                        sink_scale=3.0, seed=4, target_kept=0.05, with_do=False),
    # distribution sweep at the 480p shape: near-uniform rows vs sink-skewed rows
    "sweep_uniform": dict(B=1, H=12, N=32760, D=128, BQ=128, BKV=64, dtype="bf16",
                          gen="uniform", q_temp=0.1, seed=51),
    "sweep_skewed": dict(B=1, H=12, N=32760, D=128, BQ=128, BKV=64, dtype="bf16",
                         gen="sink", n_sink=1, sink_scale=6.0, seed=52),
}

SWEEP_K = (0.01, 0.03, 0.05, 0.10)
SWEEP_P = (0.30, 0.60, 0.90)


def calibrated_p(name: str) -> float:
    with open(_CALIB) as f:
        return float(json.load(f)[name]["p"])


def params(name: str) -> dict:
    """Workload parameters with the calibrated p filled in."""
    w = dict(WORKLOADS[name])
    if w.get("p") == "calibrated":
        w["p"] = calibrated_p(name)
    return w


def make_inputs(name: str, *, heads: int | None = None, n: int | None = None,
                with_do: bool | None = None) -> synth.Inputs:
    """Draw the workload's inputs. `heads` and `n` shrink the draw for quick cases (a
    different draw, not a slice of the full one)."""
    w = WORKLOADS[name]
    H = heads if heads is not None else w["H"]
    N = n if n is not None else w["N"]
    do = w.get("with_do", True) if with_do is None else with_do
    if w["gen"] == "sink":
        return synth.sink_inputs(w["B"], H, N, w["D"], w["BKV"], seed=w["seed"],
                                 dtype=w["dtype"], n_sink=w["n_sink"],
                                 sink_scale=w["sink_scale"], with_do=do)
    if w["gen"] == "uniform":
        return synth.uniform_inputs(w["B"], H, N, w["D"], w["BKV"], seed=w["seed"],
                                    dtype=w["dtype"], q_temp=w["q_temp"], with_do=do)
    if w["gen"] == "fourier":
        assert n is None, "the fourier recipe's N is fixed by its grid"
        return synth.fourier_inputs(w["B"], H, w["grid"], w["D"], w["BQ"], w["BKV"],
                                    seed=w["seed"], dtype=w["dtype"], n_sink=w["n_sink"],
                                    sink_scale=w["sink_scale"], with_do=do)
    raise ValueError(w["gen"])
