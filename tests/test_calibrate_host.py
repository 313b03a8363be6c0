"""Host logic of the Top-p calibration: the step search on known step functions (no GPU)."""
import math

from block_sparse_attention_spa2_amd.calibrate import calibrate_count


def test_uniform_steps_nearest_and_midpoint():
    count = lambda p: math.floor(p * 100)  # steps at multiples of 0.01
    p, c, (lo, hi) = calibrate_count(count, 37.4)
    assert c == 37 and abs(lo - 0.37) < 1e-12 and abs(hi - 0.38) < 1e-12
    assert abs(p - 0.375) < 1e-12 and count(p) == c
    p, c, _ = calibrate_count(count, 37.6)
    assert c == 38 and count(p) == 38


def test_tie_goes_to_the_upper_step():
    count = lambda p: math.floor(p * 10)
    p, c, _ = calibrate_count(count, 4.5)
    assert c == 5 and count(p) == 5


def test_lower_step_when_nearer():
    count = lambda p: 0 if p < 0.5 else 100
    p, c, (lo, hi) = calibrate_count(count, 30)
    assert c == 0 and lo < 1e-12
    assert abs(hi - 0.5) < 1e-12 and abs(p - 0.25) < 1e-12


def test_top_step_runs_to_one():
    count = lambda p: 0 if p < 0.9 else 7
    p, c, (lo, hi) = calibrate_count(count, 6)
    assert c == 7 and abs(lo - 0.9) < 1e-12 and hi == 1.0 and count(p) == 7
