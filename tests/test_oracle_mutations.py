"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a copy of an oracle function (CPU only), reruns the
pins that should expose it, and requires at least one of them to fail.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.spa2_oracle as so
from tests import test_oracle as pins


def _strict_topp(prow, k_frac, p_frac):
    sel = _orig_select(prow, k_frac, p_frac)
    # mistake: "> p stops" instead of ">= p stops"
    order, excl = sel["order"], sel["excl"]
    topp = np.sort(order[excl <= p_frac]) if p_frac > 0 else np.zeros(0, np.int64)
    kept = np.union1d(sel["topk"], topp)
    return dict(sel, topp=topp, kept=kept)


def _ties_desc(prow, k_frac, p_frac):
    # mistake: ties broken by index descending
    prow = np.asarray(prow, np.float64)
    flipped = _orig_select(prow[::-1], k_frac, p_frac)
    t = len(prow) - 1
    return dict(flipped, kept=np.sort(t - flipped["kept"]), topk=np.sort(t - flipped["topk"]),
                topp=np.sort(t - flipped["topp"]), order=t - flipped["order"])


def _floor_k(k_frac, t_n):
    return int(min(t_n, max(0, math.floor(k_frac * t_n))))  # mistake: floor


def _pool_by_b(x, b):
    x = np.asarray(x, np.float64)
    t = so.n_blocks(x.shape[0], b)
    pad = np.zeros((t * b, x.shape[1]))
    pad[: x.shape[0]] = x
    return pad.reshape(t, b, -1).sum(axis=1) / b  # mistake: divides the tail by b


def _probs_no_scale(qbar, kbar):
    s = qbar @ kbar.T  # mistake: 1/sqrt(d) dropped
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _fwd_no_renorm(q, k, v, mask, bq, bkv):
    # mistake: dense softmax weights of the kept keys, not renormalised
    n = q.shape[0]
    s = q @ k.T / math.sqrt(q.shape[1])
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    tok = np.repeat(np.repeat(mask, bq, 0)[:n], bkv, 1)[:, :n]
    o = (p * tok) @ v
    return o, np.log((np.exp(s - s.max(1, keepdims=True)) * tok).sum(1)) + s.max(1)


def _bwd_no_rowsum(q, k, v, do, mask, bq, bkv):
    # mistake: dS = P * dP, the softmax Jacobian's row-sum term dropped
    n, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(mask.shape[0]):
        lo, hi = so.block_range(n, bq, i)
        keys = so._kept_keys(n, bkv, np.flatnonzero(mask[i]))
        s = q[lo:hi] @ k[keys].T / math.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ds = p * (do[lo:hi] @ v[keys].T)
        dq[lo:hi] = ds @ k[keys] / math.sqrt(d)
        dk[keys] += ds.T @ q[lo:hi] / math.sqrt(d)
        dv[keys] += p.T @ do[lo:hi]
    return dq, dk, dv


def _bwd_transposed_dv(q, k, v, do, mask, bq, bkv):
    dq, dk, dv = _orig_bwd(q, k, v, do, mask, bq, bkv)
    return dq, dk, dv[::-1].copy()  # mistake: rows of dV scattered to the wrong keys


_orig_select = so.select_row
_orig_bwd = so.attn_bwd_head

MUTATIONS = [
    ("select_row", _strict_topp, [pins.test_worked_rows_from_pages, pins.test_sink_row_strict_rule_would_keep_two]),
    ("select_row", _ties_desc, [pins.test_ties_break_by_index, pins.test_worked_rows_from_pages]),
    ("topk_count", _floor_k, [lambda: pins.test_topk_count(0.01, 16, 1), lambda: pins.test_topk_count(0.02, 512, 11)]),
    ("pool_blocks", _pool_by_b, [pins.test_pool_closed_forms]),
    ("pooled_probs", _probs_no_scale, [pins.test_pooled_probs_closed_forms]),
    ("attn_fwd_head", _fwd_no_renorm, [lambda: pins.test_sparse_equals_token_masked_attention(1),
                                       pins.test_error_decomposition_closed_form]),
    ("attn_bwd_head", _bwd_no_rowsum, [pins.test_backward_equals_autograd, pins.test_backward_invariants]),
    ("attn_bwd_head", _bwd_transposed_dv, [pins.test_backward_equals_autograd, pins.test_backward_finite_differences]),
]


@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_pins_catch_planted_mistake(idx, monkeypatch):
    name, bad, checks = MUTATIONS[idx]
    monkeypatch.setattr(so, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    failures = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught the planted mistake in {name}"
