"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU. None of them retypes the oracle's own formula: each
compares it with a worked example from the pages, brute-force enumeration, a closed
form, an invariant, or an independent library routine (torch float64 attention).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gen import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ratio(text):
    """A fixture entry written as a quotient, e.g. "0.1/7"."""
    num, den = text.split("/")
    return float(num) / float(den)


def _rows():
    with open(os.path.join(GOLDEN, "worked_rows.json")) as f:
        g = json.load(f)
    rows = {}
    for name, vals in g["rows"].items():
        rows[name] = np.array([_ratio(v) if isinstance(v, str) else v for v in vals])
    return g, rows


# ------------------------------------------------------------------ worked examples
def test_worked_rows_from_pages():
    g, rows = _rows()
    for case in g["cases"]:
        sel = oracle.select_row(rows[case["row"]], case["k"], case["p"])
        assert list(sel["kept"]) == case["kept"], case["name"]
        if "p_band" in case:
            assert list(sel["p_band"]) == case["p_band"], case["name"]


def test_sink_row_strict_rule_would_keep_two():
    """The sink example separates ">= p stops" from "> p stops": with the exclusive prefix
    rule the runner-up (prefix 0.6) is excluded; a strict rule would keep it."""
    _, rows = _rows()
    sel = oracle.select_row(rows["sink10"], 0.0, 0.6)
    assert sel["excl"][1] == 0.6 and 1 not in sel["topp"]


# ------------------------------------------------------------------ Top-k count
@pytest.mark.parametrize("k,tn,nk", [(0.2, 10, 2), (0.07, 100, 7), (0.01, 16, 1), (0.02, 512, 11),
                                     (0.02, 1182, 24), (0.05, 128, 7), (1.0, 37, 37), (0.0, 9, 0),
                                     (0.10, 512, 52), (0.2, 16, 4)])
def test_topk_count(k, tn, nk):
    assert oracle.topk_count(k, tn) == nk


# ------------------------------------------------------------------ brute force selection
def _brute(prow, k, p):
    """Enumerate subsets: Top-k = the max-mass subset of size n_k; Top-p = the max-mass
    subset among the smallest sizes whose best mass reaches p."""
    tn = len(prow)
    nk = oracle.topk_count(k, tn)
    best = {}
    for s in range(tn + 1):
        cands = [(math.fsum(prow[list(c)]), c) for c in itertools.combinations(range(tn), s)]
        best[s] = max(cands)
    topk = set(best[nk][1])
    topp = set()
    if p > 0:
        for s in range(1, tn + 1):
            if best[s][0] >= p:
                topp = set(best[s][1])
                break
        else:
            topp = set(range(tn))
    return topk, topp


@pytest.mark.parametrize("seed", range(12))
def test_selection_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    tn = int(rng.integers(3, 11))
    prow = rng.dirichlet(np.full(tn, rng.choice([0.3, 1.0, 5.0])))
    for k in (0.0, 0.1, 0.25, 0.5):
        for p in (0.0, 0.3, 0.6, 0.9):
            if k == 0.0 and p == 0.0:
                continue
            sel = oracle.select_row(prow, k, p)
            if len(sel["p_band"]) or abs(np.sort(np.cumsum(np.sort(prow)[::-1]) - p)).min() < 1e-9:
                continue  # a prefix sum sits on the threshold: the rule, not rounding, is tested
            topk, topp = _brute(prow, k, p)
            assert set(sel["topk"]) == topk
            assert set(sel["topp"]) == topp
            assert set(sel["kept"]) == topk | topp


def test_ties_break_by_index():
    prow = np.full(8, 1 / 8)
    sel = oracle.select_row(prow, 0.25, 0.0)
    assert list(sel["kept"]) == [0, 1]
    prow = np.array([0.1, 0.3, 0.1, 0.3, 0.2])
    sel = oracle.select_row(prow, 0.6, 0.0)  # n_k = 3: both 0.3 then the 0.2
    assert list(sel["kept"]) == [1, 3, 4]
    assert list(sel["order"][:3]) == [1, 3, 4]


@pytest.mark.parametrize("seed", range(6))
def test_union_superset_and_monotone(seed):
    rng = np.random.default_rng(seed)
    tn = 64
    prow = rng.dirichlet(np.full(tn, 0.2))
    prev = None
    for k in (0.0, 0.02, 0.05, 0.1, 0.3, 1.0):
        for p in (0.0, 0.1, 0.5, 0.9, 1.0):
            if k == 0 and p == 0:
                continue
            sel = oracle.select_row(prow, k, p)
            kept = set(sel["kept"])
            assert set(sel["topk"]) <= kept and set(sel["topp"]) <= kept
            assert len(kept) >= oracle.topk_count(k, tn)
            assert prow[list(kept)].sum() >= min(p, prow.sum()) - 1e-12
            # grows with p at fixed k
            bigger = set(oracle.select_row(prow, k, min(1.0, p + 0.05))["kept"])
            assert kept <= bigger
            # grows with k at fixed p
            bigger = set(oracle.select_row(prow, min(1.0, k + 0.05), p)["kept"])
            assert kept <= bigger
    assert len(oracle.select_row(prow, 1.0, 0.0)["kept"]) == tn
    assert len(oracle.select_row(prow, 0.0, 1.0)["kept"]) >= tn - 1


# ------------------------------------------------------------------ pooling and P-bar
def test_pool_closed_forms():
    n, d, b = 300, 5, 64  # 5 blocks, last one partial (44 rows)
    r = np.arange(n, dtype=np.float64)
    x = np.stack([r, 2 * r + 1, np.full(n, 3.25), (-1.0) ** r, r * r], axis=1)
    got = oracle.pool_blocks(x, b)
    assert got.shape == (5, d)
    for i in range(5):
        lo, hi = i * b, min(n, (i + 1) * b)
        m = hi - lo
        assert got[i, 0] == (lo + hi - 1) / 2  # arithmetic series
        assert got[i, 1] == lo + hi  # 2 * mean + 1
        assert got[i, 2] == 3.25
        assert got[i, 3] == (0.0 if m % 2 == 0 else (1.0 if lo % 2 == 0 else -1.0) / m)
        # sum of squares lo..hi-1 = S(hi-1) - S(lo-1), S(t) = t(t+1)(2t+1)/6
        s = lambda t: t * (t + 1) * (2 * t + 1) / 6
        assert got[i, 4] == pytest.approx((s(hi - 1) - s(lo - 1)) / m, rel=1e-15)


def test_pooled_probs_closed_forms():
    d = 16
    qbar = np.zeros((3, d))
    kbar = np.zeros((2, d))
    qbar[0, 0] = 2.0
    qbar[1, 1] = -1.0
    kbar[0, 0] = 3.0
    kbar[1, 1] = 4.0
    pb = oracle.pooled_probs(qbar, kbar)
    # two blocks: P_0 = logistic(s_0 - s_1), s = q.k / sqrt(d)
    s = np.array([[6.0, 0.0], [0.0, -4.0], [0.0, 0.0]]) / 4.0
    for i in range(3):
        assert pb[i, 0] == pytest.approx(1 / (1 + math.exp(s[i, 1] - s[i, 0])), rel=1e-15)
        assert pb[i].sum() == pytest.approx(1.0, abs=1e-15)
    assert pb[2, 0] == 0.5
    # equal key blocks give a uniform row
    pb = oracle.pooled_probs(np.ones((1, 4)), np.ones((7, 4)))
    assert np.all(pb == pb[0, 0]) and pb[0, 0] == pytest.approx(1 / 7, rel=1e-15)


def test_block_mask_end_to_end_small():
    """Pool -> P-bar -> select on hand-made blocks: query block 0 aligned with key block 2,
    query block 1 aligned with key block 0."""
    d, bq, bkv = 8, 4, 2
    e = np.eye(d)
    q = np.concatenate([np.tile(5 * e[2], (4, 1)), np.tile(5 * e[0], (4, 1))])
    k = np.concatenate([np.tile(e[0], (2, 1)), np.tile(e[1], (2, 1)), np.tile(e[2], (2, 1)),
                        np.tile(e[3], (2, 1))])
    m = oracle.block_mask_head(q, k, bq, bkv, 0.25, 0.0)
    assert m.tolist() == [[False, False, True, False], [True, False, False, False]]
    m = oracle.block_mask_head(q, k, bq, bkv, 1.0, 0.0)
    assert m.all()


# ------------------------------------------------------------------ attention forward
def _token_mask(mask, n, bq, bkv):
    rows = np.repeat(mask, bq, axis=0)[:n]
    return np.repeat(rows, bkv, axis=1)[:, :n]


def _torch_attn(q, k, v, tok_mask=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    am = None if tok_mask is None else torch.from_numpy(tok_mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], attn_mask=am)[0, 0].numpy()


def _case(seed, n=300, d=16, bq=64, bkv=32, k=0.2, p=0.5):
    inp = synth.sink_inputs(1, 1, n, d, bkv, seed=seed, dtype="f32", sink_scale=2.0)
    q, kk, v, do = (inp.head_f64(x, 0, 0) for x in ("q", "k", "v", "do"))
    mask = oracle.block_mask_head(q, kk, bq, bkv, k, p)
    return q, kk, v, do, mask


def test_dense_equals_library_attention():
    q, k, v, _, _ = _case(7)
    tm, tn = oracle.n_blocks(300, 64), oracle.n_blocks(300, 32)
    full = np.ones((tm, tn), dtype=bool)
    o, lse = oracle.attn_fwd_head(q, k, v, full, 64, 32)
    ref = _torch_attn(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    s = torch.from_numpy(q @ k.T / 4.0)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)
    # k = 100% through the whole mask pipeline is dense too
    m = oracle.block_mask_head(q, k, 64, 32, 1.0, 0.0)
    assert m.all()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sparse_equals_token_masked_attention(seed):
    n, bq, bkv = 300, 64, 32  # ragged tails: 300 = 4*64 + 44 = 9*32 + 12
    q, k, v, _, mask = _case(seed, n=n, bq=bq, bkv=bkv)
    assert 0 < mask.mean() < 1
    o, lse = oracle.attn_fwd_head(q, k, v, mask, bq, bkv)
    tok = _token_mask(mask, n, bq, bkv)
    ref = _torch_attn(q, k, v, tok)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    s = q @ k.T / 4.0
    s[~tok] = -np.inf
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(s), 1).numpy(), atol=1e-12)


def test_error_decomposition_closed_form():
    """O_dense - O_sparse = (p*(1-m) + (1 - 1/tau)(p*m)) V with tau the kept dense mass,
    and LSE_dense - LSE_sparse = -ln tau (the renormalisation term of the decomposition)."""
    n, bq, bkv = 300, 64, 32
    q, k, v, _, mask = _case(11, n=n, bq=bq, bkv=bkv)
    tok = _token_mask(mask, n, bq, bkv).astype(np.float64)
    s = torch.from_numpy(q @ k.T / 4.0)
    pd = torch.softmax(s, dim=1).numpy()
    tau = (pd * tok).sum(axis=1, keepdims=True)
    e = (pd * (1 - tok) + (1 - 1 / tau) * (pd * tok)) @ v
    o_dense, lse_dense = oracle.attn_fwd_head(q, k, v, np.ones_like(mask), bq, bkv)
    o_sp, lse_sp = oracle.attn_fwd_head(q, k, v, mask, bq, bkv)
    np.testing.assert_allclose(o_dense - o_sp, e, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_dense - lse_sp, -np.log(tau[:, 0]), rtol=0, atol=1e-12)
    # each output row is a convex combination of its kept value rows
    np.testing.assert_allclose(o_sp, (pd * tok) @ v / tau, rtol=0, atol=1e-12)


def test_error_terms_against_definition():
    """error_terms_head, which works from the two forwards' outputs only, equals the sums of
    the decomposition's terms built from the dense weights p and the token mask m; an empty
    row (tau = 0) puts its whole dense output into the dropped term."""
    n, bq, bkv = 300, 64, 32
    q, k, v, _, mask = _case(12, n=n, bq=bq, bkv=bkv)
    mask[2] = False  # rows 128..191 keep nothing
    tok = _token_mask(mask, n, bq, bkv).astype(np.float64)
    pd = torch.softmax(torch.from_numpy(q @ k.T / 4.0), dim=1).numpy()
    tau = (pd * tok).sum(axis=1, keepdims=True)
    dropped = (pd * (1 - tok)) @ v
    with np.errstate(divide="ignore", invalid="ignore"):
        renorm = np.where(tau > 0, (1 - 1 / tau) * ((pd * tok) @ v), 0.0)
    o_dense, lse_dense = oracle.attn_fwd_head(q, k, v, np.ones_like(mask), bq, bkv)
    o_sp, lse_sp = oracle.attn_fwd_head(q, k, v, mask, bq, bkv)
    sums, t = oracle.error_terms_head(o_sp, lse_sp, o_dense, lse_dense)
    np.testing.assert_allclose(t, tau[:, 0], rtol=1e-12, atol=0)
    want = [np.abs(o_dense).sum(), np.abs(o_dense - o_sp).sum(), np.abs(dropped).sum(),
            np.abs(renorm).sum()]
    np.testing.assert_allclose(sums, want, rtol=1e-11)
    assert np.allclose(np.abs(dropped[128:192]).sum(), np.abs(o_dense[128:192]).sum(), rtol=1e-12)


def test_empty_row_convention():
    q, k, v, do, mask = _case(5)
    mask[1] = False
    o, lse = oracle.attn_fwd_head(q, k, v, mask, 64, 32)
    assert np.all(o[64:128] == 0) and np.all(np.isneginf(lse[64:128]))
    dq, _, _ = oracle.attn_bwd_head(q, k, v, do, mask, 64, 32)
    assert np.all(dq[64:128] == 0)


# ------------------------------------------------------------------ attention backward
def test_backward_equals_autograd():
    n, bq, bkv = 300, 64, 32
    q, k, v, do, mask = _case(21, n=n, bq=bq, bkv=bkv)
    tok = torch.from_numpy(_token_mask(mask, n, bq, bkv))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None],
                                                         tv[None, None], attn_mask=tok)[0, 0]
    o.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.attn_bwd_head(q, k, v, do, mask, bq, bkv)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_backward_finite_differences():
    n, d, bq, bkv = 40, 4, 16, 8
    inp = synth.sink_inputs(1, 1, n, d, bkv, seed=3, dtype="f32")
    q, k, v, do = (inp.head_f64(x, 0, 0) for x in ("q", "k", "v", "do"))
    mask = oracle.block_mask_head(q, k, bq, bkv, 0.3, 0.4)
    assert 0 < mask.mean() < 1
    dq, dk, dv = oracle.attn_bwd_head(q, k, v, do, mask, bq, bkv)

    def loss(qq, kk, vv):
        return float((oracle.attn_fwd_head(qq, kk, vv, mask, bq, bkv)[0] * do).sum())

    h = 1e-6
    rng = np.random.default_rng(0)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            r, c = int(rng.integers(n)), int(rng.integers(d))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][r, c] += h
            up = loss(*args)
            args[which][r, c] -= 2 * h
            dn = loss(*args)
            assert (up - dn) / (2 * h) == pytest.approx(grad[r, c], abs=1e-7)


def test_backward_invariants():
    n, bq, bkv = 300, 64, 32
    q, k, v, do, mask = _case(31, n=n, bq=bq, bkv=bkv)
    dq, dk, dv = oracle.attn_bwd_head(q, k, v, do, mask, bq, bkv)
    # the softmax Jacobian annihilates constants: keys' gradients sum to zero
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # every row's weights sum to one: value gradients sum to the total output gradient
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-11)


# ------------------------------------------------------------------ generator storage
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # exact ties
    ours = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
