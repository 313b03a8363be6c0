"""Parity at the full Wan-shaped sizes, in the launch configuration the benchmark times
(same entry points, same shapes, same calibrated k/p).

Masks are compared for every head; O/LSE/dQ on sampled query blocks and dK/dV on sampled
key blocks (the first key block is the sink that nearly every row keeps), which the
oracle computes exactly block by block."""
import numpy as np
import pytest
import torch

import json
import os

import block_sparse_attention_spa2_amd as spa2
from block_sparse_attention_spa2_amd.calibrate import calibrate
import oracle
from gen import configs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wan13b():
    w = configs.params("wan13b_480p")
    print(f"[wan13b_480p] drawing inputs, p={w['p']}", flush=True)
    inp = configs.make_inputs("wan13b_480p")
    mask, infos = gu.oracle_masks(inp, w["BQ"], w["BKV"], w["k"], w["p"])
    dev = {x: gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v", "do")}
    return dict(w=w, inp=inp, mask=mask, infos=infos, dev=dev)


def test_wan13b_mask_all_heads(wan13b):
    w, d = wan13b["w"], wan13b["dev"]
    bm = spa2.mask(d["q"], d["k"], w["k"], w["p"], w["BQ"], w["BKV"])
    g = bm.mask.cpu().numpy().astype(bool)
    cls = gu.classify_mask(g, wan13b["mask"], wan13b["infos"])
    print(f"[wan13b_480p] kept {g.mean():.6f} (oracle {wan13b['mask'].mean():.6f}); {cls}")
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    assert abs(wan13b["mask"].mean() - 0.05) < 1e-4


def _oracle_lists(mask, like, bq, bkv):
    """Row/column lists and scheduling orders of the oracle's own mask, built by the
    library's list kernels (so the attention check does not depend on the GPU mask)."""
    return spa2.mask_lists(torch.from_numpy(mask.astype(np.uint8)).cuda(), like, bq, bkv)


def _rows(blocks, b, n):
    return [np.arange(i * b, min(n, (i + 1) * b)) for i in blocks]


def test_wan13b_fwd_bwd_sampled(wan13b):
    """Forward and backward on the oracle's mask at the 480p shape, in the benchmark's
    launch configuration; O, LSE and dQ on three query blocks of every head (the first,
    the partial last and a random one), dK and dV on two or three key blocks (the partial
    last, a random one, and the sink block 0 on two heads), each block held to the bar on
    its own."""
    w, d, inp = wan13b["w"], wan13b["dev"], wan13b["inp"]
    bq, bkv, N = w["BQ"], w["BKV"], w["N"]
    om = wan13b["mask"]
    bm = _oracle_lists(om, d["q"], bq, bkv)
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of)
    dq, dk, dv = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm, o_f32=of)
    on, ln = gu.to_f64(o), lse.cpu().numpy().astype(np.float64)
    dqn, dkn, dvn = gu.to_f64(dq), gu.to_f64(dk), gu.to_f64(dv)
    tm, tn = om.shape[-2:]
    rng = np.random.default_rng(0)
    worst = {}
    for h in range(w["H"]):
        m = om[0, h]
        q, k, v, do = (inp.head_f64(x, 0, h) for x in ("q", "k", "v", "do"))
        qblocks = sorted({0, tm - 1, int(rng.integers(tm))})
        kblocks = sorted({tn - 1, int(rng.integers(1, tn - 1))} | ({0} if h < 2 else set()))
        rows = sorted(set(qblocks) | {i for j in kblocks for i in np.flatnonzero(m[:, j])})
        o_ref, lse_ref = oracle.attn_fwd_head(q, k, v, m, bq, bkv, rows=qblocks)
        dq_ref, dk_ref, dv_ref = oracle.attn_bwd_head(q, k, v, do, m, bq, bkv, rows=rows)
        qseg, kseg = _rows(qblocks, bq, N), _rows(kblocks, bkv, N)
        qr, kr = np.concatenate(qseg), np.concatenate(kseg)
        qloc = np.split(np.arange(qr.size), np.cumsum([x.size for x in qseg])[:-1])
        kloc = np.split(np.arange(kr.size), np.cumsum([x.size for x in kseg])[:-1])
        for nm, got, want, idx, loc in (("O", on, o_ref, qr, qloc), ("dQ", dqn, dq_ref, qr, qloc),
                                        ("dK", dkn, dk_ref, kr, kloc), ("dV", dvn, dv_ref, kr, kloc)):
            st = gu.check_close(f"{nm} h{h}", got[0, h][idx], want[idx], "bf16", block=loc)
            worst[nm] = max(worst.get(nm, 0.0), st["block_rel_l2"])
        gu.check_lse(ln[0, h][qr], lse_ref[qr], "bf16")
    print(f"[wan13b_480p] worst block rel L2: {worst}")


def test_staged_backward_equals_bwd(wan13b):
    """spa2_bwd equals its two stages (dQ with the row term, then dK/dV) called one by one,
    bit for bit; the three-stage form with the separate row-term pass agrees to rounding."""
    w, d = wan13b["w"], wan13b["dev"]
    bm = spa2.mask(d["q"], d["k"], w["k"], w["p"], w["BQ"], w["BKV"])
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of)
    g1 = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm, o_f32=of)
    ws = spa2.bwd_workspace(d["q"], bm.bq, bm.bkv)
    dvec = spa2.row_term(ws, d["q"])
    dq = spa2.bwd_dq_rowterm(d["q"], d["k"], d["v"], o, lse, d["do"], ws, bm,
                             torch.empty_like(o), o_f32=of)
    dk, dv = spa2.bwd_dkdv(d["q"], d["k"], d["v"], lse, d["do"], dvec, bm,
                           torch.empty_like(o), torch.empty_like(o))
    for a, b in zip(g1, (dq, dk, dv)):
        assert torch.equal(a, b)
    ws3 = spa2.bwd_workspace(d["q"], bm.bq, bm.bkv)
    dvec3 = spa2.row_term(ws3, d["q"])
    spa2.bwd_prep(o, d["do"], dvec3, o_f32=of)
    scale = dvec.abs().max().item()
    assert (dvec3 - dvec).abs().max().item() <= 1e-5 * scale
    dk3, dv3 = spa2.bwd_dkdv(d["q"], d["k"], d["v"], lse, d["do"], dvec3, bm,
                             torch.empty_like(o), torch.empty_like(o))
    dq3 = spa2.bwd_dq(d["q"], d["k"], d["v"], lse, d["do"], ws3, bm, torch.empty_like(o))
    for nm, a, b in (("dQ", dq, dq3), ("dK", dk, dk3), ("dV", dv, dv3)):
        a, b = a.float(), b.float()
        rel = ((a - b).norm() / a.norm()).item()
        print(f"[wan13b_480p] {nm}: separate row-term pass vs fused, rel L2 {rel:.2e}")
        assert rel <= 1e-3, (nm, rel)


def test_wan13b_calibration_matches_oracle(wan13b):
    """GPU bisection for 5% kept pairs at k = 2% lands on the step the oracle-only script
    found (tests/golden/calibrated_p.json): same count, same flat interval."""
    d = wan13b["dev"]
    with open(os.path.join(os.path.dirname(__file__), "golden", "calibrated_p.json")) as f:
        golden = json.load(f)["wan13b_480p"]
    cal = calibrate(d["q"], d["k"], golden["k"], 0.05)
    print(f"[wan13b_480p] calibrated p={cal.p!r} kept {cal.kept_pairs} interval {cal.interval}")
    assert cal.kept_pairs == golden["kept_pairs"]
    lo, hi = golden["interval"]
    assert abs(cal.interval[0] - lo) < 1e-11 and abs(cal.interval[1] - hi) < 1e-11
    assert lo < cal.p < hi


@pytest.fixture(scope="module")
def wan14b():
    w = configs.params("wan14b_720p")
    print(f"[wan14b_720p] drawing inputs, p={w['p']}", flush=True)
    inp = configs.make_inputs("wan14b_720p")
    mask, infos = gu.oracle_masks(inp, w["BQ"], w["BKV"], w["k"], w["p"])
    dev = {x: gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v")}
    return dict(w=w, inp=inp, mask=mask, infos=infos, dev=dev)


def test_wan14b_mask_all_heads(wan14b):
    w, d = wan14b["w"], wan14b["dev"]
    bm = spa2.mask(d["q"], d["k"], w["k"], w["p"], w["BQ"], w["BKV"])
    g = bm.mask.cpu().numpy().astype(bool)
    cls = gu.classify_mask(g, wan14b["mask"], wan14b["infos"])
    print(f"[wan14b_720p] kept {g.mean():.6f} (oracle {wan14b['mask'].mean():.6f}); {cls}")
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    assert abs(wan14b["mask"].mean() - 0.05) < 1e-4
    # the lists agree with the mask
    cnt = bm.row_cnt.cpu().numpy()
    assert np.array_equal(cnt, g.sum(-1))
    ccnt = bm.col_cnt.cpu().numpy()
    assert np.array_equal(ccnt, g.sum(-2))


def test_wan14b_fwd_sampled(wan14b):
    """Forward at the 720p shape (591 x 1182 block grid, q tail 80 rows, k tail 16 keys) on
    the oracle's mask, three query blocks of every head including the partial last one,
    each block held to the bar on its own."""
    w, d, inp = wan14b["w"], wan14b["dev"], wan14b["inp"]
    bq, bkv, N = w["BQ"], w["BKV"], w["N"]
    om = wan14b["mask"]
    bm = _oracle_lists(om, d["q"], bq, bkv)
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm)
    on, ln = gu.to_f64(o), lse.cpu().numpy().astype(np.float64)
    tm = om.shape[-2]
    rng = np.random.default_rng(1)
    worst = 0.0
    for h in range(w["H"]):
        q, k, v = (inp.head_f64(x, 0, h) for x in ("q", "k", "v"))
        qblocks = sorted({0, tm - 1, int(rng.integers(tm))})
        o_ref, lse_ref = oracle.attn_fwd_head(q, k, v, om[0, h], bq, bkv, rows=qblocks)
        qseg = _rows(qblocks, bq, N)
        qr = np.concatenate(qseg)
        loc = np.split(np.arange(qr.size), np.cumsum([x.size for x in qseg])[:-1])
        st = gu.check_close(f"O h{h}", on[0, h][qr], o_ref[qr], "bf16", block=loc)
        worst = max(worst, st["block_rel_l2"])
        gu.check_lse(ln[0, h][qr], lse_ref[qr], "bf16")
    print(f"[wan14b_720p] worst block rel L2 of O: {worst:.2e}")
