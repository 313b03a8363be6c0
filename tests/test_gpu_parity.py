"""GPU parity: every stage of the HIP path against the float64 oracle, element by element,
at sizes the oracle finishes in seconds that span several tiles and ragged tails.

Bars: masks bit-exact except blocks whose exclusive prefix mass lies within 1e-6 of p
(counted and printed); O/dQ/dK/dV within 2e-2 relative L2 (bf16) or 1e-4 max-abs (fp32);
LSE within 1e-3 (bf16) / 1e-4 (fp32); pooled vectors exact (bf16) and P-bar within 1e-12
relative, both double precision."""
import numpy as np
import pytest
import torch

import block_sparse_attention_spa2_amd as spa2
from block_sparse_attention_spa2_amd.calibrate import calibrate
import oracle
from gen import configs, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "tiny_fp32":
        w = configs.params("tiny_fp32")
        return configs.make_inputs("tiny_fp32"), w["BQ"], w["BKV"], w["k"], w["p"]
    if name == "mid_bf16":
        w = configs.params("mid_bf16")
        return configs.make_inputs("mid_bf16"), w["BQ"], w["BKV"], w["k"], w["p"]
    spec = {
        # name: (B, H, N, D, BQ, BKV, dtype, seed, k, p)
        "ragged_bf16": (2, 2, 1000, 128, 128, 64, "bf16", 11, 0.10, 0.50),
        "ragged_bf16_d64": (1, 3, 777, 64, 64, 64, "bf16", 12, 0.15, 0.40),
        "ragged_f32_d128": (1, 2, 600, 128, 128, 64, "f32", 13, 0.20, 0.50),
        "ragged_f32_d64_bq128": (1, 2, 700, 64, 128, 64, "f32", 14, 0.20, 0.30),
        "single_block": (1, 2, 50, 64, 64, 64, "bf16", 15, 0.50, 0.50),
        "one_row": (1, 1, 1, 128, 128, 64, "bf16", 16, 0.50, 0.50),
        # block-size variants (b_q 256 and b_kv 128 run as two kernel tiles; b_kv 32 has
        # its own tile); ragged so that a second tile of the last block is partial or empty
        "bkv32_bf16": (1, 2, 1000, 128, 128, 32, "bf16", 21, 0.10, 0.50),
        "bkv128_bf16": (1, 2, 1000, 128, 128, 128, "bf16", 22, 0.15, 0.50),
        "bq256_bf16": (1, 2, 1000, 128, 256, 64, "bf16", 23, 0.10, 0.50),
        "bq256_bkv128_d64_bf16": (1, 2, 777, 64, 256, 128, "bf16", 24, 0.20, 0.50),
        "bq64_bkv32_d64_bf16": (1, 2, 700, 64, 64, 32, "bf16", 25, 0.10, 0.40),
        "bq64_bkv32_f32": (1, 2, 600, 64, 64, 32, "f32", 26, 0.15, 0.50),
        "bq256_bkv128_f32": (1, 2, 600, 128, 256, 128, "f32", 27, 0.25, 0.50),
        # 64-row query tiles at D = 128 (the forward's four-workgroup form: two and four
        # 32-key steps per mask block)
        "bq64_bf16": (1, 2, 1000, 128, 64, 64, "bf16", 28, 0.10, 0.50),
        "bq64_bkv128_bf16": (1, 2, 900, 128, 64, 128, "bf16", 29, 0.15, 0.50),
    }[name]
    B, H, N, D, BQ, BKV, dt, seed, k, p = spec
    return synth.sink_inputs(B, H, N, D, 64, seed=seed, dtype=dt), BQ, BKV, k, p


CASES = ["tiny_fp32", "ragged_bf16", "ragged_bf16_d64", "ragged_f32_d128",
         "ragged_f32_d64_bq128", "single_block", "one_row", "mid_bf16",
         "bkv32_bf16", "bkv128_bf16", "bq256_bf16", "bq256_bkv128_d64_bf16",
         "bq64_bkv32_d64_bf16", "bq64_bkv32_f32", "bq256_bkv128_f32", "bq64_bf16",
         "bq64_bkv128_bf16"]
_CACHE = {}


def ref(name):
    """Inputs, device tensors and oracle results for a case (cached per session)."""
    if name not in _CACHE:
        inp, bq, bkv, k, p = _case(name)
        print(f"[case {name}] shape={inp.q.shape} dtype={inp.dtype} bq={bq} k={k} p={p}",
              flush=True)
        mask, infos = gu.oracle_masks(inp, bq, bkv, k, p)
        q, kk, v, do = (inp.f64(x) for x in ("q", "k", "v", "do"))
        o, lse = oracle.attn_fwd(q, kk, v, mask, bq, bkv)
        dq, dk, dv = oracle.attn_bwd(q, kk, v, do, mask, bq, bkv)
        dev = {x: gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v", "do")}
        _CACHE[name] = dict(inp=inp, bq=bq, bkv=bkv, k=k, p=p, mask=mask, infos=infos, o=o,
                            lse=lse, dq=dq, dk=dk, dv=dv, dev=dev)
    return _CACHE[name]


def _oracle_bm(r):
    return spa2.mask_lists(torch.from_numpy(r["mask"].astype(np.uint8)).cuda(), r["dev"]["q"],
                           r["bq"], r["bkv"])


@pytest.mark.parametrize("name", CASES)
def test_pool(name):
    r = ref(name)
    qbar, kbar = spa2.pool(r["dev"]["q"], r["dev"]["k"], r["bq"], r["bkv"])
    B, H = r["inp"].q.shape[:2]
    gq = qbar.cpu().numpy().reshape(B * H, *qbar.shape[2:])
    gk = kbar.cpu().numpy().reshape(B * H, *kbar.shape[2:])
    for hh, info in enumerate(r["infos"]):
        if r["inp"].dtype == "bf16":  # block sums of bf16 values are exact in double
            assert np.array_equal(gq[hh], info["qbar"]) and np.array_equal(gk[hh], info["kbar"])
        else:
            np.testing.assert_allclose(gq[hh], info["qbar"], rtol=1e-15, atol=1e-16)
            np.testing.assert_allclose(gk[hh], info["kbar"], rtol=1e-15, atol=1e-16)


@pytest.mark.parametrize("name", CASES)
def test_pbar_and_mask(name):
    r = ref(name)
    bm, pbar = spa2.mask(r["dev"]["q"], r["dev"]["k"], r["k"], r["p"], r["bq"], r["bkv"],
                         return_pbar=True)
    torch.cuda.synchronize()
    B, H = r["inp"].q.shape[:2]
    gp = pbar.cpu().numpy().reshape(B * H, *pbar.shape[2:])
    for hh, info in enumerate(r["infos"]):
        np.testing.assert_allclose(gp[hh], info["pbar"], rtol=1e-12, atol=1e-300)
    gmask = bm.mask.cpu().numpy().astype(bool)
    cls = gu.classify_mask(gmask, r["mask"], r["infos"])
    print(f"[{name}] mask mismatches: {cls}")
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    # lists are the ascending compaction of the mask the kernel produced
    row_cnt, col_cnt = gu.lists_from_mask(gmask)
    assert np.array_equal(bm.row_cnt.cpu().numpy(), row_cnt)
    assert np.array_equal(bm.col_cnt.cpu().numpy(), col_cnt)
    ri, ci = bm.row_idx.cpu().numpy(), bm.col_idx.cpu().numpy()
    for b in range(B):
        for h in range(H):
            for i in range(gmask.shape[2]):
                assert list(ri[b, h, i, :row_cnt[b, h, i]]) == list(np.flatnonzero(gmask[b, h, i]))
            for j in range(gmask.shape[3]):
                assert list(ci[b, h, j, :col_cnt[b, h, j]]) == list(np.flatnonzero(gmask[b, h, :, j]))


@pytest.mark.parametrize("n,bkv,d,seed", [(40000, 64, 64, 30), (79872, 64, 64, 31),
                                          (41600, 32, 64, 28), (79936, 64, 128, 29)])
def test_mask_long_rows(n, bkv, d, seed):
    """Long rows (T_n = 625, 1248, 1300 and 1249, with ragged T_m; the selection kernel holds
    16 or 32 blocks per lane): P-bar and the mask against the oracle, lists against the
    mask."""
    inp = synth.sink_inputs(1, 1, n, d, 64, seed=seed, dtype="bf16")
    print(f"[long rows] n={n} bkv={bkv} d={d} T_n={-(-n // bkv)}", flush=True)
    k, p = 0.02, 0.3
    mask, infos = gu.oracle_masks(inp, 128, bkv, k, p)
    q, kk = gu.to_dev(inp.q), gu.to_dev(inp.k)
    bm, pbar = spa2.mask(q, kk, k, p, 128, bkv, return_pbar=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(pbar.cpu().numpy()[0, 0], infos[0]["pbar"], rtol=1e-12, atol=1e-300)
    gmask = bm.mask.cpu().numpy().astype(bool)
    cls = gu.classify_mask(gmask, mask, infos)
    print(f"[long rows] mask mismatches: {cls}")
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    row_cnt, col_cnt = gu.lists_from_mask(gmask)
    assert np.array_equal(bm.row_cnt.cpu().numpy(), row_cnt)
    assert np.array_equal(bm.col_cnt.cpu().numpy(), col_cnt)


@pytest.mark.parametrize("name", CASES)
def test_select_on_oracle_pbar(name):
    """The selection kernel alone, fed the oracle's own P-bar: the same values on both
    sides, so only the prefix-sum order can differ (p-band)."""
    r = ref(name)
    B, H = r["inp"].q.shape[:2]
    pb = np.stack([info["pbar"] for info in r["infos"]]).reshape(B, H, *r["mask"].shape[2:])
    bm = spa2.select(torch.from_numpy(pb).cuda(), r["k"], r["p"], r["dev"]["q"], r["bq"], r["bkv"])
    cls = gu.classify_mask(bm.mask.cpu().numpy().astype(bool), r["mask"], r["infos"])
    assert cls["other"] == 0 and cls["k_band"] == 0, cls


def _crafted_pbar_rows(tn, n_rows, seed):
    """P-bar rows that drive every branch of the selection kernel: all values equal, two
    levels, equal high 32 bits with different low bits, exact zeros, equal values in one
    lane (blocks j and j + 64 share a lane) and in neighbouring lanes, and random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    while len(rows) < n_rows:
        cands = [
            np.full(tn, 1.0),
            np.where(rng.random(tn) < 0.2, 3.0, 1.0),
            1.0 + rng.integers(0, 8, tn) * 2.0 ** -40,
            np.where(rng.random(tn) < 0.05, rng.random(tn) + 0.1, 0.0),
            np.resize(rng.random(64), tn),
            np.repeat(rng.random((tn + 1) // 2), 2)[:tn],
            np.r_[20.0, np.full(tn - 1, 1.0)],
            # the pages' sink row when tn = 10 (its elided tail spread evenly)
            np.r_[0.6, 0.2, 0.1, np.full(7, 0.1 / 7)] if tn == 10 else rng.random(tn),
            rng.random(tn) ** 4,
        ]
        for c in cands:
            if c.sum() == 0:
                c[rng.integers(tn)] = 1.0
            rows.append(c / c.sum())
    return np.stack(rows[:n_rows])


@pytest.mark.parametrize("n,seed", [(640, 0), (32768, 1), (5000, 2), (50000, 4), (262144, 3)])
@pytest.mark.parametrize("kf,pf", [(0.2, 0.6), (0.02, 0.3), (0.1, 0.0), (0.0, 0.6), (0.5, 0.9)])
def test_select_crafted_rows(n, seed, kf, pf):
    """The selection kernel on crafted P-bar rows (ties, equal high words, zeros) keeps
    exactly the oracle's blocks: both sides see the same values and sum the prefix in the
    same rank order, so no band is excused. N = 640 gives the pages' 10-block rows; the
    sizes cover rows of 8, 16 and 64 register rounds (T_n up to 4096, the largest)."""
    bq, bkv = 128, 64
    tm, tn = spa2.num_blocks(n, bq), spa2.num_blocks(n, bkv)
    pb = _crafted_pbar_rows(tn, tm, seed).reshape(1, 1, tm, tn)
    like = torch.empty((1, 1, n, 64), dtype=torch.bfloat16, device="cuda")
    bm = spa2.select(torch.from_numpy(pb).cuda(), kf, pf, like, bq, bkv)
    got = bm.mask.cpu().numpy().astype(bool)[0, 0]
    cnt = bm.row_cnt.cpu().numpy()[0, 0]
    idx = bm.row_idx.cpu().numpy()[0, 0]
    for i in range(tm):
        want = oracle.select_row(pb[0, 0, i], kf, pf)["kept"]
        assert list(np.flatnonzero(got[i])) == list(want), (i, kf, pf)
        assert list(idx[i, :cnt[i]]) == list(want), (i, kf, pf)


@pytest.mark.parametrize("name", CASES)
def test_fwd(name):
    r = ref(name)
    bm = _oracle_bm(r)
    o, lse = spa2.fwd(r["dev"]["q"], r["dev"]["k"], r["dev"]["v"], bm)
    st = gu.check_close("O", gu.to_f64(o), r["o"], r["inp"].dtype, block=r["bq"])
    e = gu.check_lse(lse.cpu().numpy().astype(np.float64), r["lse"], r["inp"].dtype)
    print(f"[{name}] fwd O {st} LSE {e:.2e}")


@pytest.mark.parametrize("name", CASES)
def test_bwd(name):
    r = ref(name)
    d = r["dev"]
    bm = _oracle_bm(r)
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of)
    dq, dk, dv = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm, o_f32=of)
    out = {}
    for nm, got, want, blk in (("dQ", dq, r["dq"], r["bq"]), ("dK", dk, r["dk"], r["bkv"]),
                               ("dV", dv, r["dv"], r["bkv"])):
        out[nm] = gu.check_close(nm, gu.to_f64(got), want, r["inp"].dtype, block=blk)
    print(f"[{name}] bwd {out}")


@pytest.mark.parametrize("name", ["ragged_bf16", "tiny_fp32", "ragged_f32_d64_bq128",
                                  "bq256_bkv128_d64_bf16", "bq64_bkv32_d64_bf16"])
def test_end_to_end_mask_fwd_bwd(name):
    """GPU mask -> GPU forward -> GPU backward, compared with the oracle's whole chain."""
    r = ref(name)
    d = r["dev"]
    bm = spa2.mask(d["q"], d["k"], r["k"], r["p"], r["bq"], r["bkv"])
    assert np.array_equal(bm.mask.cpu().numpy().astype(bool), r["mask"])
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of)
    dq, dk, dv = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm, o_f32=of)
    gu.check_close("O", gu.to_f64(o), r["o"], r["inp"].dtype, block=r["bq"])
    for nm, got, want, blk in (("dQ", dq, r["dq"], r["bq"]), ("dK", dk, r["dk"], r["bkv"]),
                               ("dV", dv, r["dv"], r["bkv"])):
        gu.check_close(nm, gu.to_f64(got), want, r["inp"].dtype, block=blk)


@pytest.mark.parametrize("name", ["ragged_bf16", "tiny_fp32", "ragged_bf16_d64", "bkv32_bf16",
                                  "bkv128_bf16", "bq256_bkv128_f32", "bq64_bf16",
                                  "bq64_bkv128_bf16", "bq256_bf16", "bq256_bkv128_d64_bf16"])
def test_dense_path(name):
    """mask = NULL runs every block; it equals the all-ones mask bit for bit and the
    oracle's dense attention."""
    r = ref(name)
    d = r["dev"]
    B, H, N, D = r["inp"].q.shape
    ones = torch.ones((B, H, spa2.num_blocks(N, r["bq"]), spa2.num_blocks(N, r["bkv"])),
                      dtype=torch.uint8, device="cuda")
    full = spa2.mask_lists(ones, d["q"], r["bq"], r["bkv"])
    o1, l1 = spa2.fwd(d["q"], d["k"], d["v"], None, r["bq"], r["bkv"])
    o2, l2 = spa2.fwd(d["q"], d["k"], d["v"], full)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = spa2.bwd(d["q"], d["k"], d["v"], o1, l1, d["do"], None, r["bq"], r["bkv"])
    g2 = spa2.bwd(d["q"], d["k"], d["v"], o2, l2, d["do"], full)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    q, k, v, do = (r["inp"].f64(x) for x in ("q", "k", "v", "do"))
    allm = np.ones((B, H) + tuple(ones.shape[2:]), dtype=bool)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, allm, r["bq"], r["bkv"])
    gu.check_close("O dense", gu.to_f64(o1), o_ref, r["inp"].dtype, block=r["bq"])
    gu.check_lse(l1.cpu().numpy().astype(np.float64), lse_ref, r["inp"].dtype)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, allm, r["bq"], r["bkv"])
    for nm, got, want, blk in (("dQ", g1[0], dq, r["bq"]), ("dK", g1[1], dk, r["bkv"]),
                               ("dV", g1[2], dv, r["bkv"])):
        gu.check_close(nm + " dense", gu.to_f64(got), want, r["inp"].dtype, block=blk)


@pytest.mark.parametrize("kf,pf", [(1.0, 0.0), (0.0, 1.0), (0.0, 0.3), (0.3, 0.0), (0.01, 0.9),
                                   (1e-12, 0.2)])
def test_mask_extremes(kf, pf):
    """Top-k only, Top-p only, everything kept, and tiny k (n_k = 0)."""
    inp = synth.sink_inputs(1, 2, 1000, 128, 64, seed=21, dtype="bf16")
    mask, infos = gu.oracle_masks(inp, 128, 64, kf, pf)
    bm = spa2.mask(gu.to_dev(inp.q), gu.to_dev(inp.k), kf, pf, 128, 64)
    cls = gu.classify_mask(bm.mask.cpu().numpy().astype(bool), mask, infos)
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    if kf == 1.0 or pf == 1.0:
        assert bm.mask.cpu().numpy().all() or cls["p_band"] > 0


def test_empty_rows():
    """A query block that keeps nothing gets O = 0, LSE = -inf, dQ = 0; the other blocks are
    unaffected."""
    r = ref("ragged_bf16")
    d = r["dev"]
    m = r["mask"].copy()
    m[0, 1, 3] = False
    m[1, 0, 7] = False  # the partial tail block
    bm = spa2.mask_lists(torch.from_numpy(m.astype(np.uint8)).cuda(), d["q"], r["bq"], r["bkv"])
    assert int(bm.row_cnt[0, 1, 3]) == 0
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm)
    dq, dk, dv = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm)
    q, k, v, do = (r["inp"].f64(x) for x in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, m, r["bq"], r["bkv"])
    refs = oracle.attn_bwd(q, k, v, do, m, r["bq"], r["bkv"])
    on, ln = gu.to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(on[0, 1, 384:512] == 0) and np.all(np.isneginf(ln[0, 1, 384:512]))
    assert np.all(gu.to_f64(dq)[0, 1, 384:512] == 0)
    gu.check_close("O", on, o_ref, "bf16", block=r["bq"])
    gu.check_lse(ln, lse_ref, "bf16")
    for nm, got, want, blk in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs,
                                  (r["bq"], r["bkv"], r["bkv"])):
        gu.check_close(nm, gu.to_f64(got), want, "bf16", block=blk)


@pytest.mark.parametrize("name", ["ragged_bf16", "bq64_bf16", "bkv128_bf16"])
def test_deterministic_and_in_bounds(name):
    """Two runs are bitwise identical, and nothing is written past the outputs (guard
    regions after each output stay intact; NaN-prefilled outputs are fully overwritten)."""
    r = ref(name)
    d = r["dev"]
    B, H, N, D = r["inp"].q.shape
    guard = 4096

    def guarded(shape, dtype, fill):
        n = int(np.prod(shape))
        flat = torch.full((n + guard,), fill, dtype=dtype, device="cuda")
        return flat, flat[:n].view(shape)

    outs = []
    for _ in range(2):
        bm = spa2.mask(d["q"], d["k"], r["k"], r["p"], r["bq"], r["bkv"])
        of, o = guarded((B, H, N, D), torch.bfloat16, float("nan"))
        lf, lse = guarded((B, H, N), torch.float32, float("nan"))
        spa2.fwd(d["q"], d["k"], d["v"], bm, out=(o, lse))
        grads = [guarded((B, H, N, D), torch.bfloat16, float("nan")) for _ in range(3)]
        spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm,
                 out=tuple(x[1] for x in grads))
        torch.cuda.synchronize()
        for flat, view in [(of, o), (lf, lse)] + grads:
            assert torch.isnan(flat[view.numel():]).all(), "write past the end of an output"
            assert not torch.isnan(view).any(), "output not fully written"
        outs.append([bm.mask.clone(), bm.row_cnt.clone(), bm.col_cnt.clone(), o.clone(),
                     lse.clone()] + [x[1].clone() for x in grads])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["ragged_bf16", "mid_bf16", "ragged_bf16_d64", "bkv32_bf16",
                                  "bq256_bkv128_d64_bf16", "bq64_bkv32_d64_bf16"])
def test_bwd_without_unrounded_o(name):
    """The backward also accepts only the rounded O (row term from bf16 O): the dQ pass's
    shift correction removes the offset part of the row term's rounding, so the result
    stays within the bar and close to the one with the unrounded O."""
    r = ref(name)
    d = r["dev"]
    bm = _oracle_bm(r)
    o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm)
    dq, dk, dv = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm)
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o2, lse2 = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of)
    g2 = spa2.bwd(d["q"], d["k"], d["v"], o2, lse2, d["do"], bm, o_f32=of)
    out = {}
    for nm, got, got2, want, blk in (("dQ", dq, g2[0], r["dq"], r["bq"]),
                                     ("dK", dk, g2[1], r["dk"], r["bkv"]),
                                     ("dV", dv, g2[2], r["dv"], r["bkv"])):
        e1 = gu.check_close(nm, gu.to_f64(got), want, r["inp"].dtype, block=blk)["rel_l2"]
        e2 = gu.check_close(nm, gu.to_f64(got2), want, r["inp"].dtype, block=blk)["rel_l2"]
        out[nm] = (round(e1, 5), round(e2, 5))
        assert e1 <= 2 * e2 + 1e-3, (nm, e1, e2)
    print(f"[{name}] rel L2 (bf16 O, unrounded O): {out}")


@pytest.mark.parametrize("name", ["ragged_bf16", "tiny_fp32", "ragged_f32_d64_bq128",
                                  "single_block"])
def test_staged_backward(name):
    """The staged entry points against the oracle: dQ with the row term then dK/dV (bit for
    bit what spa2_bwd does), and the three-pass form with the separate row-term pass."""
    r = ref(name)
    d = r["dev"]
    bm = _oracle_bm(r)
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
    # row term against its definition, rowsum(dO * O) in float64
    want = (d["do"].double() * of.double()).sum(-1)
    assert torch.allclose(dvec.double(), want, rtol=1e-5, atol=1e-6 * want.abs().max().item())
    ws3 = spa2.bwd_workspace(d["q"], bm.bq, bm.bkv)
    dvec3 = spa2.row_term(ws3, d["q"])
    spa2.bwd_prep(o, d["do"], dvec3, o_f32=of)
    dk3, dv3 = spa2.bwd_dkdv(d["q"], d["k"], d["v"], lse, d["do"], dvec3, bm,
                             torch.empty_like(o), torch.empty_like(o))
    dq3 = spa2.bwd_dq(d["q"], d["k"], d["v"], lse, d["do"], ws3, bm, torch.empty_like(o))
    for nm, got, want, blk in (("dQ", dq3, r["dq"], r["bq"]), ("dK", dk3, r["dk"], r["bkv"]),
                               ("dV", dv3, r["dv"], r["bkv"])):
        gu.check_close(nm, gu.to_f64(got), want, r["inp"].dtype, block=blk)


def test_o_f32_is_unrounded_o():
    """o_f32 rounds (to nearest even) to exactly the O written in the input dtype."""
    r = ref("ragged_bf16")
    d = r["dev"]
    of = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, _ = spa2.fwd(d["q"], d["k"], d["v"], _oracle_bm(r), o_f32=of)
    assert torch.equal(of.to(torch.bfloat16), o)
    gu.check_close("O f32", of.cpu().numpy().astype(np.float64), r["o"], "bf16", block=r["bq"])


def _xcd_ranges(items):
    q, r = items // 8, items % 8
    lo = 0
    for x in range(8):
        n = q + (1 if x < r else 0)
        yield lo, lo + n
        lo += n


@pytest.mark.parametrize("name", ["ragged_bf16", "mid_bf16", "tiny_fp32"])
def test_schedule_order(name):
    """row_order / col_order: each of the eight contiguous index ranges is a permutation of
    itself. Rows head by head (heads ascending), each head's rows by kept count. Columns
    kept by at least a quarter of the query blocks first, by count; then the others head by
    head, each head's by count. Outputs do not depend on the order."""
    r = ref(name)
    d = r["dev"]
    bm = spa2.mask(d["q"], d["k"], r["k"], r["p"], r["bq"], r["bkv"])
    tm, tn = bm.mask.shape[-2:]
    for cnt_t, ord_t, per_head, hoist in ((bm.row_cnt, bm.row_order, tm, 0),
                                          (bm.col_cnt, bm.col_order, tn, max(1, tm // 4))):
        cnt = cnt_t.cpu().numpy().reshape(-1)
        order = ord_t.cpu().numpy().reshape(-1)
        for lo, hi in _xcd_ranges(cnt.size):
            part = order[lo:hi]
            assert np.array_equal(np.sort(part), np.arange(lo, hi))
            c = np.minimum(cnt[part], tn if per_head == tm else tm)
            n_top = int(np.sum(c >= hoist)) if hoist else 0
            top, rest = part[:n_top], part[n_top:]
            if hoist:
                assert np.all(c[:n_top] >= hoist) and np.all(c[n_top:] < hoist)
                assert np.all(np.diff(cnt[top]) <= 0)
            head = rest // per_head
            assert np.all(np.diff(head) >= 0)
            same = np.diff(head) == 0
            assert np.all(np.diff(cnt[rest])[same] <= 0)
    natural = spa2.BlockMask(bm.mask, bm.row_cnt, bm.row_idx, bm.col_cnt, bm.col_idx,
                             bm.bq, bm.bkv)
    of1 = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    of2 = torch.empty_like(of1)
    o1, l1 = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=of1)
    o2, l2 = spa2.fwd(d["q"], d["k"], d["v"], natural, o_f32=of2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(of1, of2)
    g1 = spa2.bwd(d["q"], d["k"], d["v"], o1, l1, d["do"], bm, o_f32=of1)
    g2 = spa2.bwd(d["q"], d["k"], d["v"], o2, l2, d["do"], natural, o_f32=of2)
    for a_, b_ in zip(g1, g2):
        assert torch.equal(a_, b_)


def test_calibrate_per_head():
    """Per-head Top-p calibration on the GPU: at each returned p the oracle keeps the same
    number of blocks as the GPU, and no neighbouring step of the oracle's count is nearer
    the target."""
    r = ref("mid_bf16")
    d, inp = r["dev"], r["inp"]
    target = 0.12
    cals = calibrate(d["q"], d["k"], r["k"], target, r["bq"], r["bkv"], per_head=True)
    assert len(cals) == d["q"].shape[0] * d["q"].shape[1]
    for hh in (0, 5):
        c = cals[hh]
        pb = r["infos"][hh]["pbar"]
        cnt = lambda p: sum(len(oracle.select_row(pb[i], r["k"], p)["kept"]) for i in range(pb.shape[0]))
        want = target * pb.size
        assert cnt(c.p) == c.kept_pairs
        lo, hi = c.interval
        below, above = cnt(lo - 1e-9), cnt(hi + 1e-9)
        if lo > 1e-9:
            assert below < c.kept_pairs
        if hi < 1.0 - 1e-9:
            assert above > c.kept_pairs
        assert abs(c.kept_pairs - want) <= abs(below - want)
        assert abs(c.kept_pairs - want) <= abs(above - want)
        print(f"[mid_bf16 head {hh}] p={c.p:.9f} kept {c.kept_fraction:.4f} (target {target})")


@pytest.mark.parametrize("name", ["tiny_fp32", "ragged_bf16", "ragged_bf16_d64"])
def test_error_terms(name):
    """Error decomposition kernel: GPU sparse and dense forwards -> spa2_error_terms, against
    the oracle's sparse and dense forwards -> error_terms_head, per head."""
    r = ref(name)
    d, inp = r["dev"], r["inp"]
    bm = _oracle_bm(r)
    os32 = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    od32 = torch.empty_like(os32)
    _, ls = spa2.fwd(d["q"], d["k"], d["v"], bm, o_f32=os32)
    _, ld = spa2.fwd(d["q"], d["k"], d["v"], None, r["bq"], r["bkv"], o_f32=od32)
    terms, tau = spa2.error_terms(os32, ls, od32, ld, r["bq"], r["bkv"], with_tau=True)
    terms, tau = terms.cpu().numpy(), tau.cpu().numpy()
    q, kk, v = (inp.f64(x) for x in ("q", "k", "v"))
    full = np.ones_like(r["mask"])
    o_d, l_d = oracle.attn_fwd(q, kk, v, full, r["bq"], r["bkv"])
    rtol, ttol = (1e-4, 1e-5) if inp.dtype == "f32" else (2e-2, 2e-3)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            want, t = oracle.error_terms_head(r["o"][b, h], r["lse"][b, h], o_d[b, h], l_d[b, h])
            np.testing.assert_allclose(terms[b, h], want, rtol=rtol)
            assert np.abs(tau[b, h] - t).max() <= ttol
    print(f"[{name}] rel L1 {terms[..., 1].sum() / terms[..., 0].sum():.4f} = dropped "
          f"{terms[..., 2].sum() / terms[..., 0].sum():.4f} + renorm "
          f"{terms[..., 3].sum() / terms[..., 0].sum():.4f} (triangle)")


def test_two_streams_concurrently():
    """The library keeps no state between calls: two problems enqueued on two streams at
    once (default priority) give bit-identical results to running them one after the
    other on the default stream."""
    ra, rb = ref("ragged_bf16"), ref("bq256_bf16")

    def valid(idx, cnt):  # list entries past the count are unused
        return idx[torch.arange(idx.shape[-1], device=idx.device) < cnt[..., None]]

    def run(r):
        d = r["dev"]
        bm = spa2.mask(d["q"], d["k"], r["k"], r["p"], r["bq"], r["bkv"])
        o, lse = spa2.fwd(d["q"], d["k"], d["v"], bm)
        grads = spa2.bwd(d["q"], d["k"], d["v"], o, lse, d["do"], bm)
        return [bm.mask, bm.row_cnt, bm.col_cnt, o, lse, *grads,
                valid(bm.row_idx, bm.row_cnt), valid(bm.col_idx, bm.col_cnt)]

    serial = [run(ra), run(rb)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(s1):
        out_a = run(ra)
    with torch.cuda.stream(s2):
        out_b = run(rb)
    torch.cuda.synchronize()
    for want, got in zip(serial, (out_a, out_b)):
        for x, y in zip(want, got):
            assert torch.equal(x, y)
