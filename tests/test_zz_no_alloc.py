"""spa2_bwd_noalloc (the backward for callers that cannot allocate: its row term lives in
a scratch array built into the library) against spa2_bwd with a caller workspace, through
the C ABI: bit for bit on consecutive calls, the second one smaller than the first, then
the first again (the scratch keeps the previous call's contents), with and without the
unrounded O, sparse and dense; and against the oracle at the parity bars."""
import numpy as np
import pytest
import torch

import block_sparse_attention_spa2_amd as spa2
import oracle
from gen import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (B, H, N, D, BQ, BKV, dtype, seed, k, p)
BIG = (2, 3, 1500, 128, 128, 64, "bf16", 31, 0.10, 0.50)
SMALL = (1, 1, 300, 64, 64, 32, "bf16", 32, 0.20, 0.40)


def _problem(spec):
    B, H, N, D, BQ, BKV, dt, seed, k, p = spec
    inp = synth.sink_inputs(B, H, N, D, 64, seed=seed, dtype=dt)
    dev = {x: gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v", "do")}
    bm = spa2.mask(dev["q"], dev["k"], k, p, BQ, BKV)
    return inp, dev, bm, BQ, BKV


def _run_both(dev, bm, bq, bkv, with_o32):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    of = torch.empty(q.shape, dtype=torch.float32, device="cuda") if with_o32 else None
    o, lse = spa2.fwd(q, k, v, bm, bq, bkv, o_f32=of)
    want = spa2.bwd(q, k, v, o, lse, do, bm, bq, bkv, o_f32=of)
    out = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    got = spa2.bwd_noalloc(q, k, v, o, lse, do, bm, out, bq, bkv, o_f32=of)
    torch.cuda.synchronize()
    return want, got


def _check(name, want, got):
    for nm, a, b in zip(("dQ", "dK", "dV"), want, got):
        assert torch.equal(a, b), f"{name}: {nm} differs from spa2_bwd"


def test_noalloc_equals_bwd_big_then_small_then_big():
    big, small = _problem(BIG), _problem(SMALL)
    for step, (spec, (inp, dev, bm, bq, bkv)) in enumerate(((BIG, big), (SMALL, small),
                                                             (BIG, big))):
        print(f"[noalloc call {step}] shape={tuple(dev['q'].shape)} bq={bq} bkv={bkv}", flush=True)
        for with_o32 in (False, True):
            want, got = _run_both(dev, bm, bq, bkv, with_o32)
            _check(f"call {step} o_f32={with_o32}", want, got)
        # against the oracle on the mask the GPU produced (its equality with the oracle's
        # mask is the mask tests' business)
        m = bm.mask.cpu().numpy().astype(bool)
        qf, kf, vf, dof = (inp.f64(x) for x in ("q", "k", "v", "do"))
        refs = oracle.attn_bwd(qf, kf, vf, dof, m, bq, bkv)
        for nm, g, r, blk in zip(("dQ", "dK", "dV"), got, refs, (bq, bkv, bkv)):
            gu.check_close(f"{nm} call {step}", gu.to_f64(g), r, "bf16", block=blk)


def test_noalloc_dense_small():
    inp, dev, _, bq, bkv = _problem(SMALL)
    want, got = _run_both(dev, None, bq, bkv, False)
    _check("dense", want, got)
