"""GPU property tests: random small shapes with partial tails, k and p at their extremes,
both dtypes and every supported block size, drawn by hypothesis (derandomized, so every
run checks the same examples). Each example runs the whole path on the GPU and compares
it with the float64 oracle at the parity bars; outputs start as NaN, so an element the
kernels never write fails the comparison."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import block_sparse_attention_spa2_amd as spa2
import oracle
from gen import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (k, p): Top-p alone with a tiny p (one block per row), Top-k alone with a tiny k (one
# block), the everything-kept ends (k = 1, p = 1) and ordinary hybrids
KP = [(0.0, 1e-6), (1e-3, 0.0), (0.1, 0.3), (0.5, 0.9), (1.0, 0.0), (0.0, 1.0), (0.05, 0.5)]


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(n=st.integers(1, 1500), d=st.sampled_from([64, 128]),
       bh=st.sampled_from([(1, 1), (1, 2), (2, 1)]), bq=st.sampled_from([64, 128, 256]),
       bkv=st.sampled_from([32, 64, 128]), dtype=st.sampled_from(["bf16", "f32"]),
       kp=st.sampled_from(KP), seed=st.integers(0, 1 << 16))
def test_random_shapes(n, d, bh, bq, bkv, dtype, kp, seed):
    B, H = bh
    kf, pf = kp
    print(f"[example] B={B} H={H} N={n} D={d} bq={bq} bkv={bkv} {dtype} k={kf} p={pf} "
          f"seed={seed}", flush=True)
    inp = synth.sink_inputs(B, H, n, d, bkv, seed=seed, dtype=dtype)
    q, k, v, do = (gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v", "do"))

    # mask: bit-exact apart from blocks on the p threshold
    mask, infos = gu.oracle_masks(inp, bq, bkv, kf, pf)
    bm = spa2.mask(q, k, kf, pf, bq, bkv)
    cls = gu.classify_mask(bm.mask.cpu().numpy().astype(bool), mask, infos)
    assert cls["other"] == 0 and cls["k_band"] == 0, cls
    assert (bm.row_cnt.cpu().numpy() >= 1).all()  # k > 0 or p > 0 keeps a block per row

    # attention on the oracle's mask, into NaN-filled outputs
    obm = spa2.mask_lists(torch.from_numpy(mask.astype(np.uint8)).cuda(), q, bq, bkv)
    tdt = q.dtype
    o, lse = _nan((B, H, n, d), tdt), _nan((B, H, n), torch.float32)
    spa2.fwd(q, k, v, obm, bq, bkv, out=(o, lse))
    grads = tuple(_nan((B, H, n, d), tdt) for _ in range(3))
    spa2.bwd(q, k, v, o, lse, do, obm, bq, bkv, out=grads)
    torch.cuda.synchronize()

    qf, kf64, vf, dof = (inp.f64(x) for x in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attn_fwd(qf, kf64, vf, mask, bq, bkv)
    refs = oracle.attn_bwd(qf, kf64, vf, dof, mask, bq, bkv)
    gu.check_close("O", gu.to_f64(o), o_ref, dtype, block=bq)
    gu.check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, dtype)
    for name, got, want, blk in zip(("dQ", "dK", "dV"), grads, refs, (bq, bkv, bkv)):
        gu.check_close(name, gu.to_f64(got), want, dtype, block=blk)
