"""Parity on the distribution-sweep workloads (480p shape: N = 32,760, D = 128, bf16,
128/64 blocks): near-uniform rows (isotropic Q, K with Q scaled by 0.1, no sink) and
sink-skewed rows (sink scale 6), the two row shapes whose Top-k and Top-p errors the pages
contrast (paper.rainbus.top summary, "核心方法"; the uniform/skewed figure of "论文图表").

Two heads of each generator (a two-head draw of the same recipe), three selections each:
Top-k alone, Top-p alone and the hybrid. Per case:
  * the GPU mask equals the oracle's except p-band blocks (counted);
  * the sparse forward on the oracle's mask matches the oracle block by block;
  * the error decomposition kernel (dense and sparse forwards of the library ->
    spa2_error_terms) matches oracle.error_terms_head on the oracle's own sparse and dense
    forwards of the whole head, and tau matches per row.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_spa2_amd as spa2
import oracle
from gen import configs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HEADS = 2
# (k, p): Top-k alone, Top-p alone, hybrid
SELECTIONS = [(0.05, 0.0), (0.0, 0.6), (0.05, 0.6)]
_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        w = configs.params(name)
        print(f"[{name}] drawing {HEADS} heads", flush=True)
        inp = configs.make_inputs(name, heads=HEADS, with_do=False)
        dev = {x: gu.to_dev(getattr(inp, x)) for x in ("q", "k", "v")}
        heads = [tuple(inp.head_f64(x, 0, h) for x in ("q", "k", "v")) for h in range(HEADS)]
        # the oracle's dense forward of each whole head (shared by the three selections)
        full = np.ones((spa2.num_blocks(w["N"], w["BQ"]), spa2.num_blocks(w["N"], w["BKV"])), bool)
        dense = [oracle.attn_fwd_head(q, k, v, full, w["BQ"], w["BKV"]) for q, k, v in heads]
        od32 = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
        _, ld = spa2.fwd(dev["q"], dev["k"], dev["v"], None, w["BQ"], w["BKV"], o_f32=od32)
        _CACHE[name] = dict(w=w, inp=inp, dev=dev, heads=heads, dense=dense, od32=od32, ld=ld)
    return _CACHE[name]


@pytest.mark.parametrize("kf,pf", SELECTIONS)
@pytest.mark.parametrize("name", ["sweep_uniform", "sweep_skewed"])
def test_sweep_mask_fwd_error_terms(name, kf, pf):
    c = _workload(name)
    w, inp, d = c["w"], c["inp"], c["dev"]
    bq, bkv = w["BQ"], w["BKV"]
    print(f"[{name}] k={kf} p={pf}", flush=True)

    mask, infos = gu.oracle_masks(inp, bq, bkv, kf, pf)
    bm = spa2.mask(d["q"], d["k"], kf, pf, bq, bkv)
    cls = gu.classify_mask(bm.mask.cpu().numpy().astype(bool), mask, infos)
    assert cls["other"] == 0 and cls["k_band"] == 0, cls

    obm = spa2.mask_lists(torch.from_numpy(mask.astype(np.uint8)).cuda(), d["q"], bq, bkv)
    os32 = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    o, ls = spa2.fwd(d["q"], d["k"], d["v"], obm, o_f32=os32)
    terms, tau = spa2.error_terms(os32, ls, c["od32"], c["ld"], bq, bkv, with_tau=True)
    on, ln = gu.to_f64(o), ls.cpu().numpy().astype(np.float64)
    terms, tau = terms.cpu().numpy(), tau.cpu().numpy()

    worst = 0.0
    rel = []
    for h, (q, k, v) in enumerate(c["heads"]):
        o_ref, lse_ref = oracle.attn_fwd_head(q, k, v, mask[0, h], bq, bkv)
        st = gu.check_close(f"O h{h}", on[0, h], o_ref, "bf16", block=bq)
        worst = max(worst, st["block_rel_l2"])
        gu.check_lse(ln[0, h], lse_ref, "bf16")
        want, t = oracle.error_terms_head(o_ref, lse_ref, *c["dense"][h])
        np.testing.assert_allclose(terms[0, h], want, rtol=2e-2)
        assert np.abs(tau[0, h] - t).max() <= 2e-3
        rel.append(want[1] / want[0])
    print(f"[{name}] k={kf} p={pf}: kept {mask.mean():.4f}, mask {cls}, worst block rel L2 of "
          f"O {worst:.2e}, oracle rel L1 vs dense per head {np.round(rel, 4).tolist()}")
