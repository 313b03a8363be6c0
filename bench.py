#!/usr/bin/env python3
"""Benchmark of the SpargeAttention2 hot path on one MI355X.

One step = the whole path on one batch: block mask (pool, P-bar, Top-k U Top-p, lists),
block-sparse forward, block-sparse backward (preprocess, dK/dV pass, dQ pass). Default
workload: the Wan2.1-1.3B-shaped 480p attention (B=1, H=12, N=32760, D=128, bf16,
b_q=128, b_kv=64, k=2%, p tuned to 95% block sparsity) on seeded synthetic inputs.

Prints ONE JSON line on stdout; progress goes to stderr.
  value        effective TFLOP/s of the whole step: (4 d A + 10 d A) / step time, where A
               is the kept query x key area in real tokens (forward 4dA, backward 10dA)
  roofline     the dominant kernel's algorithmic FLOPs per launch / its event-timed
               average duration, against the 2.5 PFLOP/s dense bf16 MFMA peak
  cpu_baseline the float64 oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn fwd+bwd ms & eff. TFLOPS at N=32760, 95% sparsity; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


KERNEL_SOURCES = {
    "fwd": ("fwd.hip", "common.h", "kernels.h"),
    "bwd_dkdv": ("bwd.hip", "common.h", "kernels.h"),
    "bwd_dq_rowterm": ("bwd.hip", "common.h", "kernels.h"),
}
TRAFFIC_PROFILES = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest(kernel):
    """SHA-256 of a kernel's HIP sources with comments and blank space removed, plus the
    compiler flags: a recorded counter reading applies only while this is unchanged."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "block_sparse_attention_spa2_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(name.encode())
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    from block_sparse_attention_spa2_amd import build
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None when there is
    no record for this kernel and workload or the kernel changed since it was taken."""
    path = TRAFFIC_PROFILES.format(workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if not line.startswith("RECORD "):
                continue
            rec = json.loads(line[len("RECORD "):])
            if rec["kernel"] == kernel and rec["workload"] == workload:
                if rec["source_sha256"] != kernel_digest(kernel):
                    return None
                return rec["bytes_per_launch"]
    return None


def copy_calibration():
    """A plain device-to-device copy of a known size (512 MiB, three times), run under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to scale those counters to bytes."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n * 2, "launches": 3}), flush=True)


def kept_area(mask, n, bq, bkv):
    """Sum over kept (i, j) of rows(i) * cols(j), in real tokens. mask: bool [B,H,Tm,Tn]."""
    import numpy as np
    tm, tn = mask.shape[-2:]
    rows = np.minimum(n, (np.arange(tm) + 1) * bq) - np.arange(tm) * bq
    cols = np.minimum(n, (np.arange(tn) + 1) * bkv) - np.arange(tn) * bkv
    return int(np.einsum("bhij,i,j->", mask.astype(np.int64), rows, cols))


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs), q))


def _dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def copy_bandwidth(reps=5):
    """GB/s of a plain 512 MiB device-to-device copy (read + write bytes), for context."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n * 2 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b_480p",
                    help="wan13b_480p (default, mask+fwd+bwd), mid_bf16, tiny_fp32, "
                         "wan14b_720p (mask+fwd: no dO)")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle parity check")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--dense-reps", type=int, default=2)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="Top-k / Top-p / hybrid sweep on near-uniform and skewed rows")
    ap.add_argument("--bq", type=int, default=None,
                    help="query block size (64, 128, 256); p is recalibrated on the GPU to the "
                         "workload's target kept fraction")
    ap.add_argument("--bkv", type=int, default=None, help="key block size (32, 64, 128)")
    ap.add_argument("--o-f32", action="store_true",
                    help="the forward also writes the unrounded O and the backward's row term "
                         "reads it (default: the row term uses the bf16 O)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        run_sweep(args)
        return

    import numpy as np
    import torch

    import block_sparse_attention_spa2_amd as spa2
    from gen import configs

    torch.cuda.set_device(0)
    w = configs.params(args.workload)
    B, H, N, D, bq, bkv = w["B"], w["H"], w["N"], w["D"], w["BQ"], w["BKV"]
    kf, pf = w["k"], w["p"]
    t0 = time.time()
    inp = configs.make_inputs(args.workload)
    train = inp.do is not None
    log(f"[bench] inputs {args.workload} B={B} H={H} N={N} D={D} drawn in {time.time() - t0:.1f}s")

    q, k, v = (_dev(getattr(inp, n)) for n in ("q", "k", "v"))
    do = _dev(inp.do) if train else None
    calibrated = None
    if (args.bq or bq) != bq or (args.bkv or bkv) != bkv:
        # block-size variant: same inputs and k, p re-tuned to the same kept fraction
        from block_sparse_attention_spa2_amd.calibrate import calibrate
        target = configs.WORKLOADS[args.workload].get("target_kept")
        if target is None:
            sys.exit(f"--bq/--bkv need a workload with a target kept fraction; "
                     f"{args.workload} has none")
        bq, bkv = args.bq or bq, args.bkv or bkv
        cal = calibrate(q, k, kf, target, bq, bkv)
        pf = cal.p
        w = dict(w, BQ=bq, BKV=bkv, p=pf)
        calibrated = {"target_kept": target, "kept_pairs": cal.kept_pairs, "pairs": cal.pairs,
                      "interval": list(cal.interval)}
        log(f"[bench] block sizes {bq}/{bkv}: p calibrated to {pf} ({cal.kept_fraction:.6f} kept)")
    bm = spa2.BlockMask.empty(B, H, N, bq, bkv, q.device)
    mws = torch.empty(spa2.mask_workspace_size(q, bq, bkv), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if train:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = spa2.bwd_workspace(q, bq, bkv)  # row term, then the dQ pass's mean keys
        dvec = spa2.row_term(bws, q)
        # the unrounded O is an optional extra output for the backward's row term; the dQ
        # pass's shift correction makes the bf16 O enough at this shape (sampled dQ 0.21%
        # vs 0.20% relative L2), so the step writes it only with --o-f32
        o_f32 = torch.empty(q.shape, dtype=torch.float32, device="cuda") if args.o_f32 else None
    else:
        dq = dk = dv = bws = dvec = o_f32 = None

    def stage_mask():
        spa2.mask(q, k, kf, pf, bq, bkv, out=bm, workspace=mws)

    def stage_fwd():
        spa2.fwd(q, k, v, bm, out=(o, lse), o_f32=o_f32)

    def stage_dq():  # dQ and the row term rowsum(dO * O), which the dK/dV pass reads
        spa2.bwd_dq_rowterm(q, k, v, o, lse, do, bws, bm, dq, o_f32=o_f32)

    def stage_dkdv():
        spa2.bwd_dkdv(q, k, v, lse, do, dvec, bm, dk, dv)

    stages = [("mask", stage_mask), ("fwd", stage_fwd)]
    if train:
        stages += [("bwd_dq_rowterm", stage_dq), ("bwd_dkdv", stage_dkdv)]

    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    gmask = bm.mask.cpu().numpy().astype(bool)
    area = kept_area(gmask, N, bq, bkv)
    kept_frac = float(gmask.mean())
    flops_fwd = 4.0 * D * area
    flops_bwd = 10.0 * D * area if train else 0.0

    parity = None
    if not args.no_check:
        parity = check_parity(inp, w, gmask, o, lse, dq, dk, dv)
        log(f"[bench] parity {parity}")

    # ---- timed region: exactly `steps` steps, events around every stage
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        evs[s][0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            evs[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    samples = {name: [evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]
               for i, (name, _) in enumerate(stages)}
    per_stage = {name: float(np.mean(x)) for name, x in samples.items()}
    spread = {name: {"median": round(_pct(x, 50), 4), "p10": round(_pct(x, 10), 4),
                     "p90": round(_pct(x, 90), 4)} for name, x in samples.items()}
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step; stages {per_stage}")

    # ---- one cold run per stage: a 1 GiB scratch write evicts L2 and the Infinity Cache
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = {}
    for name, fn in stages:
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        cold[name] = round(e0.elapsed_time(e1), 4)
    del scratch

    # ---- dense baseline: the same kernels with every block kept (mask = NULL)
    dense = {}
    if args.dense_reps > 0:
        od, ld = torch.empty_like(q), torch.empty_like(lse)
        spa2.fwd(q, k, v, None, bq, bkv, out=(od, ld))
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        for _ in range(args.dense_reps):
            spa2.fwd(q, k, v, None, bq, bkv, out=(od, ld))
        e1.record(stream)
        if train:
            for _ in range(args.dense_reps):
                spa2.bwd(q, k, v, od, ld, do, None, bq, bkv, out=(dq, dk, dv))
        e2.record(stream)
        torch.cuda.synchronize()
        dense = dict(fwd_ms=e0.elapsed_time(e1) / args.dense_reps)
        if train:
            dense["bwd_ms"] = e1.elapsed_time(e2) / args.dense_reps
        del od, ld
        log(f"[bench] dense {dense}")

    kernel_flops = {"fwd": flops_fwd}
    if train:
        kernel_flops.update(bwd_dkdv=8.0 * D * area, bwd_dq_rowterm=2.0 * D * area)
    dom = max(kernel_flops, key=lambda n: per_stage[n])
    achieved = kernel_flops[dom] / (per_stage[dom] * 1e-3) / 1e12
    roofline = dict(bound="mfma", kernel=dom, achieved=round(achieved, 2),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                    traffic=None if calibrated else recorded_traffic(dom, args.workload),
                    flops_per_launch=kernel_flops[dom], ms_per_launch=round(per_stage[dom], 4))
    mask_bytes = 2.0 * B * H * N * D * q.element_size()  # Q and K read once
    copy_gbs = copy_bandwidth()
    # the mask stage split: pooling (reads Q and K: the HBM-bound part) against the rest
    # (fp64 P-bar GEMM, per-row selection, lists), from separate timed pool calls
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    spa2.pool(q, k, bq, bkv)
    pe[0].record()
    for _ in range(10):
        spa2.pool(q, k, bq, bkv)
    pe[1].record()
    torch.cuda.synchronize()
    pool_ms = pe[0].elapsed_time(pe[1]) / 10
    # every timed kernel against both ceilings: MFMA (algorithmic flops) and memory (the
    # recorded counter bytes, when the kernel is unchanged since they were taken)
    kernels = {}
    for name, fl in kernel_flops.items():
        t = per_stage[name] * 1e-3
        rec = None if calibrated else recorded_traffic(name, args.workload)  # recorded at 128/64
        kernels[name] = {"ms": round(per_stage[name], 4), "tflops": round(fl / t / 1e12, 2),
                         "mfma_frac": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic_bytes": rec,
                         "GB/s": None if rec is None else round(rec / t / 1e9, 1),
                         "hbm_frac": None if rec is None else round(rec / t / 1e9 / PEAK_HBM_GBS, 4),
                         "copy_frac": None if rec is None else round(rec / t / 1e9 / copy_gbs, 4)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inp, w, gmask, flops_fwd + flops_bwd)
        log(f"[bench] cpu baseline {cpu}")

    sparse_attn = sum(per_stage[n] for n in per_stage if n != "mask")
    value = (flops_fwd + flops_bwd) / (ms_step * 1e-3) / 1e12
    speedup = None
    if dense:
        speedup = {"fwd_kernel": round(dense["fwd_ms"] / per_stage["fwd"], 2),
                   "fwd_incl_mask": round(dense["fwd_ms"] / (per_stage["fwd"] + per_stage["mask"]), 2)}
        if train:
            speedup["fwd_bwd_incl_mask"] = round((dense["fwd_ms"] + dense["bwd_ms"]) / ms_step, 2)
    shape = ("Wan2.1-14B 720p" if args.workload == "wan14b_720p" else
             "Wan2.1-1.3B 480p" if args.workload == "wan13b_480p" else args.workload)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded generator, {shape} attention shape)",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "D": D, "bq": bq,
                   "bkv": bkv, "k": kf, "p": pf, "kept_fraction": round(kept_frac, 6),
                   "kept_area_tokens2": area, "p_calibrated": calibrated,
                   "unrounded_o": bool(args.o_f32),
                   "step": "mask+fwd+bwd" if train else "mask+fwd"},
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "stages_ms": {k_: round(v_, 4) for k_, v_ in per_stage.items()},
        "stages_spread_ms": spread,
        "stages_cold_ms": cold,
        ("fwd_bwd_ms" if train else "fwd_ms"): round(sparse_attn, 4),
        ("fwd_bwd_tflops" if train else "fwd_only_tflops"):
            round((flops_fwd + flops_bwd) / (sparse_attn * 1e-3) / 1e12, 2),
        "fwd_tflops": round(flops_fwd / (per_stage["fwd"] * 1e-3) / 1e12, 2),
        "mask_split_ms": {"pool": round(pool_ms, 4),
                          "scores_select_lists": round(per_stage["mask"] - pool_ms, 4),
                          "pool_GB/s": round(mask_bytes / (pool_ms * 1e-3) / 1e9, 1)},
        "mask_hbm": {"bytes": mask_bytes,
                     "GB/s": round(mask_bytes / (per_stage["mask"] * 1e-3) / 1e9, 1),
                     "frac": round(mask_bytes / (per_stage["mask"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "copy_GB/s": round(copy_gbs, 1)},
        "dense_ms": {k_: round(v_, 3) for k_, v_ in dense.items()},
        "speedup_vs_dense": speedup,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


def run_sweep(args):
    """Top-k only, Top-p only and hybrid masks on the near-uniform and the sink-skewed
    generators at the 480p shape: kept fraction, mask and forward time, and the relative
    L1 error of O against the dense forward of the same kernel family, split into the two
    terms of the error decomposition (dropped probability mass, renormalisation of the
    kept mass). One oracle spot check of the mask per generator on two heads."""
    import numpy as np
    import torch

    import block_sparse_attention_spa2_amd as spa2
    from gen import configs

    torch.cuda.set_device(0)
    results = []
    checks = {}
    for wl in ("sweep_uniform", "sweep_skewed"):
        w = configs.params(wl)
        B, H, N, D, bq, bkv = w["B"], w["H"], w["N"], w["D"], w["BQ"], w["BKV"]
        t0 = time.time()
        inp = configs.make_inputs(wl, with_do=False)
        q, k, v = (_dev(getattr(inp, n)) for n in ("q", "k", "v"))
        log(f"[sweep] {wl} inputs drawn in {time.time() - t0:.1f}s")
        od32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        od, ld = spa2.fwd(q, k, v, None, bq, bkv, o_f32=od32)
        os32 = torch.empty_like(od32)
        o, lse = torch.empty_like(q), torch.empty_like(ld)
        bm = spa2.BlockMask.empty(B, H, N, bq, bkv, q.device)
        mws = torch.empty(spa2.mask_workspace_size(q, bq, bkv), dtype=torch.uint8, device="cuda")
        grid = ([(kf, 0.0) for kf in configs.SWEEP_K] + [(0.0, pf) for pf in configs.SWEEP_P]
                + [(kf, pf) for kf in configs.SWEEP_K for pf in configs.SWEEP_P])
        for kf, pf in grid:
            mode = "topk" if pf == 0 else "topp" if kf == 0 else "hybrid"
            ts = {"mask": [], "fwd": []}
            for _ in range(args.warmup + args.steps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record()
                spa2.mask(q, k, kf, pf, bq, bkv, out=bm, workspace=mws)
                e[1].record()
                spa2.fwd(q, k, v, bm, out=(o, lse), o_f32=os32)
                e[2].record()
                torch.cuda.synchronize()
                ts["mask"].append(e[0].elapsed_time(e[1]))
                ts["fwd"].append(e[1].elapsed_time(e[2]))
            # error decomposition (spa2_error_terms): sums of |O_dense|, |O_dense - O_sparse|,
            # |dropped-mass term|, |renormalisation term| per head; tau per row
            terms, tau = spa2.error_terms(os32, lse, od32, ld, bq, bkv, with_tau=True)
            tot = terms.sum(dim=(0, 1)).tolist()
            l1_dense = tot[0]
            e_drop, e_renorm = tot[2] / l1_dense, tot[3] / l1_dense
            results.append({
                "generator": wl, "mode": mode, "k": kf, "p": pf,
                "kept_fraction": round(bm.mask.float().mean().item(), 6),
                "mask_ms": round(_pct(ts["mask"][args.warmup:], 50), 4),
                "fwd_ms": round(_pct(ts["fwd"][args.warmup:], 50), 4),
                "rel_l1": round(tot[1] / l1_dense, 5),
                "rel_l1_dropped_mass": round(e_drop, 5),
                "rel_l1_renormalisation": round(e_renorm, 5),
                "mean_dropped_mass": round(float((1.0 - tau).mean().item()), 5),
            })
            log(f"[sweep] {results[-1]}")
        # oracle spot check: one hybrid setting, two heads
        import oracle
        kf, pf = 0.05, 0.60
        spa2.mask(q, k, kf, pf, bq, bkv, out=bm, workspace=mws)
        g = bm.mask.cpu().numpy().astype(bool)
        mism = band = 0
        for h in (0, H - 1):
            m, info = oracle.block_mask_head(inp.head_f64("q", 0, h), inp.head_f64("k", 0, h),
                                             bq, bkv, kf, pf, with_info=True)
            for i, j in np.argwhere(m != g[0, h]):
                if j in set(info["rows"][i]["p_band"]):
                    band += 1
                else:
                    mism += 1
        checks[wl] = {"k": kf, "p": pf, "heads": [0, H - 1], "mask_mismatch_outside_p_band": mism,
                      "mask_p_band_flips": band}
        assert mism == 0, (wl, mism)
        del q, k, v, od, od32, os32, o, lse, ld, bm, mws
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": results, "oracle_spot_check": checks}), flush=True)


def check_parity(inp, w, gmask, o, lse, dq, dk, dv):
    """Masks of every head against the oracle; O, LSE and dQ of sampled query blocks and
    dK, dV of sampled key blocks of the first and last head."""
    import numpy as np

    import oracle

    B, H, N, D, bq, bkv = w["B"], w["H"], w["N"], w["D"], w["BQ"], w["BKV"]
    t0 = time.time()
    mism = band = 0
    masks = {}
    for b in range(B):
        for h in range(H):
            m, info = oracle.block_mask_head(inp.head_f64("q", b, h), inp.head_f64("k", b, h),
                                             bq, bkv, w["k"], w["p"], with_info=True)
            masks[(b, h)] = m
            diff = np.argwhere(m != gmask[b, h])
            for i, j in diff:
                if j in set(info["rows"][i]["p_band"]):
                    band += 1
                else:
                    mism += 1
    assert mism == 0, f"mask mismatches outside the p band: {mism}"
    to64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    train = dq is not None
    on, ln = to64(o), lse.cpu().numpy()
    if train:
        dqn, dkn, dvn = to64(dq), to64(dk), to64(dv)
    errs = {}
    tm, tn = gmask.shape[-2:]
    for h in sorted({0, H - 1}):
        m = masks[(0, h)]
        q, k, v = (inp.head_f64(x, 0, h) for x in ("q", "k", "v"))
        qblocks = [0, tm // 3, tm - 1]
        kblocks = [1, tn // 2, tn - 1]
        o_ref, lse_ref = oracle.attn_fwd_head(q, k, v, m, bq, bkv, rows=qblocks)
        qsegs = [np.arange(i * bq, min(N, (i + 1) * bq)) for i in qblocks]
        qr = np.concatenate(qsegs)
        # every sampled block is held to the bar on its own (worst block reported)
        cmp = [("O", on[0, h], o_ref, qsegs)]
        if train:
            do = inp.head_f64("do", 0, h)
            rows = sorted(set(qblocks) | {i for j in kblocks for i in np.flatnonzero(m[:, j])})
            dq_ref, dk_ref, dv_ref = oracle.attn_bwd_head(q, k, v, do, m, bq, bkv, rows=rows)
            ksegs = [np.arange(j * bkv, min(N, (j + 1) * bkv)) for j in kblocks]
            cmp += [("dQ", dqn[0, h], dq_ref, qsegs), ("dK", dkn[0, h], dk_ref, ksegs),
                    ("dV", dvn[0, h], dv_ref, ksegs)]
        for name, got, ref, segs in cmp:
            for sg in segs:
                e = float(np.linalg.norm(got[sg] - ref[sg]) / np.linalg.norm(ref[sg]))
                errs[name] = max(errs.get(name, 0.0), e)
        errs["LSE_abs"] = max(errs.get("LSE_abs", 0.0), float(np.abs(ln[0, h][qr] - lse_ref[qr]).max()))
    tol = 2e-2 if inp.dtype == "bf16" else 1e-4
    for name in ("O", "dQ", "dK", "dV"):
        if name in errs:
            assert errs[name] <= tol, f"{name} rel-L2 {errs[name]}"
    return {"mask_mismatch_outside_p_band": mism, "mask_p_band_flips": band,
            "rel_l2_worst_sampled_block": {k_: float(f"{v_:.3e}") for k_, v_ in errs.items()},
            "seconds": round(time.time() - t0, 1)}


def cpu_baseline(inp, w, gmask, total_flops, budget_s=20.0, stride=1):
    """The float64 oracle on a bounded sample of the workload, extrapolated to the whole
    step: the mask of whole heads plus forward and backward of every `stride`-th query
    block, repeated head by head until about `budget_s` seconds have passed (at 480p the
    whole step fits in that time)."""
    import numpy as np

    import oracle

    B, H, N, D, bq, bkv = w["B"], w["H"], w["N"], w["D"], w["BQ"], w["BKV"]
    tm = gmask.shape[2]
    t_mask = t_fb = 0.0
    heads = 0
    qblocks_done = 0
    t_start = time.time()
    for h in range(H):
        q, k, v = (inp.head_f64(x, 0, h) for x in ("q", "k", "v"))
        t0 = time.time()
        m = oracle.block_mask_head(q, k, bq, bkv, w["k"], w["p"])
        t1 = time.time()
        rows = list(range(h % stride, tm, stride))
        oracle.attn_fwd_head(q, k, v, m, bq, bkv, rows=rows)
        if inp.do is not None:
            oracle.attn_bwd_head(q, k, v, inp.head_f64("do", 0, h), m, bq, bkv, rows=rows)
        t2 = time.time()
        t_mask += t1 - t0
        t_fb += t2 - t1
        heads += 1
        qblocks_done += len(rows)
        if time.time() - t_start > budget_s:
            break
    est = (t_mask / heads) * B * H + (t_fb / qblocks_done) * B * H * tm
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": round(total_flops / est / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(threads, len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": (f"float64 oracle: mask of {heads} whole head(s) and forward"
                       f"{'+backward' if inp.do is not None else ''} of "
                       f"{'every' if stride == 1 else f'every {stride}th'} query block of "
                       f"those heads ({qblocks_done} of "
                       f"{B * H * tm} blocks), extrapolated to the full step "
                       f"({est:.1f} s estimated)"),
            "seconds_measured": round(time.time() - t_start, 1), "cpu_model": _cpu_model()}


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


if __name__ == "__main__":
    main()
