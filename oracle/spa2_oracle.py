"""Plain float64 reference of the SpargeAttention2 hot path.

TEST INFRASTRUCTURE. This module is the oracle that the GPU library is checked against.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may use it; the
product path never imports it. It shares no code, table or helper with the HIP library.

Everything is float64 numpy on the values actually stored (bf16 or fp32 inputs upcast).
Each function follows one step of the method as the pages define it and cites it. The
pages are cited by address and section:

  [rainbus]  paper.rainbus.top/paper/2602.13515 (Chinese structured summary), sections
             "前置知识" (background: Top-k/Top-p masks, block-sparse attention),
             "研究动机" (motivation, with the two worked example rows),
             "方法步骤详情" (method steps 1-6), "技术新颖性" (mask formula and the
             error decomposition), "局限与改进" / "独立分析的弱点" (b_q=128, b_kv=64).
  [gist]     gist.science/paper/2602.13515, section 2 "Methodology" (A: hybrid masking,
             C: efficient kernel implementation).
  [gist-nl]  gist.science/nl/paper/2602.13515 (Dutch summary; restates the mask formula).
  [abstract] chatpaper.ai abstract page (95% sparsity, trainable implementation).

Readings taken where the pages are silent (each is listed with its reason in the design
notes of the repository):
  * pool = arithmetic mean over the block's valid rows;
  * N not divisible by the block size: ceil block count, the last block is partial;
  * Top-k count n_k = ceil(k*T_n - 1e-9) clamped to [0, T_n], per row;
  * Top-p keeps rank r of the (value desc, index asc) order iff the exclusive prefix
    e_r = sum of the r larger values is < p (inclusive "reaches p" stop rule);
  * ties in P-bar are ordered by block index ascending;
  * attention is non-causal; softmax is renormalised over the kept keys only;
  * a row with no kept block has O = 0 and LSE = -inf;
  * the mask carries no gradient (hard mask, the same in forward and backward).
"""
from __future__ import annotations

import math

import numpy as np

# Band widths used to report (not to decide) near-threshold blocks.
P_BAND = 1e-6  # |e_r - p| <= 1e-6: membership may flip under rounding of the prefix sum
K_BAND = 1e-6  # |P_j - P_kth| <= 1e-6 * P_kth: rank order near the k-th value is fragile


# ---------------------------------------------------------------------------------------
# Step 1: block partition  ([rainbus] 方法步骤详情, step 1; 前置知识, block-sparse attention)
# ---------------------------------------------------------------------------------------
def n_blocks(n: int, b: int) -> int:
    """Number of blocks of size b covering n rows: ceil(n / b) (partial last block)."""
    return -(-n // b)


def block_range(n: int, b: int, i: int) -> tuple[int, int]:
    """Rows [lo, hi) of block i; the last block stops at n."""
    return i * b, min(n, (i + 1) * b)


# ---------------------------------------------------------------------------------------
# Step 2a: block mean pooling  ([rainbus] 方法步骤详情, step 2: pool(Q), pool(K))
# ---------------------------------------------------------------------------------------
def pool_blocks(x: np.ndarray, b: int) -> np.ndarray:
    """Mean of each block's valid rows. x: [N, d] -> [ceil(N/b), d], float64.

    The sum runs over the rows in order (a running sum), then divides by the row count.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    t = n_blocks(n, b)
    out = np.empty((t, d), dtype=np.float64)
    for i in range(t):
        lo, hi = block_range(n, b, i)
        running = np.cumsum(x[lo:hi], axis=0)  # sequential accumulation down the rows
        out[i] = running[-1] / float(hi - lo)
    return out


# ---------------------------------------------------------------------------------------
# Step 2b: pooled block attention  ([rainbus] 方法步骤详情, step 2:
#          P-bar = softmax(pool(Q) pool(K)^T / sqrt(d)), softmax over each row)
# ---------------------------------------------------------------------------------------
def pooled_probs(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """P-bar [T_m, T_n] = row softmax of qbar kbar^T / sqrt(d), over all T_n blocks."""
    d = qbar.shape[1]
    s = (qbar @ kbar.T) / math.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------------------
# Step 3: hybrid Top-k U Top-p block mask
#   [rainbus] 前置知识 (Top-k keeps the k most probable entries of a row; Top-p keeps the
#   smallest set whose cumulative probability reaches p); 方法步骤详情, step 3
#   (M1 = Top-k(P-bar, k%), M2 = Top-p(P-bar, p%), M-bar = M1 U M2); 技术新颖性 (the
#   row-wise formula: keep j iff j in Top-k(P-bar_i,:, k%) U Top-p(P-bar_i,:, p%));
#   [gist] 2.A; [gist-nl] (same union).
# ---------------------------------------------------------------------------------------
def topk_count(k_frac: float, t_n: int) -> int:
    """Top-k keeps k% of a row's T_n blocks: n_k = ceil(k*T_n - 1e-9), clamped to [0, T_n]."""
    return int(min(t_n, max(0, math.ceil(k_frac * t_n - 1e-9))))


def select_row(prow: np.ndarray, k_frac: float, p_frac: float) -> dict:
    """Hybrid selection on one P-bar row.

    Returns a dict with
      kept   : ascending int array of kept block indices (Top-k U Top-p)
      topk   : ascending int array of the Top-k blocks
      topp   : ascending int array of the Top-p blocks
      order  : block indices by (value desc, index asc)
      excl   : exclusive prefix sums e_r in that order (running float64 sum)
      p_band : blocks not kept by Top-k whose exclusive prefix lies within P_BAND of p
               (their Top-p membership can flip under rounding of the prefix sum)
      k_band : blocks whose value is within K_BAND (relative) of the n_k-th value
    """
    prow = np.asarray(prow, dtype=np.float64)
    t_n = prow.shape[0]
    idx = np.arange(t_n)
    order = np.lexsort((idx, -prow))  # primary: value descending; ties: index ascending
    n_k = topk_count(k_frac, t_n)
    in_topk = np.zeros(t_n, dtype=bool)
    in_topk[order[:n_k]] = True

    # e_r = sum of the r larger values; np.cumsum accumulates left to right.
    excl = np.zeros(t_n, dtype=np.float64)
    if t_n > 1:
        excl[1:] = np.cumsum(prow[order])[:-1]
    # Top-p: the smallest prefix whose mass reaches p = every rank whose exclusive prefix
    # is still below p (the block that makes the sum reach p is included).
    in_topp = np.zeros(t_n, dtype=bool)
    in_topp[order[excl < p_frac]] = True

    kept = np.flatnonzero(in_topk | in_topp)
    ranks = np.arange(t_n)
    p_band = np.sort(order[(ranks >= n_k) & (np.abs(excl - p_frac) <= P_BAND)])
    k_band = np.zeros(0, dtype=np.int64)
    if n_k > 0:
        kth = prow[order[n_k - 1]]
        k_band = np.flatnonzero(np.abs(prow - kth) <= K_BAND * kth)
    return dict(kept=kept, topk=np.flatnonzero(in_topk), topp=np.flatnonzero(in_topp),
                order=order, excl=excl, p_band=p_band, k_band=k_band)


def block_mask_head(q: np.ndarray, k: np.ndarray, bq: int, bkv: int,
                    k_frac: float, p_frac: float, with_info: bool = False):
    """Block mask M-bar [T_m, T_n] (bool) of one head from Q, K [N, d].

    pool -> P-bar -> per-row hybrid selection. With with_info, also returns P-bar, the
    pooled vectors and the per-row selection dicts (for band reporting).
    """
    qbar = pool_blocks(q, bq)
    kbar = pool_blocks(k, bkv)
    pbar = pooled_probs(qbar, kbar)
    t_m, t_n = pbar.shape
    mask = np.zeros((t_m, t_n), dtype=bool)
    rows = []
    for i in range(t_m):
        sel = select_row(pbar[i], k_frac, p_frac)
        mask[i, sel["kept"]] = True
        rows.append(sel)
    if with_info:
        return mask, dict(qbar=qbar, kbar=kbar, pbar=pbar, rows=rows)
    return mask


def block_mask(q: np.ndarray, k: np.ndarray, bq: int, bkv: int,
               k_frac: float, p_frac: float) -> np.ndarray:
    """Block mask for [B, H, N, d] inputs -> bool [B, H, T_m, T_n]; heads are independent."""
    b_, h_, n, _ = q.shape
    out = np.zeros((b_, h_, n_blocks(n, bq), n_blocks(n, bkv)), dtype=bool)
    for b in range(b_):
        for h in range(h_):
            out[b, h] = block_mask_head(q[b, h], k[b, h], bq, bkv, k_frac, p_frac)
    return out


# ---------------------------------------------------------------------------------------
# Step 4: block-sparse attention forward
#   [rainbus] 方法步骤详情, step 4 (for each kept block pair, S_ij = Q_i K_j^T / sqrt(d),
#   softmax taken online, output accumulated); 前置知识 (masked pairs skip both Q K^T and
#   P V); 技术新颖性 (the error term (1 - 1/tau) shows the kept weights are renormalised).
#   The oracle computes the same result directly: a softmax over the union of the kept
#   blocks' keys for every query row, no online rescaling.
# ---------------------------------------------------------------------------------------
def _kept_keys(n: int, bkv: int, cols) -> np.ndarray:
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(*block_range(n, bkv, j)) for j in cols])


def attn_fwd_head(q, k, v, mask, bq: int, bkv: int, rows=None):
    """O [N, d], LSE [N] (natural log) for one head under block mask [T_m, T_n].

    rows: optional iterable of query-block indices to compute (others stay O = 0,
    LSE = -inf); each computed block is exact, so sampled checks stay exact."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    for i in (range(mask.shape[0]) if rows is None else rows):
        lo, hi = block_range(n, bq, i)
        keys = _kept_keys(n, bkv, np.flatnonzero(mask[i]))
        if keys.size == 0:
            continue  # no kept block: O = 0, LSE = -inf
        s = (q[lo:hi] @ k[keys].T) * scale
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        out[lo:hi] = (e / l) @ v[keys]
        lse[lo:hi] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def attn_fwd(q, k, v, mask, bq: int, bkv: int):
    """Batched forward over [B, H, N, d] with mask [B, H, T_m, T_n]."""
    b_, h_, n, d = q.shape
    out = np.empty((b_, h_, n, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b_, h_, n), dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            out[b, h], lse[b, h] = attn_fwd_head(q[b, h], k[b, h], v[b, h], mask[b, h], bq, bkv)
    return out, lse


# ---------------------------------------------------------------------------------------
# Error decomposition  ([rainbus] 技术新颖性: O_dense - O_sparse = (p (1-m)) V +
#   (1 - 1/tau)(p m) V, p the dense weights, m the kept-key mask, tau the dense mass on
#   the kept keys). From the two forwards: tau = exp(LSE_sparse - LSE_dense) (0 for a row
#   with no kept key), (p m) V = tau O_sparse, so the terms are O_dense - tau O_sparse
#   (dropped mass) and (tau - 1) O_sparse (renormalisation).
# ---------------------------------------------------------------------------------------
def error_terms_head(o_sparse, lse_sparse, o_dense, lse_dense):
    """Per head: (sum |O_dense|, sum |O_dense - O_sparse|, sum |dropped|, sum |renorm|),
    and tau [N]."""
    o_s = np.asarray(o_sparse, np.float64)
    o_d = np.asarray(o_dense, np.float64)
    ls = np.asarray(lse_sparse, np.float64)
    ld = np.asarray(lse_dense, np.float64)
    tau = np.where(np.isneginf(ls), 0.0, np.exp(ls - ld))
    t = tau[:, None]
    sums = (np.abs(o_d).sum(), np.abs(o_d - o_s).sum(), np.abs(o_d - t * o_s).sum(),
            np.abs((t - 1.0) * o_s).sum())
    return np.array(sums), tau


# ---------------------------------------------------------------------------------------
# Backward ([rainbus] 核心方法 and [abstract]: the sparse attention is trainable, with a
# forward and a backward pass). The pages give no backward formulas; these are the
# derivatives of the forward above with the mask held fixed:
#   dP = dO V_C^T,  dS = P * (dP - rowsum(P * dP)),
#   dQ = dS K_C / sqrt(d),  dK_C += dS^T Q / sqrt(d),  dV_C += P^T dO.
# ---------------------------------------------------------------------------------------
def attn_bwd_head(q, k, v, do, mask, bq: int, bkv: int, rows=None):
    """dQ, dK, dV [N, d] for one head.

    rows: optional iterable of query-block indices whose contributions are summed. dQ of a
    listed block is complete; dK/dV of key block j are complete when every query block
    that keeps j is listed."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in (range(mask.shape[0]) if rows is None else rows):
        lo, hi = block_range(n, bq, i)
        keys = _kept_keys(n, bkv, np.flatnonzero(mask[i]))
        if keys.size == 0:
            continue
        s = (q[lo:hi] @ k[keys].T) * scale
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = do[lo:hi] @ v[keys].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[lo:hi] = (ds @ k[keys]) * scale
        dk[keys] += (ds.T @ q[lo:hi]) * scale
        dv[keys] += p.T @ do[lo:hi]
    return dq, dk, dv


def attn_bwd(q, k, v, do, mask, bq: int, bkv: int):
    """Batched backward over [B, H, N, d]."""
    b_, h_ = q.shape[:2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            dq[b, h], dk[b, h], dv[b, h] = attn_bwd_head(
                q[b, h], k[b, h], v[b, h], do[b, h], mask[b, h], bq, bkv)
    return dq, dk, dv
