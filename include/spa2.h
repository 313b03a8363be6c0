/*
 * spa2.h - C ABI of the SpargeAttention2 hot path on AMD MI355X (gfx950).
 *
 * The method (SpargeAttention2, arXiv 2602.13515) predicts a block mask from pooled
 * queries and keys and then runs attention only over the kept blocks:
 *   1. partition Q into T_m = ceil(N/BQ) query blocks and K, V into T_n = ceil(N/BKV)
 *      key blocks (paper.rainbus.top summary, section "方法步骤详情", step 1);
 *   2. mean-pool every block and form P-bar = softmax(pool(Q) pool(K)^T / sqrt(D)) per
 *      row (same section, step 2);
 *   3. keep key block j of query block i iff j is in Top-k(P-bar_i, k%) U
 *      Top-p(P-bar_i, p%) (step 3; the union formula of section "技术新颖性");
 *   4. compute attention for the kept block pairs only, with the softmax taken over
 *      the kept keys (step 4; section "前置知识", block-sparse attention), forward and
 *      backward (the sparse attention is trainable: abstract and section "核心方法").
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. Q, K, V, O, dO, dQ, dK, dV
 *     are contiguous [B, H, N, D] in desc->dtype (D fastest). LSE is float [B, H, N].
 *   - Alignment (the kernels move rows in 16-byte pieces): [B, H, N, D] tensors and the
 *     optional fp32 O start on a 16-byte boundary, double arrays on 8 bytes, float and
 *     int32 arrays (LSE, Dv, lists, orders, workspaces other than the mask workspace) on
 *     4 bytes. Every hipMalloc or PyTorch allocation is; otherwise SPA2_E_ALIGN.
 *   - Descriptor structs are HOST memory and are read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call
 *     enqueues its kernels on that stream and returns without synchronising.
 *   - The library never allocates device memory. Calls that need scratch space take a
 *     caller-provided workspace whose size comes from the matching *_workspace_size call.
 *   - Every argument is validated before any HIP call; an invalid call returns its error
 *     code and writes nothing. A failed kernel launch returns SPA2_E_HIP (details from
 *     spa2_last_error()). No C++ exception crosses this boundary.
 *   - Supported: dtype F32 or BF16, D in {64, 128}, BQ in {64, 128, 256},
 *     BKV in {32, 64, 128}, 1 <= N <= 2^20, B*H >= 1, T_n <= 4096,
 *     B*H*max(T_m, T_n) <= 2^26. The method's sizes
 *     are BQ = 128, BKV = 64; the others are the block-size variants the pages suggest
 *     trying (rainbus summary, "局限与改进": fixed block sizes are a limitation). The
 *     attention kernels work on tiles of at most 128 rows and 64 keys (the bf16 forward
 *     at D = 128 on 32-key steps), so a larger block is processed as several tiles (same
 *     lists; mask = NULL and an all-ones mask give the same bits).
 *   - Attention is non-causal; the scale is 1/sqrt(D); LSE is the natural-log
 *     log-sum-exp of the scaled scores over the kept keys. Outputs are rounded to the
 *     input dtype (round to nearest even) from fp32 accumulators. A query row whose
 *     block keeps no key block gets O = 0, LSE = -inf and dQ = 0.
 */
#ifndef SPA2_H
#define SPA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPA2_OK = 0,
  SPA2_E_NULL = 1,      /* a required pointer is NULL */
  SPA2_E_SHAPE = 2,     /* B, H, N, D, BQ or BKV out of the supported range */
  SPA2_E_DTYPE = 3,     /* unknown dtype */
  SPA2_E_PARAM = 4,     /* k or p outside [0, 1], NaN, or both zero */
  SPA2_E_WORKSPACE = 5, /* workspace NULL or smaller than the size call reports */
  SPA2_E_HIP = 6,       /* a HIP runtime call or kernel launch failed */
  SPA2_E_ALIGN = 7,     /* a device pointer is not aligned as the conventions require */
  SPA2_E_SCRATCH = 8    /* too large for the built-in scratch of spa2_bwd_noalloc */
} spa2_status;

typedef enum { SPA2_F32 = 0, SPA2_BF16 = 1 } spa2_dtype;

/* Problem shape. T_m = ceil(N/BQ), T_n = ceil(N/BKV); the last block of each may be
 * partial (it covers the rows up to N only). */
typedef struct {
  int32_t B, H, N, D; /* batch, heads, tokens, head dimension */
  int32_t BQ, BKV;    /* query and key block sizes (the method uses 128 and 64) */
  int32_t dtype;      /* spa2_dtype of every [B, H, N, D] tensor */
} spa2_desc;

/* Block mask M-bar and its compacted lists, all device memory owned by the caller.
 *   mask    uint8 [B, H, T_m, T_n]   1 = block pair kept
 *   row_cnt int32 [B, H, T_m]        kept key blocks per query block
 *   row_idx int32 [B, H, T_m, T_n]   their indices, ascending; entries past row_cnt unused
 *   col_cnt int32 [B, H, T_n]        query blocks that keep each key block
 *   col_idx int32 [B, H, T_n, T_m]   their indices, ascending; entries past col_cnt unused
 *   row_order int32 [B, H, T_m]      optional (NULL = natural order): the order in which
 *                                    the attention kernels take query blocks
 *   col_order int32 [B, H, T_n]      optional: the same for key blocks (dK/dV pass)
 * The forward reads the row lists; the backward reads both. The orders only schedule work
 * (results do not depend on them): the flattened block index range is cut into eight
 * contiguous parts (one per XCD of the GPU, sharing an L2 cache). A part of row_order
 * lists its query blocks head by head, each head's by kept count, largest first (blocks
 * running together on an XCD then read one head's key blocks). A part of col_order lists
 * first the key blocks kept by at least a quarter of the query blocks (largest count
 * first, so the longest lists start at once), then the others head by head, largest
 * first. Blocks of equal count appear in no particular order. The mask calls write the
 * orders when non-NULL. */
typedef struct {
  uint8_t* mask;
  int32_t* row_cnt;
  int32_t* row_idx;
  int32_t* col_cnt;
  int32_t* col_idx;
  int32_t* row_order;
  int32_t* col_order;
} spa2_blockmask;

/* Text for a status code (static storage). */
const char* spa2_status_str(spa2_status s);

/* Detail of the last SPA2_E_HIP on the calling thread ("" if none; thread-local). */
const char* spa2_last_error(void);

/* Block counts for a descriptor (host only, no validation beyond positivity). */
int32_t spa2_num_blocks(int32_t n, int32_t block);

/* Step 2, pooling (rainbus summary, "方法步骤详情", step 2: pool(Q), pool(K)).
 * qbar: double [B, H, T_m, D], kbar: double [B, H, T_n, D] (device, caller-owned):
 * the arithmetic mean of each block's valid rows, accumulated in double. */
spa2_status spa2_pool(const spa2_desc* desc, const void* q, const void* k, double* qbar,
                      double* kbar, void* stream);

/* Workspace bytes that spa2_mask needs for this descriptor (pooled vectors, rows padded
 * to D + 2, and the pooled score matrix, all double, plus 256 bytes so that the buffer
 * may start at any address). */
spa2_status spa2_mask_workspace_size(const spa2_desc* desc, size_t* bytes);

/* Steps 1-3: pool, P-bar, Top-k U Top-p, compacted row and column lists.
 * k_frac, p_frac in [0, 1], not both 0. Per row, Top-k keeps the first
 * n_k = min(T_n, ceil(k_frac * T_n - 1e-9)) blocks of the order (P-bar descending,
 * block index ascending); Top-p keeps every block of that order whose exclusive prefix
 * sum of P-bar is below p_frac (the smallest prefix that reaches p); the mask is their
 * union (rainbus summary, "前置知识" for the Top-k / Top-p rules, "研究动机" for the
 * worked rows, "技术新颖性" for the union). P-bar is computed in double precision.
 * pbar_out: optional double [B, H, T_m, T_n] copy of P-bar (NULL = not written).
 * workspace: device buffer of at least spa2_mask_workspace_size bytes. */
spa2_status spa2_mask(const spa2_desc* desc, const void* q, const void* k, double k_frac,
                      double p_frac, const spa2_blockmask* out, double* pbar_out,
                      void* workspace, size_t ws_bytes, void* stream);

/* Step 3 alone: the hybrid selection on a given P-bar (double [B, H, T_m, T_n], rows
 * summing to 1) -> mask and lists. Same rule as spa2_mask. */
spa2_status spa2_select(const spa2_desc* desc, const double* pbar, double k_frac,
                        double p_frac, const spa2_blockmask* out, void* stream);

/* Rebuild row and column lists from a caller-filled out->mask (for masks made outside
 * this library). */
spa2_status spa2_mask_lists(const spa2_desc* desc, const spa2_blockmask* m, void* stream);

/* Step 4, forward (rainbus summary, "方法步骤详情", step 4): for every query row, the
 * softmax of q.k/sqrt(D) over the keys of the kept key blocks, O = weights . V, and
 * LSE. m = NULL runs dense attention (every block kept) through the same kernel.
 * o: [B, H, N, D] dtype, lse: float [B, H, N].
 * o_f32: optional float [B, H, N, D] copy of O before rounding to dtype (NULL = not
 * written). Handing it to the backward lets the row term rowsum(dO * O) use the
 * unrounded O. With bf16 the dQ pass removes the offset part of the row term's error
 * either way, so it is an accuracy refinement, not a requirement (sampled dQ 0.21% vs
 * 0.20% relative L2 at the 480p shape, 1.3% vs 0.9% on the 8192-token case); it costs
 * 4 bytes per element of extra writes. */
spa2_status spa2_fwd(const spa2_desc* desc, const void* q, const void* k, const void* v,
                     const spa2_blockmask* m, void* o, float* lse, float* o_f32,
                     void* stream);

/* Workspace bytes that spa2_bwd needs. The workspace holds, from its start, the row term
 * rowsum(dO * O) (float [B, H, N]; the dQ pass stores it, the dK/dV pass reads it) and, for
 * bf16, the mean key of every key tile of the dQ pass (bf16 [B, H, tiles, D], from the
 * first 256-byte boundary after the row term; tiles = 2 T_n for b_kv = 128, else T_n),
 * formed at the start of each dQ pass as the reference vectors of its rounding
 * corrections: B H N 4 bytes for fp32, B H N 4 + 256 + B H tiles D 2 for bf16. */
spa2_status spa2_bwd_workspace_size(const spa2_desc* desc, size_t* bytes);

/* The same size as a plain return value, 0 for an invalid descriptor (or NULL), which
 * spa2_bwd then rejects with its own status. The backward is deterministic and always
 * needs this buffer. */
size_t spa2_bwd_workspace_bytes(const spa2_desc* desc);

/* Backward of spa2_fwd with the same mask held fixed (the mask gets no gradient):
 *   dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = dS K / sqrt(D),
 *   dK = dS^T Q / sqrt(D), dV = P^T dO, over kept pairs only, with P rebuilt from LSE.
 * o, lse (and o_f32 if not NULL) are the forward's outputs for the same inputs and mask;
 * rowsum(dO * O) reads o_f32 when given, else o. m = NULL is dense.
 * dq, dk, dv: [B, H, N, D] dtype (fully overwritten). Deterministic: every output
 * element is reduced in a fixed order. */
spa2_status spa2_bwd(const spa2_desc* desc, const void* q, const void* k, const void* v,
                     const void* o, const float* o_f32, const float* lse, const void* dout,
                     const spa2_blockmask* m, void* dq, void* dk, void* dv, void* workspace,
                     size_t ws_bytes, void* stream);

/* Bytes of device scratch that spa2_bwd_noalloc holds per GPU: the backward workspace of
 * up to this size (spa2_bwd_workspace_bytes), e.g. 40 heads of 75,600 tokens at D = 128
 * with 64-key blocks (24.2 MB). */
#define SPA2_NOALLOC_SCRATCH_BYTES (32u << 20)

/* spa2_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid allocation). The
 * workspace is a scratch array built into the library (SPA2_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends); the call itself allocates nothing. Same arguments,
 * kernels and results as spa2_bwd (bit for bit). Returns SPA2_E_SCRATCH, before any HIP
 * call, when spa2_bwd_workspace_bytes exceeds the scratch. The scratch is shared by every
 * call on a GPU and keeps the last call's contents (nothing in it needs clearing: the dQ
 * pass writes every mean key and row term before they are read), so calls that overlap on one GPU
 * (other streams, other threads) race: serialise them. The first call on a device looks
 * up the scratch address there (hipGetSymbolAddress on the stream's device). */
spa2_status spa2_bwd_noalloc(const spa2_desc* desc, const void* q, const void* k, const void* v,
                             const void* o, const float* o_f32, const float* lse,
                             const void* dout, const spa2_blockmask* m, void* dq, void* dk,
                             void* dv, void* stream);

/* The passes of spa2_bwd, callable one by one (for example to time them, or to run the
 * dK/dV pass on another stream). spa2_bwd is exactly spa2_bwd_dq_rowterm, then
 * spa2_bwd_dkdv, on one stream.
 *   spa2_bwd_dq_rowterm: dQ from the row lists (one workgroup per query block), and the
 *                  row term rowsum(dO * O), O = o_f32 if given, computed by the same pass
 *                  from the dO rows it loads anyway, stored at the workspace's start;
 *   spa2_bwd_dkdv: dK, dV from the column lists (one workgroup per key block);
 *   spa2_bwd_prep: the row term alone (a separate pass over O and dO);
 *   spa2_bwd_dq:   dQ alone, reading the row term from the workspace's start.
 * workspace / ws_bytes: as for spa2_bwd (the dQ passes write its mean keys); dvec: the row
 * term, float [B, H, N] (device), normally the first B H N floats of that workspace.
 * The row term must be for the same O and dO (from either pass; the two sum in
 * different orders, so results agree to rounding, not bit for bit). */
spa2_status spa2_bwd_dq_rowterm(const spa2_desc* desc, const void* q, const void* k,
                                const void* v, const void* o, const float* o_f32,
                                const float* lse, const void* dout,
                                const spa2_blockmask* m, void* workspace, size_t ws_bytes,
                                void* dq, void* stream);
spa2_status spa2_bwd_prep(const spa2_desc* desc, const void* o, const float* o_f32,
                          const void* dout, float* dvec, void* stream);
spa2_status spa2_bwd_dkdv(const spa2_desc* desc, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, const float* dvec,
                          const spa2_blockmask* m, void* dk, void* dv, void* stream);
spa2_status spa2_bwd_dq(const spa2_desc* desc, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, void* workspace, size_t ws_bytes,
                        const spa2_blockmask* m, void* dq, void* stream);

/* Error decomposition of the sparse output against the dense one (rainbus summary,
 * "技术新颖性": with p the dense attention weights, m the kept-key mask and
 * tau = sum(p * m) the dense mass on kept keys of a row,
 *   O_dense - O_sparse = (p * (1 - m)) V + (1 - 1/tau) (p * m) V,
 * the first term being the dropped mass, the second the renormalisation of the kept
 * weights). Since (p * m) V = tau O_sparse and tau = exp(LSE_sparse - LSE_dense), both
 * terms follow from the two forwards' outputs:
 *   dropped = O_dense - tau O_sparse,   renormalisation = (tau - 1) O_sparse.
 * o_sparse, o_dense: float [B, H, N, D] (the o_f32 outputs of spa2_fwd with the mask and
 * with m = NULL); lse_sparse, lse_dense: float [B, H, N]. A row with no kept key has
 * tau = 0. Writes terms[B, H, 4] (double, device), per head:
 *   [0] sum |O_dense|, [1] sum |O_dense - O_sparse|, [2] sum |dropped|,
 *   [3] sum |renormalisation|   (sums over the head's N x D elements; relative L1 errors
 *   are [1]/[0], [2]/[0], [3]/[0]),
 * and, if tau is not NULL, tau[B, H, N] (float, device). Sums are accumulated in double
 * with atomic adds, so the last bits may vary between runs. */
spa2_status spa2_error_terms(const spa2_desc* desc, const float* o_sparse, const float* lse_sparse,
                             const float* o_dense, const float* lse_dense, double* terms,
                             float* tau, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA2_H */
