// C ABI of the SpargeAttention2 hot path: argument validation and dispatch.
// Every check runs before the first HIP call, so an invalid call writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "../../include/spa2.h"
#include "kernels.h"

// Scratch memory of spa2_bwd_noalloc (the backward's workspace: row term and mean keys),
// for callers that cannot allocate. Every GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress (scratch_on_device below).
static __device__ __align__(256) unsigned char scratch[SPA2_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* where, hipError_t e) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
}

int blocks(int n, int b) { return (n + b - 1) / b; }

spa2_status check_desc(const spa2_desc* d, spa2::Shape* out) {
  if (!d) return SPA2_E_NULL;
  if (d->dtype != SPA2_F32 && d->dtype != SPA2_BF16) return SPA2_E_DTYPE;
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->N > (1 << 20)) return SPA2_E_SHAPE;
  if ((long long)d->B * d->H > (1LL << 24)) return SPA2_E_SHAPE;
  if (d->D != 64 && d->D != 128) return SPA2_E_SHAPE;
  if (d->BQ != 64 && d->BQ != 128 && d->BQ != 256) return SPA2_E_SHAPE;
  if (d->BKV != 32 && d->BKV != 64 && d->BKV != 128) return SPA2_E_SHAPE;
  const int tn = blocks(d->N, d->BKV), tm = blocks(d->N, d->BQ);
  if (tn > spa2::kMaxTn) return SPA2_E_SHAPE;
  // launch grids are counted in int (up to two tiles per block): B*H*max(T_m, T_n) <= 2^26
  // keeps them far from overflow and is beyond any problem that fits in device memory
  if ((long long)d->B * d->H * (tm > tn ? tm : tn) > (1LL << 26)) return SPA2_E_SHAPE;
  *out = spa2::Shape{d->B, d->H, d->N, d->D, d->BQ, d->BKV, d->dtype, tm, tn};
  return SPA2_OK;
}

spa2_status check_fracs(double k, double p) {
  if (std::isnan(k) || std::isnan(p)) return SPA2_E_PARAM;
  if (k < 0.0 || k > 1.0 || p < 0.0 || p > 1.0) return SPA2_E_PARAM;
  if (k == 0.0 && p == 0.0) return SPA2_E_PARAM;
  return SPA2_OK;
}

// Top-k count: ceil(k * T_n - 1e-9) clamped to [0, T_n].
int topk_count(double k, int tn) {
  const double c = std::ceil(k * (double)tn - 1e-9);
  if (c < 0.0) return 0;
  if (c > (double)tn) return tn;
  return (int)c;
}

spa2_status check_blockmask(const spa2_blockmask* m, bool need_lists) {
  if (!m || !m->mask) return SPA2_E_NULL;
  if (need_lists && (!m->row_cnt || !m->row_idx || !m->col_cnt || !m->col_idx)) return SPA2_E_NULL;
  return SPA2_OK;
}

// Alignment the kernels' vector loads need: 16 bytes for [B, H, N, D] tensors (rows are
// moved in 16-byte pieces), 8 for double arrays, 4 for float and int32 arrays. NULL passes.
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}
bool aligned4(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 4)) return false;
  return true;
}
bool lists_aligned(const spa2_blockmask* m) {
  return !m || aligned4({m->row_cnt, m->row_idx, m->col_cnt, m->col_idx, m->row_order, m->col_order});
}

// The mask workspace holds q-bar, k-bar (rows kPoolPitch(D) doubles apart) and the pooled
// scores (double), from the first 256-byte boundary of the caller's buffer: the slack
// makes any start address usable.
constexpr size_t kWsAlign = 256;
size_t mask_ws_bytes(const spa2::Shape& s) {
  const size_t bh = (size_t)s.BH(), pitch = (size_t)spa2::kPoolPitch(s.D);
  return bh * ((size_t)(s.Tm + s.Tn) * pitch + (size_t)s.Tm * s.Tn) * sizeof(double) + kWsAlign;
}

// The backward workspace holds the row term (float per query row) from its start, then,
// for bf16, the mean key of every key tile from the first 256-byte boundary after it.
size_t bwd_ws_bytes(const spa2::Shape& s) {
  const size_t kmean = spa2::bwd_kmean_bytes(s);
  return (size_t)s.BH() * s.N * sizeof(float) + (kmean ? kWsAlign + kmean : 0);
}
void* bwd_kmean(void* ws, const spa2::Shape& s) {
  const uintptr_t end = (uintptr_t)ws + (size_t)s.BH() * s.N * sizeof(float);
  return (void*)((end + kWsAlign - 1) & ~(uintptr_t)(kWsAlign - 1));
}

spa2_status hip_status(const char* where, hipError_t e) {
  if (e == hipSuccess) return SPA2_OK;
  set_error(where, e);
  return SPA2_E_HIP;
}

// Lists are complete: write the scheduling orders the caller asked for. Query blocks go
// head by head within each XCD's part (the forward and dQ passes then share K/V tiles in
// L2); key blocks go longest first across the whole part (a head's attention-sink column
// can hold most of the query blocks and must start first).
spa2_status write_orders(const spa2::Shape& s, const spa2_blockmask& m, hipStream_t hs) {
  // rows head by head (per_head = T_m), columns by count over the whole range
  const spa2::OrderJob rows{m.row_cnt, s.BH() * s.Tm, s.Tn, s.Tm, 0, m.row_order};
  const spa2::OrderJob cols{m.col_cnt, s.BH() * s.Tn, s.Tm, s.Tn, s.Tm / 4 > 1 ? s.Tm / 4 : 1,
                            m.col_order};
  return hip_status("order", spa2::launch_orders(m.row_order ? &rows : nullptr,
                                                 m.col_order ? &cols : nullptr, hs));
}

// Device address of `scratch` on the device that runs `stream`, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

spa2_status scratch_on_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_status("hipStreamGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(g_last_error, sizeof(g_last_error), "scratch: device %d out of range", dev);
    return SPA2_E_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status("hipGetDevice", e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status("hipSetDevice", e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status("hipGetSymbolAddress(scratch)", e);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SPA2_OK;
}

}  // namespace

extern "C" {

const char* spa2_status_str(spa2_status s) {
  switch (s) {
    case SPA2_OK: return "ok";
    case SPA2_E_NULL: return "a required pointer is NULL";
    case SPA2_E_SHAPE: return "shape out of the supported range";
    case SPA2_E_DTYPE: return "unknown dtype";
    case SPA2_E_PARAM: return "k/p fraction outside [0, 1], NaN, or both zero";
    case SPA2_E_WORKSPACE: return "workspace missing or too small";
    case SPA2_E_HIP: return "HIP runtime error";
    case SPA2_E_ALIGN: return "a device pointer is not aligned for the kernels' vector loads";
    case SPA2_E_SCRATCH: return "problem too large for the built-in scratch of the no-allocation call";
  }
  return "unknown status";
}

const char* spa2_last_error(void) { return g_last_error; }

int32_t spa2_num_blocks(int32_t n, int32_t block) {
  if (n < 1 || block < 1) return 0;
  return blocks(n, block);
}

spa2_status spa2_pool(const spa2_desc* desc, const void* q, const void* k, double* qbar,
                      double* kbar, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !qbar || !kbar) return SPA2_E_NULL;
  if (!aligned16({q, k}) || !aligned(qbar, 8) || !aligned(kbar, 8)) return SPA2_E_ALIGN;
  return hip_status("pool", spa2::launch_pool(s, q, k, qbar, kbar, s.D, (hipStream_t)stream));
}

spa2_status spa2_mask_workspace_size(const spa2_desc* desc, size_t* bytes) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!bytes) return SPA2_E_NULL;
  *bytes = mask_ws_bytes(s);
  return SPA2_OK;
}

spa2_status spa2_mask(const spa2_desc* desc, const void* q, const void* k, double k_frac,
                      double p_frac, const spa2_blockmask* out, double* pbar_out,
                      void* workspace, size_t ws_bytes, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k) return SPA2_E_NULL;
  if ((st = check_blockmask(out, true)) != SPA2_OK) return st;
  if ((st = check_fracs(k_frac, p_frac)) != SPA2_OK) return st;
  if (!workspace || ws_bytes < mask_ws_bytes(s)) return SPA2_E_WORKSPACE;
  if (!aligned16({q, k}) || !aligned(pbar_out, 8) || !lists_aligned(out)) return SPA2_E_ALIGN;

  const hipStream_t hs = (hipStream_t)stream;
  double* qbar = (double*)(((uintptr_t)workspace + kWsAlign - 1) & ~(uintptr_t)(kWsAlign - 1));
  const int pitch = spa2::kPoolPitch(s.D);
  double* kbar = qbar + (size_t)s.BH() * s.Tm * pitch;
  double* scores = kbar + (size_t)s.BH() * s.Tn * pitch;
  if ((st = hip_status("pool", spa2::launch_pool(s, q, k, qbar, kbar, pitch, hs))) != SPA2_OK) return st;
  if ((st = hip_status("scores", spa2::launch_scores(s, qbar, kbar, pitch, scores, hs))) != SPA2_OK)
    return st;
  if ((st = hip_status("select", spa2::launch_select(s, scores, true, pbar_out,
                                                     topk_count(k_frac, s.Tn), p_frac, *out,
                                                     hs))) != SPA2_OK)
    return st;
  if ((st = hip_status("cols", spa2::launch_cols(s, *out, hs))) != SPA2_OK) return st;
  return write_orders(s, *out, hs);
}

spa2_status spa2_select(const spa2_desc* desc, const double* pbar, double k_frac, double p_frac,
                        const spa2_blockmask* out, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!pbar) return SPA2_E_NULL;
  if ((st = check_blockmask(out, true)) != SPA2_OK) return st;
  if ((st = check_fracs(k_frac, p_frac)) != SPA2_OK) return st;
  if (!aligned(pbar, 8) || !lists_aligned(out)) return SPA2_E_ALIGN;
  const hipStream_t hs = (hipStream_t)stream;
  if ((st = hip_status("select", spa2::launch_select(s, pbar, false, nullptr,
                                                     topk_count(k_frac, s.Tn), p_frac, *out,
                                                     hs))) != SPA2_OK)
    return st;
  if ((st = hip_status("cols", spa2::launch_cols(s, *out, hs))) != SPA2_OK) return st;
  return write_orders(s, *out, hs);
}

spa2_status spa2_mask_lists(const spa2_desc* desc, const spa2_blockmask* m, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if ((st = check_blockmask(m, true)) != SPA2_OK) return st;
  if (!lists_aligned(m)) return SPA2_E_ALIGN;
  const hipStream_t hs = (hipStream_t)stream;
  if ((st = hip_status("rows", spa2::launch_rows(s, *m, hs))) != SPA2_OK) return st;
  if ((st = hip_status("cols", spa2::launch_cols(s, *m, hs))) != SPA2_OK) return st;
  return write_orders(s, *m, hs);
}

spa2_status spa2_fwd(const spa2_desc* desc, const void* q, const void* k, const void* v,
                     const spa2_blockmask* m, void* o, float* lse, float* o_f32,
                     void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !o || !lse) return SPA2_E_NULL;
  if (m && (!m->row_cnt || !m->row_idx)) return SPA2_E_NULL;
  if (!aligned16({q, k, v, o, o_f32}) || !aligned(lse, 4) || !lists_aligned(m)) return SPA2_E_ALIGN;
  return hip_status("fwd", spa2::launch_fwd(s, q, k, v, m ? m->row_cnt : nullptr,
                                            m ? m->row_idx : nullptr, m ? m->row_order : nullptr,
                                            o, lse, o_f32, (hipStream_t)stream));
}

spa2_status spa2_bwd_workspace_size(const spa2_desc* desc, size_t* bytes) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!bytes) return SPA2_E_NULL;
  *bytes = bwd_ws_bytes(s);
  return SPA2_OK;
}

size_t spa2_bwd_workspace_bytes(const spa2_desc* desc) {
  size_t bytes = 0;
  return spa2_bwd_workspace_size(desc, &bytes) == SPA2_OK ? bytes : 0;
}

spa2_status spa2_bwd(const spa2_desc* desc, const void* q, const void* k, const void* v,
                     const void* o, const float* o_f32, const float* lse, const void* dout,
                     const spa2_blockmask* m, void* dq, void* dk, void* dv, void* workspace,
                     size_t ws_bytes, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return SPA2_E_NULL;
  if (m && (!m->row_cnt || !m->row_idx || !m->col_cnt || !m->col_idx)) return SPA2_E_NULL;
  if (!workspace || ws_bytes < bwd_ws_bytes(s)) return SPA2_E_WORKSPACE;
  if (!aligned16({q, k, v, o, o_f32, dout, dq, dk, dv}) || !aligned4({lse, workspace}) ||
      !lists_aligned(m))
    return SPA2_E_ALIGN;
  return hip_status("bwd", spa2::launch_bwd(s, q, k, v, o, o_f32, lse, dout, m, dq, dk, dv,
                                            (float*)workspace, bwd_kmean(workspace, s),
                                            spa2::kBwdDqRow | spa2::kBwdDkdv, (hipStream_t)stream));
}

spa2_status spa2_bwd_noalloc(const spa2_desc* desc, const void* q, const void* k, const void* v,
                             const void* o, const float* o_f32, const float* lse,
                             const void* dout, const spa2_blockmask* m, void* dq, void* dk,
                             void* dv, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return SPA2_E_NULL;
  if (m && (!m->row_cnt || !m->row_idx || !m->col_cnt || !m->col_idx)) return SPA2_E_NULL;
  if (!aligned16({q, k, v, o, o_f32, dout, dq, dk, dv}) || !aligned4({lse}) || !lists_aligned(m))
    return SPA2_E_ALIGN;
  if (bwd_ws_bytes(s) > (size_t)SPA2_NOALLOC_SCRATCH_BYTES) return SPA2_E_SCRATCH;
  const hipStream_t hs = (hipStream_t)stream;
  void* ws = nullptr;
  if ((st = scratch_on_device(hs, &ws)) != SPA2_OK) return st;
  return hip_status("bwd_noalloc", spa2::launch_bwd(s, q, k, v, o, o_f32, lse, dout, m, dq, dk, dv,
                                                    (float*)ws, bwd_kmean(ws, s),
                                                    spa2::kBwdDqRow | spa2::kBwdDkdv, hs));
}

spa2_status spa2_bwd_dq_rowterm(const spa2_desc* desc, const void* q, const void* k,
                                const void* v, const void* o, const float* o_f32,
                                const float* lse, const void* dout,
                                const spa2_blockmask* m, void* workspace, size_t ws_bytes,
                                void* dq, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq) return SPA2_E_NULL;
  if (m && (!m->row_cnt || !m->row_idx)) return SPA2_E_NULL;
  if (!workspace || ws_bytes < bwd_ws_bytes(s)) return SPA2_E_WORKSPACE;
  if (!aligned16({q, k, v, o, o_f32, dout, dq}) || !aligned4({lse, workspace}) ||
      !lists_aligned(m))
    return SPA2_E_ALIGN;
  return hip_status("bwd_dq_rowterm",
                    spa2::launch_bwd(s, q, k, v, o, o_f32, lse, dout, m, dq, nullptr, nullptr,
                                     (float*)workspace, bwd_kmean(workspace, s), spa2::kBwdDqRow,
                                     (hipStream_t)stream));
}

spa2_status spa2_error_terms(const spa2_desc* desc, const float* o_sparse, const float* lse_sparse,
                             const float* o_dense, const float* lse_dense, double* terms,
                             float* tau, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!o_sparse || !lse_sparse || !o_dense || !lse_dense || !terms) return SPA2_E_NULL;
  if (!aligned16({o_sparse, o_dense}) || !aligned4({lse_sparse, lse_dense, tau}) ||
      !aligned(terms, 8))
    return SPA2_E_ALIGN;
  return hip_status("error_terms",
                    spa2::launch_error_terms(s, o_sparse, lse_sparse, o_dense, lse_dense, terms,
                                             tau, (hipStream_t)stream));
}

spa2_status spa2_bwd_prep(const spa2_desc* desc, const void* o, const float* o_f32,
                          const void* dout, float* dvec, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!o || !dout || !dvec) return SPA2_E_NULL;
  if (!aligned16({o, o_f32, dout}) || !aligned(dvec, 4)) return SPA2_E_ALIGN;
  return hip_status("bwd_prep", spa2::launch_bwd(s, nullptr, nullptr, nullptr, o, o_f32, nullptr, dout,
                                                 nullptr, nullptr, nullptr, nullptr, dvec,
                                                 nullptr, spa2::kBwdPrep, (hipStream_t)stream));
}

spa2_status spa2_bwd_dkdv(const spa2_desc* desc, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, const float* dvec,
                          const spa2_blockmask* m, void* dk, void* dv, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !lse || !dout || !dvec || !dk || !dv) return SPA2_E_NULL;
  if (m && (!m->col_cnt || !m->col_idx)) return SPA2_E_NULL;
  if (!aligned16({q, k, v, dout, dk, dv}) || !aligned4({lse, dvec}) || !lists_aligned(m))
    return SPA2_E_ALIGN;
  return hip_status("bwd_dkdv", spa2::launch_bwd(s, q, k, v, nullptr, nullptr, lse, dout, m, nullptr, dk,
                                                 dv, (float*)dvec, nullptr, spa2::kBwdDkdv,
                                                 (hipStream_t)stream));
}

spa2_status spa2_bwd_dq(const spa2_desc* desc, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, void* workspace, size_t ws_bytes,
                        const spa2_blockmask* m, void* dq, void* stream) {
  spa2::Shape s;
  spa2_status st = check_desc(desc, &s);
  if (st != SPA2_OK) return st;
  if (!q || !k || !v || !lse || !dout || !dq) return SPA2_E_NULL;
  if (m && (!m->row_cnt || !m->row_idx)) return SPA2_E_NULL;
  if (!workspace || ws_bytes < bwd_ws_bytes(s)) return SPA2_E_WORKSPACE;
  if (!aligned16({q, k, v, dout, dq}) || !aligned4({lse, workspace}) || !lists_aligned(m))
    return SPA2_E_ALIGN;
  return hip_status("bwd_dq", spa2::launch_bwd(s, q, k, v, nullptr, nullptr, lse, dout, m, dq, nullptr,
                                               nullptr, (float*)workspace, bwd_kmean(workspace, s),
                                               spa2::kBwdDq, (hipStream_t)stream));
}

}  // extern "C"
