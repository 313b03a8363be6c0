// Internal launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spa2.h"

namespace spa2 {

struct Shape {
  int B, H, N, D, BQ, BKV, dtype;
  int Tm, Tn;   // query / key block counts
  int BH() const { return B * H; }
  // The attention kernels work on tiles of at most 128 query rows and 64 keys; a larger
  // mask block (BQ = 256, BKV = 128) is two consecutive tiles.
  int bq_tile() const { return BQ > 128 ? 128 : BQ; }
  int bkv_tile() const { return BKV > 64 ? 64 : BKV; }
  int qsub() const { return BQ > 128 ? 1 : 0; }  // log2(BQ / bq_tile())
  int ksub() const { return BKV > 64 ? 1 : 0; }  // log2(BKV / bkv_tile())
};

// Largest key-block count per row: the selection kernel holds a row in registers, 64 blocks
// per lane at most.
constexpr int kMaxTn = 4096;

// q-bar / k-bar rows are `pitch` doubles apart (D for the public layout; the mask
// workspace uses kPoolPitch(D))
hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar,
                       int pitch, hipStream_t st);
hipError_t launch_scores(const Shape& s, const double* qbar, const double* kbar, int pitch,
                         double* scores, hipStream_t st);
constexpr int kPoolPitch(int D) { return D + 2; }
// from_scores: src holds raw pooled scores (softmax applied here); else src holds P-bar.
hipError_t launch_select(const Shape& s, const double* src, bool from_scores, double* pbar_out,
                         int n_k, double p_frac, const spa2_blockmask& m, hipStream_t st);
// A scheduling order to list: the kept counts of `items` lists (clamped to [0, maxc]),
// written as a permutation to `order`; per_head > 0 groups the items head by head
// (per_head items per head), 0 sorts the whole range by count; with per_head > 0, items
// whose count reaches hoist (> 0) come first.
struct OrderJob {
  const int32_t* cnt;
  int items;
  int maxc;
  int per_head;
  int hoist;
  int32_t* order;
};
// One launch for up to two orders (either pointer may be NULL).
hipError_t launch_orders(const OrderJob* a, const OrderJob* b, hipStream_t st);
hipError_t launch_rows(const Shape& s, const spa2_blockmask& m, hipStream_t st);
hipError_t launch_cols(const Shape& s, const spa2_blockmask& m, hipStream_t st);

hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const int32_t* row_cnt, const int32_t* row_idx, const int32_t* row_order,
                      void* o, float* lse, float* o_f32, hipStream_t st);
hipError_t launch_error_terms(const Shape& s, const float* os, const float* ls, const float* od,
                              const float* ld, double* terms, float* tau, hipStream_t st);

// stage bits for launch_bwd
// kBwdDqRow: the dQ pass that also computes the row term (instead of kBwdPrep), run
// before the dK/dV pass.
constexpr int kBwdPrep = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdDqRow = 8, kBwdAll = 7;
// Key tiles of the dQ pass per head (the bf16 pass keeps one mean key per tile).
inline int bwd_key_tiles(const Shape& s) { return s.Tn << s.ksub(); }
// Bytes of the per-tile mean keys (bf16 [B*H, key tiles, D]); none for fp32.
inline size_t bwd_kmean_bytes(const Shape& s) {
  return s.dtype == SPA2_BF16 ? (size_t)s.BH() * bwd_key_tiles(s) * s.D * 2 : 0;
}
// dvec: the row term, float [B*H*N]; kmean: bwd_kmean_bytes, 16-byte aligned (the dQ
// stages of a bf16 backward write it first, then read it)
hipError_t launch_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                      const float* o_f32, const float* lse, const void* dout, const spa2_blockmask* m, void* dq,
                      void* dk, void* dv, float* dvec, void* kmean, int stages, hipStream_t st);

}  // namespace spa2
