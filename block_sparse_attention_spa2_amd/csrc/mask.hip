// Mask prediction on gfx950: block mean pooling, pooled scores, per-row hybrid
// Top-k U Top-p selection, compacted row and column lists.
//
// Method (SpargeAttention2, paper.rainbus.top summary, section "方法步骤详情", steps 1-3;
// the Top-k / Top-p rules of section "前置知识"; the union formula of "技术新颖性"):
//   q-bar_i = mean of query block i, k-bar_j = mean of key block j,
//   P-bar_i = softmax_j(q-bar_i . k-bar_j / sqrt(D)),
//   keep j iff j is among the first n_k blocks of row i's order (P-bar desc, index asc)
//   or its exclusive prefix mass in that order is below p.
// Everything in this file is double precision, so the mask is decided on the same values
// the float64 reference sees (bf16 block sums in double are exact).
#include <float.h>
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace spa2 {

// ------------------------------------------------------------------------------------
// Pooling: one workgroup per block. Threads read 16-byte chunks of the block's rows
// (coalesced), accumulate in double, and reduce the row groups through LDS.
// ------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   double* __restrict__ qbar,
                                                   double* __restrict__ kbar, int BH, int N, int BQ,
                                                   int BKV, int Tm, int Tn) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int TPR = D / EPC;              // threads per row
  constexpr int RP = 256 / TPR;             // rows in flight
  __shared__ double red[RP][D];

  int item = blockIdx.x;
  const T* src;
  double* dst;
  int b, nblk;
  if (item < BH * Tm) {
    src = q;
    dst = qbar;
    b = BQ;
    nblk = Tm;
  } else {
    item -= BH * Tm;
    src = k;
    dst = kbar;
    b = BKV;
    nblk = Tn;
  }
  const int bh = item / nblk, blk = item % nblk;
  const int lo = blk * b, hi = min(N, lo + b);
  const T* base = src + (size_t)bh * N * D;
  const int c = threadIdx.x % TPR, r0 = threadIdx.x / TPR;

  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  for (int r = lo + r0; r < hi; r += RP) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(base + (size_t)r * D + c * EPC);
    const T* x = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += (double)Elem<T>::to_f32(x[e]);
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[r0][c * EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int r = 0; r < RP; ++r) s += red[r][threadIdx.x];
    dst[((size_t)bh * nblk + blk) * D + threadIdx.x] = s / (double)(hi - lo);
  }
}

// ------------------------------------------------------------------------------------
// Pooled scores S-bar = q-bar k-bar^T / sqrt(D) on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64). Workgroup tile 64 x 64; wave w owns rows [16w, 16w+16).
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qbar,
                                                     const double* __restrict__ kbar,
                                                     double* __restrict__ scores, int Tm, int Tn,
                                                     int tiles_m, int tiles_n, double sqrt_d) {
  constexpr int KC = 32;       // reduction chunk
  constexpr int PITCH = KC + 1;  // doubles; odd pitch spreads rows over banks
  __shared__ double qs[64 * PITCH];
  __shared__ double ks[64 * PITCH];

  const int per_head = tiles_m * tiles_n;
  const int bh = blockIdx.x / per_head;
  const int tm = (blockIdx.x % per_head) / tiles_n, tn = blockIdx.x % tiles_n;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, g = l >> 4, c16 = l & 15;
  const double* qb = qbar + (size_t)bh * Tm * D;
  const double* kb = kbar + (size_t)bh * Tn * D;

  f64x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};

  for (int dc = 0; dc < D; dc += KC) {
    for (int e = threadIdx.x; e < 64 * KC; e += 256) {
      const int r = e / KC, cc = e % KC;
      const int qi = tm * 64 + r, kj = tn * 64 + r;
      qs[r * PITCH + cc] = qi < Tm ? qb[(size_t)qi * D + dc + cc] : 0.0;
      ks[r * PITCH + cc] = kj < Tn ? kb[(size_t)kj * D + dc + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int k4 = 0; k4 < KC; k4 += 4) {
      const double a = qs[(w * 16 + c16) * PITCH + k4 + g];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const double bv = ks[(ct * 16 + c16) * PITCH + k4 + g];
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // v_mfma_f64_16x16x4_f64 returns C[g + 4 e][l % 16] in element e of lane l (the fp32
  // results use 4 g + e instead).
  double* out = scores + (size_t)bh * Tm * Tn;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int col = tn * 64 + ct * 16 + c16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = tm * 64 + w * 16 + g + 4 * e;
      if (row < Tm && col < Tn) out[(size_t)row * Tn + col] = acc[ct][e] / sqrt_d;
    }
  }
}

// ------------------------------------------------------------------------------------
// Wave-level reductions and scans (64 lanes; no workgroup barrier involved).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_isum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// exclusive prefix over lanes, in lane order
__device__ __forceinline__ double wave_excl_scan(double x) {
  const int l = lane_id();
  double inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (l >= o) inc += y;
  }
  const double up = __shfl_up(inc, 1);
  return l == 0 ? 0.0 : up;  // no subtraction: the sum of the lanes before this one
}
__device__ __forceinline__ int wave_excl_iscan(int x) {
  const int l = lane_id();
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (l >= o) inc += y;
  }
  return inc - x;
}
// Orders this wave's LDS accesses: everything before is visible to every lane after.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// (value desc, index asc): true if (va, ia) comes before (vb, ib)
__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

// ------------------------------------------------------------------------------------
// Per-row selection: one wave per (head, query block); the workgroup's waves work on
// independent rows in their own LDS slices, so no workgroup barrier is needed.
//   1. (from scores) P-bar row = exp(s - max) / sum, optionally stored;
//   2. candidates: the largest threshold tau (found by bisection) such that the blocks
//      with P-bar >= tau number at least n_k and carry mass >= p (plus a rounding
//      margin). Those blocks are the first ranks of the (value desc, index asc) order,
//      and that prefix already reaches both the Top-k count and the Top-p mass, so
//      Top-k U Top-p lies inside it. Only the candidates need sorting (all blocks when
//      the row is flat enough);
//   3. bitonic sort of the candidate (P-bar, index) pairs into (value desc, index asc);
//   4. exclusive prefix sums in that order; n_p = #ranks whose prefix is below p;
//   5. keep the first L = max(n_k, n_p) ranks (Top-k U Top-p is a prefix of the order);
//   6. write the mask row and the ascending kept-index list.
// Dynamic LDS per wave: 21 * sort_n bytes (row, candidates, indices, flags).
// ------------------------------------------------------------------------------------
template <bool FROM_SCORES>
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ src,
                                                     double* __restrict__ pbar_out, int rows,
                                                     int Tn, int sort_n, int n_k, double p_frac,
                                                     uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ row_cnt,
                                                     int32_t* __restrict__ row_idx) {
  extern __shared__ __attribute__((aligned(16))) char sel_smem[];
  const int l = lane_id();
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (blockDim.x >> 6) + wave;  // (bh, i) flattened
  if (row >= rows) return;  // whole wave leaves; nothing below synchronises the workgroup
  char* mine = sel_smem + (size_t)wave * (((size_t)sort_n * 21 + 15) & ~(size_t)15);
  double* pv = reinterpret_cast<double*>(mine);  // the row, by block index
  double* val = pv + sort_n;                      // candidates, then sorted
  int* idx = reinterpret_cast<int*>(val + sort_n);
  uint8_t* keep = reinterpret_cast<uint8_t*>(idx + sort_n);
  const double* in = src + (size_t)row * Tn;

  // 1. the row's probabilities
  double vmax = -DBL_MAX;
  if (FROM_SCORES) {
    double mx = -DBL_MAX;
#pragma unroll 4
    for (int j = l; j < Tn; j += 64) {
      const double sv = in[j];
      pv[j] = sv;
      mx = fmax(mx, sv);
    }
    mx = wave_max(mx);
    double sm = 0.0;
    for (int j = l; j < Tn; j += 64) {
      const double e = exp(pv[j] - mx);
      pv[j] = e;
      sm += e;
    }
    sm = wave_sum(sm);
    for (int j = l; j < Tn; j += 64) {
      const double p = pv[j] / sm;
      pv[j] = p;
      vmax = fmax(vmax, p);
      if (pbar_out) pbar_out[(size_t)row * Tn + j] = p;
    }
  } else {
#pragma unroll 4
    for (int j = l; j < Tn; j += 64) {
      const double p = in[j];
      pv[j] = p;
      vmax = fmax(vmax, p);
    }
  }
  vmax = wave_max(vmax);
  wave_lds_sync();

  // 2. candidate threshold; lane l owns the contiguous block range [c_lo, c_hi)
  const int per = (Tn + 63) / 64;
  const int c_lo = min(Tn, l * per), c_hi = min(Tn, c_lo + per);
  const double need = p_frac > 0.0 ? p_frac + 1e-12 : 0.0;  // margin over summation order
  auto probe = [&](double tau, int& c, double& m) {
    int cl = 0;
    double ml = 0.0;
    for (int j = c_lo; j < c_hi; ++j) {
      const double v = pv[j];
      if (v >= tau) {
        ++cl;
        ml += v;
      }
    }
    c = wave_isum(cl);
    m = wave_sum(ml);
  };
  double tau = -1.0;  // every block
  {
    int c;
    double m;
    probe(0.0, c, m);
    if (c >= n_k && m >= need) {
      double lo = 0.0, hi = vmax * 2.0 + 1e-300;  // lo valid, hi not (no block reaches it)
      for (int it = 0; it < 40; ++it) {
        const double mid = 0.5 * (lo + hi);
        probe(mid, c, m);
        if (c >= n_k && m >= need) {
          lo = mid;
          if (c <= 64) break;  // few enough to sort
        } else {
          hi = mid;
        }
      }
      tau = lo;
    }
  }

  // gather the candidates in block order
  int cl = 0;
  for (int j = c_lo; j < c_hi; ++j) cl += pv[j] >= tau;
  int pos = wave_excl_iscan(cl);
  const int cand = wave_isum(cl);
  for (int j = c_lo; j < c_hi; ++j)
    if (pv[j] >= tau) {
      val[pos] = pv[j];
      idx[pos] = j;
      ++pos;
    }
  int sn = 2;
  while (sn < cand) sn <<= 1;
  for (int j = cand + l; j < sn; j += 64) {
    val[j] = -1.0;  // padding sorts after every probability
    idx[j] = Tn + j;
  }
  wave_lds_sync();

  // 3. bitonic sort into (value desc, index asc); each lane keeps up to four
  // compare-exchange pairs in flight per pass, without branches
  const int half = sn >> 1;
  for (int kk = 2; kk <= sn; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      const int lg = __builtin_ctz(jj);
      for (int base = 0; base < half; base += 256) {
        int i1[4], i2[4];
        double v1[4], v2[4];
        int x1[4], x2[4];
        bool act[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pr = base + q * 64 + l;
          act[q] = pr < half;
          i1[q] = ((pr >> lg) << (lg + 1)) + (pr & (jj - 1));
          i2[q] = i1[q] + jj;
          if (act[q]) {
            v1[q] = val[i1[q]];
            v2[q] = val[i2[q]];
            x1[q] = idx[i1[q]];
            x2[q] = idx[i2[q]];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (!act[q]) continue;
          const bool fwd = (i1[q] & kk) == 0;  // this half-block runs in the primary order
          const bool b21 = before(v2[q], x2[q], v1[q], x1[q]);
          const bool swap = fwd ? b21 : !b21;   // pairs never tie: indices differ
          val[i1[q]] = swap ? v2[q] : v1[q];
          val[i2[q]] = swap ? v1[q] : v2[q];
          idx[i1[q]] = swap ? x2[q] : x1[q];
          idx[i2[q]] = swap ? x1[q] : x2[q];
        }
      }
      wave_lds_sync();
    }
  }

  // 4. exclusive prefix mass over the candidate ranks; lane l owns a contiguous range
  const int rper = (cand + 63) / 64;
  const int r_lo = min(cand, l * rper), r_hi = min(cand, r_lo + rper);
  double local = 0.0;
  for (int r = r_lo; r < r_hi; ++r) local += val[r];
  double run = wave_excl_scan(local);
  int below = 0;
  for (int r = r_lo; r < r_hi; ++r) {
    if (run < p_frac) ++below;
    run += val[r];
  }
  const int n_p = wave_isum(below);
  const int L = min(cand, max(n_k, n_p));  // cand >= both by the choice of tau

  // 5. flag the first L ranks
  for (int j = l; j < Tn; j += 64) keep[j] = 0;
  wave_lds_sync();
  for (int r = l; r < L; r += 64) keep[idx[r]] = 1;
  wave_lds_sync();

  // 6. mask row and ascending compaction
  uint8_t* mrow = mask + (size_t)row * Tn;
  for (int j = l; j < Tn; j += 64) mrow[j] = keep[j];
  int cnt = 0;
  for (int j = c_lo; j < c_hi; ++j) cnt += keep[j];
  int opos = wave_excl_iscan(cnt);
  int32_t* out = row_idx + (size_t)row * Tn;
  for (int j = c_lo; j < c_hi; ++j)
    if (keep[j]) out[opos++] = j;
  if (l == 0) row_cnt[row] = L;
}

// Row lists from a caller-filled mask (one thread per row).
__global__ void rows_kernel(const uint8_t* __restrict__ mask, int rows, int Tn,
                            int32_t* __restrict__ row_cnt, int32_t* __restrict__ row_idx) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const uint8_t* m = mask + (size_t)r * Tn;
  int32_t* out = row_idx + (size_t)r * Tn;
  int c = 0;
  for (int j = 0; j < Tn; ++j)
    if (m[j]) out[c++] = j;
  row_cnt[r] = c;
}

// Column lists: a workgroup covers 16 key blocks (columns) of one head; its 256 threads
// are 16 columns x 16 slices of the query-block rows. Each thread counts its slice, the
// counts are scanned over slices in LDS, and a second pass writes the ascending indices.
__global__ __launch_bounds__(256) void cols_kernel(const uint8_t* __restrict__ mask, int Tm,
                                                   int Tn, int col_groups,
                                                   int32_t* __restrict__ col_cnt,
                                                   int32_t* __restrict__ col_idx) {
  __shared__ int cnts[16][17];
  const int bh = blockIdx.x / col_groups;
  const int c = threadIdx.x & 15, part = threadIdx.x >> 4;
  const int j = (blockIdx.x % col_groups) * 16 + c;
  const int rp = (Tm + 15) / 16;
  const int i0 = min(Tm, part * rp), i1 = min(Tm, i0 + rp);
  const uint8_t* m = mask + (size_t)bh * Tm * Tn;
  int n = 0;
  if (j < Tn)
    for (int i = i0; i < i1; ++i) n += m[(size_t)i * Tn + j];
  cnts[part][c] = n;
  __syncthreads();
  int off = 0;
  for (int p = 0; p < part; ++p) off += cnts[p][c];
  if (j < Tn) {
    int32_t* out = col_idx + ((size_t)bh * Tn + j) * Tm;
    for (int i = i0; i < i1; ++i)
      if (m[(size_t)i * Tn + j]) out[off++] = i;
    if (part == 15) col_cnt[(size_t)bh * Tn + j] = off;
  }
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar,
                       hipStream_t st) {
  const dim3 grid(s.BH() * (s.Tm + s.Tn));
#define SPA2_POOL(T, D)                                                                      \
  pool_kernel<T, D><<<grid, 256, 0, st>>>((const T*)q, (const T*)k, qbar, kbar, s.BH(), s.N, \
                                          s.BQ, s.BKV, s.Tm, s.Tn)
  if (s.dtype == SPA2_BF16) {
    if (s.D == 64) SPA2_POOL(bf16, 64); else SPA2_POOL(bf16, 128);
  } else {
    if (s.D == 64) SPA2_POOL(float, 64); else SPA2_POOL(float, 128);
  }
#undef SPA2_POOL
  return hipGetLastError();
}

hipError_t launch_scores(const Shape& s, const double* qbar, const double* kbar, double* scores,
                         hipStream_t st) {
  const int tm = (s.Tm + 63) / 64, tn = (s.Tn + 63) / 64;
  const dim3 grid(s.BH() * tm * tn);
  const double sqrt_d = sqrt((double)s.D);
  if (s.D == 64)
    scores_kernel<64><<<grid, 256, 0, st>>>(qbar, kbar, scores, s.Tm, s.Tn, tm, tn, sqrt_d);
  else
    scores_kernel<128><<<grid, 256, 0, st>>>(qbar, kbar, scores, s.Tm, s.Tn, tm, tn, sqrt_d);
  return hipGetLastError();
}

static int sort_size(int tn) {
  int n = 2;
  while (n < tn) n <<= 1;
  return n;
}

hipError_t launch_select(const Shape& s, const double* src, bool from_scores, double* pbar_out,
                         int n_k, double p_frac, const spa2_blockmask& m, hipStream_t st) {
  const int sn = sort_size(s.Tn);
  const size_t per_wave = ((size_t)sn * 21 + 15) & ~(size_t)15;  // 2 doubles + int + byte
  // rows per workgroup: up to 4 waves, as many as fit in 160 KB of LDS
  const int wpg = (int)std::max<size_t>(1, std::min<size_t>(4, (160 * 1024) / per_wave));
  const int rows = s.BH() * s.Tm;
  const dim3 grid((rows + wpg - 1) / wpg);
  const size_t lds = per_wave * wpg;
  if (from_scores) {
    hipFuncSetAttribute((const void*)select_kernel<true>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    select_kernel<true><<<grid, 64 * wpg, lds, st>>>(src, pbar_out, rows, s.Tn, sn, n_k, p_frac,
                                                     m.mask, m.row_cnt, m.row_idx);
  } else {
    hipFuncSetAttribute((const void*)select_kernel<false>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    select_kernel<false><<<grid, 64 * wpg, lds, st>>>(src, nullptr, rows, s.Tn, sn, n_k, p_frac,
                                                      m.mask, m.row_cnt, m.row_idx);
  }
  return hipGetLastError();
}

hipError_t launch_rows(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int rows = s.BH() * s.Tm;
  rows_kernel<<<(rows + 255) / 256, 256, 0, st>>>(m.mask, rows, s.Tn, m.row_cnt, m.row_idx);
  return hipGetLastError();
}

hipError_t launch_cols(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int groups = (s.Tn + 15) / 16;
  cols_kernel<<<s.BH() * groups, 256, 0, st>>>(m.mask, s.Tm, s.Tn, groups, m.col_cnt, m.col_idx);
  return hipGetLastError();
}

}  // namespace spa2
