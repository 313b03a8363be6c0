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
// Workgroup reductions / scan over 256 threads (4 waves).
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

__device__ double block_max(double x, double* scratch) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = fmax(fmax(scratch[0], scratch[1]), fmax(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}
__device__ double block_sum(double x, double* scratch) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
  __syncthreads();
  return r;
}
__device__ int block_isum(int x, int* scratch) {
  x = wave_isum(x);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  const int r = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return r;
}
// Exclusive prefix over threads in thread order (double).
__device__ double block_excl_scan(double x, double* scratch) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (l >= o) inc += y;
  }
  if (l == 63) scratch[w] = inc;
  const double up = __shfl_up(inc, 1);
  const double excl = l == 0 ? 0.0 : up;  // exclusive within the wave, no subtraction
  __syncthreads();
  double before = 0.0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  __syncthreads();
  return before + excl;
}
__device__ int block_excl_iscan(int x, int* scratch) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (l >= o) inc += y;
  }
  if (l == 63) scratch[w] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  __syncthreads();
  return before + inc - x;
}

// (value desc, index asc): true if (va, ia) comes before (vb, ib)
__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ------------------------------------------------------------------------------------
// Per-row selection: one workgroup per (head, query block).
//   1. (from scores) P-bar row = exp(s - max) / sum, optionally stored;
//   2. bitonic sort of (P-bar, index) pairs in LDS into (value desc, index asc) order;
//   3. exclusive prefix sums in that order; n_p = #ranks whose prefix is below p;
//   4. keep the first L = max(n_k, n_p) ranks (Top-k U Top-p is a prefix of the order);
//   5. write the mask row and the ascending kept-index list.
// Dynamic LDS: sort_n doubles + sort_n ints + sort_n bytes.
// ------------------------------------------------------------------------------------
template <bool FROM_SCORES>
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ src,
                                                     double* __restrict__ pbar_out, int Tm, int Tn,
                                                     int sort_n, int n_k, double p_frac,
                                                     uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ row_cnt,
                                                     int32_t* __restrict__ row_idx) {
  extern __shared__ __attribute__((aligned(16))) char sel_smem[];
  double* val = reinterpret_cast<double*>(sel_smem);
  int* idx = reinterpret_cast<int*>(val + sort_n);
  uint8_t* keep = reinterpret_cast<uint8_t*>(idx + sort_n);
  __shared__ double dscr[4];
  __shared__ int iscr[4];

  const int row = blockIdx.x;  // (bh, i) flattened
  const int tid = threadIdx.x;
  const double* in = src + (size_t)row * Tn;

  // 1. the row's probabilities
  if (FROM_SCORES) {
    double mx = -DBL_MAX;
    for (int j = tid; j < Tn; j += 256) mx = fmax(mx, in[j]);
    mx = block_max(mx, dscr);
    double sm = 0.0;
    for (int j = tid; j < Tn; j += 256) {
      const double e = exp(in[j] - mx);
      val[j] = e;
      sm += e;
    }
    sm = block_sum(sm, dscr);
    for (int j = tid; j < Tn; j += 256) {
      const double pv = val[j] / sm;
      val[j] = pv;
      if (pbar_out) pbar_out[(size_t)row * Tn + j] = pv;
    }
  } else {
    for (int j = tid; j < Tn; j += 256) val[j] = in[j];
  }
  for (int j = tid; j < sort_n; j += 256) {
    if (j >= Tn) val[j] = -1.0;  // padding sorts after every probability
    idx[j] = j;
  }
  __syncthreads();

  // 2. bitonic sort into (value desc, index asc)
  const int half = sort_n >> 1;
  for (int kk = 2; kk <= sort_n; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int pr = tid; pr < half; pr += 256) {
        const int i1 = 2 * jj * (pr / jj) + (pr % jj);
        const int i2 = i1 + jj;
        const double v1 = val[i1], v2 = val[i2];
        const int x1 = idx[i1], x2 = idx[i2];
        const bool fwd = (i1 & kk) == 0;  // this half-block is ordered in the primary order
        const bool swap = fwd ? before(v2, x2, v1, x1) : before(v1, x1, v2, x2);
        if (swap) {
          val[i1] = v2;
          val[i2] = v1;
          idx[i1] = x2;
          idx[i2] = x1;
        }
      }
      __syncthreads();
    }
  }

  // 3. exclusive prefix mass over ranks 0 .. Tn-1; thread t owns a contiguous rank range
  const int per = (Tn + 255) / 256;
  const int r_lo = min(Tn, tid * per), r_hi = min(Tn, r_lo + per);
  double local = 0.0;
  for (int r = r_lo; r < r_hi; ++r) local += val[r];
  double run = block_excl_scan(local, dscr);
  int below = 0;
  for (int r = r_lo; r < r_hi; ++r) {
    if (run < p_frac) ++below;
    run += val[r];
  }
  const int n_p = block_isum(below, iscr);
  const int L = max(n_k, n_p);

  // 4. flag the first L ranks
  for (int j = tid; j < Tn; j += 256) keep[j] = 0;
  __syncthreads();
  for (int r = tid; r < L; r += 256) keep[idx[r]] = 1;
  __syncthreads();

  // 5. mask row and ascending compaction
  uint8_t* mrow = mask + (size_t)row * Tn;
  for (int j = tid; j < Tn; j += 256) mrow[j] = keep[j];
  const int c_lo = min(Tn, tid * per), c_hi = min(Tn, c_lo + per);
  int cnt = 0;
  for (int j = c_lo; j < c_hi; ++j) cnt += keep[j];
  int pos = block_excl_iscan(cnt, iscr);
  int32_t* out = row_idx + (size_t)row * Tn;
  for (int j = c_lo; j < c_hi; ++j)
    if (keep[j]) out[pos++] = j;
  if (tid == 0) row_cnt[row] = L;
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

// Column lists: thread per key block; reads mask rows coalesced across threads.
__global__ void cols_kernel(const uint8_t* __restrict__ mask, int Tm, int Tn, int col_groups,
                            int32_t* __restrict__ col_cnt, int32_t* __restrict__ col_idx) {
  const int bh = blockIdx.x / col_groups;
  const int j = (blockIdx.x % col_groups) * blockDim.x + threadIdx.x;
  if (j >= Tn) return;
  const uint8_t* m = mask + (size_t)bh * Tm * Tn;
  int32_t* out = col_idx + ((size_t)bh * Tn + j) * Tm;
  int c = 0;
  for (int i = 0; i < Tm; ++i)
    if (m[(size_t)i * Tn + j]) out[c++] = i;
  col_cnt[(size_t)bh * Tn + j] = c;
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
  const size_t lds = (size_t)sn * (sizeof(double) + sizeof(int) + 1);
  const dim3 grid(s.BH() * s.Tm);
  if (from_scores)
    select_kernel<true><<<grid, 256, lds, st>>>(src, pbar_out, s.Tm, s.Tn, sn, n_k, p_frac,
                                                m.mask, m.row_cnt, m.row_idx);
  else
    select_kernel<false><<<grid, 256, lds, st>>>(src, nullptr, s.Tm, s.Tn, sn, n_k, p_frac,
                                                 m.mask, m.row_cnt, m.row_idx);
  return hipGetLastError();
}

hipError_t launch_rows(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int rows = s.BH() * s.Tm;
  rows_kernel<<<(rows + 255) / 256, 256, 0, st>>>(m.mask, rows, s.Tn, m.row_cnt, m.row_idx);
  return hipGetLastError();
}

hipError_t launch_cols(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int groups = (s.Tn + 255) / 256;
  cols_kernel<<<s.BH() * groups, 256, 0, st>>>(m.mask, s.Tm, s.Tn, groups, m.col_cnt, m.col_idx);
  return hipGetLastError();
}

}  // namespace spa2
