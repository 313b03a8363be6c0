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
                                                   int BKV, int Tm, int Tn, int pitch) {
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
    dst[((size_t)bh * nblk + blk) * pitch + threadIdx.x] = s / (double)(hi - lo);
  }
}

// ------------------------------------------------------------------------------------
// Pooled scores S-bar = q-bar k-bar^T / sqrt(D) on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64). One workgroup per 64 x 64 tile of one head (workgroups in
// XCD-contiguous order, so an XCD's L2 holds the pooled vectors of its heads); wave w
// computes rows 16 w .. 16 w + 15 against the 64 columns (four MFMA tiles). The reduction
// runs over chunks of 16 dims: each chunk of q-bar and k-bar rows is loaded once per
// workgroup (four threads per row, 32 contiguous bytes each) into a double-buffered LDS
// stage while the previous chunk's products run. `pitch` (doubles) is the row stride of
// q-bar and k-bar: rows exactly 1 KB apart meet in a few L2 channels, and a pitch of
// D + 2 spreads them. Rows and keys past the matrix read a clamped row and are not stored.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qbar,
                                                     const double* __restrict__ kbar,
                                                     double* __restrict__ scores, int Tm, int Tn,
                                                     int pitch, int tiles_m, int tiles_n,
                                                     double sqrt_d) {
  constexpr int KC = 16;      // dims per chunk
  constexpr int NC = D / KC;  // chunks
  constexpr int LP = KC + 2;  // LDS row pitch in doubles (spreads rows over the banks)
  __shared__ double sa[2][64 * LP];
  __shared__ double sb[2][64 * LP];
  const int tile = xcd_item(blockIdx.x, gridDim.x);
  const int per_head = tiles_m * tiles_n;
  const int bh = tile / per_head;
  const int tm = (tile % per_head) / tiles_n, tn = tile % tiles_n;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // loader: thread -> row lr of both tiles, dims lp .. lp + 3 of each chunk
  const int lr = tid >> 2, lp = (tid & 3) * 4;
  const double* qrow = qbar + ((size_t)bh * Tm + min(tm * 64 + lr, Tm - 1)) * pitch + lp;
  const double* krow = kbar + ((size_t)bh * Tn + min(tn * 64 + lr, Tn - 1)) * pitch + lp;
  f64x2 ra0, ra1, rb0, rb1;
  auto gload = [&](int c) {
    ra0 = *reinterpret_cast<const f64x2*>(qrow + c * KC);
    ra1 = *reinterpret_cast<const f64x2*>(qrow + c * KC + 2);
    rb0 = *reinterpret_cast<const f64x2*>(krow + c * KC);
    rb1 = *reinterpret_cast<const f64x2*>(krow + c * KC + 2);
  };
  auto sstore = [&](int buf) {
    double* a = sa[buf] + lr * LP + lp;
    double* b = sb[buf] + lr * LP + lp;
    a[0] = ra0[0]; a[1] = ra0[1]; a[2] = ra1[0]; a[3] = ra1[1];
    b[0] = rb0[0]; b[1] = rb0[1]; b[2] = rb1[0]; b[3] = rb1[1];
  };
  gload(0);
  sstore(0);
  __syncthreads();

  f64x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int c = 0; c < NC; ++c) {
    const int buf = c & 1;
    if (c + 1 < NC) gload(c + 1);  // in flight during this chunk's products
    const double* A = sa[buf] + (w * 16 + c16) * LP + g;
    const double* Bm = sb[buf] + c16 * LP + g;
#pragma unroll
    for (int st = 0; st < KC / 4; ++st) {
      const double av = A[4 * st];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, Bm[ct * 16 * LP + 4 * st], acc[ct], 0, 0, 0);
    }
    if (c + 1 < NC) sstore(buf ^ 1);  // that stage was last read before the previous barrier
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
// Cross-lane moves on the VALU (no LDS round trip) for the selection's inner loop.
// DPP quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror; then the 16- and
// 32-lane swaps. Each step pairs lanes symmetrically, so every lane ends with the same
// result.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
template <bool W32>
__device__ __forceinline__ double swap_max_f64(double x) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
  const auto rl = W32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                      : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto rh = W32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                      : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const double a = __builtin_bit_cast(double, ((unsigned long long)(unsigned)rh[0] << 32) | (unsigned)rl[0]);
  const double b = __builtin_bit_cast(double, ((unsigned long long)(unsigned)rh[1] << 32) | (unsigned)rl[1]);
  return fmax(a, b);
}
__device__ __forceinline__ double wave_max_fast(double x) {
  x = fmax(x, dpp_f64<0xB1>(x));   // lane ^ 1
  x = fmax(x, dpp_f64<0x4E>(x));   // lane ^ 2
  x = fmax(x, dpp_f64<0x141>(x));  // mirror within 8
  x = fmax(x, dpp_f64<0x140>(x));  // mirror within 16
  x = swap_max_f64<false>(x);      // lanes l, l ^ 16
  return swap_max_f64<true>(x);    // lanes l, l ^ 32
}
__device__ __forceinline__ int wave_min_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
// Ordering key of a window head: the high word of a positive double (sign, exponent
// and the top 20 mantissa bits, which order like the value), 0 for the empty slot (-1).
__device__ __forceinline__ unsigned key_hi(double x) {
  return x > 0.0 ? (unsigned)(__builtin_bit_cast(unsigned long long, x) >> 32) : 0u;
}
__device__ __forceinline__ unsigned max_dpp_u32_step(unsigned x, unsigned y) { return x > y ? x : y; }
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
  x = max_dpp_u32_step(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
  x = max_dpp_u32_step(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
  x = max_dpp_u32_step(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
  x = max_dpp_u32_step(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max_dpp_u32_step((unsigned)r16[0], (unsigned)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max_dpp_u32_step((unsigned)r32[0], (unsigned)r32[1]);
}
// A double from lane `src` (wave-uniform) to every lane.
__device__ __forceinline__ double readlane_f64(double x, int src) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, src);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), src);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// ------------------------------------------------------------------------------------
// Per-row selection: one wave per (head, query block), the row held in registers
// (lane l owns blocks j = l + 64 t, t < PER), no LDS.
//   1. (from scores) P-bar row = exp(s - max) / sum, optionally stored;
//   2. each lane keeps a small window: its W largest blocks in (value desc, index asc)
//      order, refilled from its remaining blocks when used up;
//   3. the row's order is produced one rank at a time: the largest window head over the
//      wave (ties: the smallest block index) is rank r. Rank r is kept iff r < n_k or
//      its exclusive prefix mass e_r (the running sum of the values already taken, in
//      rank order) is below p. Both tests fail for good once they fail, so the first
//      rejected rank ends the row: Top-k U Top-p is the prefix taken so far;
//   4. mask row and the ascending kept-index list from the lanes' kept bits.
// ------------------------------------------------------------------------------------
template <int PER, bool FROM_SCORES>
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ src,
                                                     double* __restrict__ pbar_out, int rows,
                                                     int Tn, int n_k, double p_frac,
                                                     uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ row_cnt,
                                                     int32_t* __restrict__ row_idx) {
  constexpr int W = 4;  // window length
  const int l = lane_id();
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);  // (bh, i) flattened
  if (row >= rows) return;  // whole wave leaves; nothing below synchronises the workgroup
  const int tcnt = (Tn + 63) / 64;  // rounds that hold any block (wave-uniform)
  const double* in = src + (size_t)row * Tn;

  // 1. the row's probabilities; slots past the row hold -1
  double v[PER];
  if (FROM_SCORES) {
    double mx = -DBL_MAX;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      v[t] = -DBL_MAX;
      if (t < tcnt && l + 64 * t < Tn) v[t] = in[l + 64 * t];
      mx = fmax(mx, v[t]);
    }
    mx = wave_max(mx);
    double sm = 0.0;
#pragma unroll
    for (int t = 0; t < PER; ++t)
      if (t < tcnt && l + 64 * t < Tn) {
        v[t] = exp(v[t] - mx);
        sm += v[t];
      }
    sm = wave_sum(sm);
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      if (t < tcnt && l + 64 * t < Tn) {
        v[t] = v[t] / sm;
        if (pbar_out) pbar_out[(size_t)row * Tn + l + 64 * t] = v[t];
      } else {
        v[t] = -1.0;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < PER; ++t) v[t] = (t < tcnt && l + 64 * t < Tn) ? in[l + 64 * t] : -1.0;
  }

  // 2. window: the lane's W first blocks in order among those after (lv, lt)
  double wv[W];
  int wt[W];
  auto refill = [&](double lv, int lt) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
      wv[k] = -1.0;
      wt[k] = 0;
    }
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      if (t >= tcnt) break;
      const double x = v[t];
      const bool after = (x < lv) | ((x == lv) & (t > lt));
      if (after && x > wv[W - 1]) {  // strictly larger: equal values keep index order
        wv[W - 1] = x;
        wt[W - 1] = t;
#pragma unroll
        for (int k = W - 1; k > 0; --k) {
          if (wv[k] > wv[k - 1]) {
            const double tv = wv[k];
            wv[k] = wv[k - 1];
            wv[k - 1] = tv;
            const int tt = wt[k];
            wt[k] = wt[k - 1];
            wt[k - 1] = tt;
          }
        }
      }
    }
  };
  refill(2.0, -1);  // every block (all values are below 2)

  // 3. ranks in order until the first rejected one. The wave maximum is taken first on
  // the high 32 bits of the window heads (positive doubles order like their bit patterns,
  // so one DPP max per step); if a single lane holds that maximum it owns the rank.
  // Otherwise (equal high words, or nothing positive left) the double maximum and the
  // index rule for equal values decide.
  unsigned long long kept = 0;  // bit t: block l + 64 t is kept
  double prefix = 0.0;          // e_r, summed in rank order
  int rank = 0;
  unsigned key = key_hi(wv[0]);
  // rank, prefix, m and owner are wave-uniform (read from one lane), so the loop and its
  // exits are scalar control flow
  for (;;) {
    if (rank >= n_k && !(prefix < p_frac)) break;  // rank r fails both tests
    const unsigned mk = __builtin_amdgcn_readfirstlane(wave_max_u32(key));
    const unsigned long long cand = __builtin_amdgcn_ballot_w64(key == mk);
    double m;
    int owner;
    if (mk != 0u && (cand & (cand - 1)) == 0) {
      owner = __builtin_ctzll(cand);
      m = readlane_f64(wv[0], owner);
    } else {
      m = readlane_f64(wave_max_fast(wv[0]), 0);
      if (m < 0.0) break;  // every block is kept
      const unsigned long long tie = __builtin_amdgcn_ballot_w64(wv[0] == m);
      owner = __builtin_ctzll(tie);
      if ((tie & (tie - 1)) != 0)  // equal values in several lanes: smallest block index
        owner = __builtin_amdgcn_readfirstlane(wave_min_int(wv[0] == m ? l + 64 * wt[0] : INT_MAX)) & 63;
    }
    if (l == owner) {
      const int lt = wt[0];
      kept |= 1ull << lt;
#pragma unroll
      for (int k = 0; k < W - 1; ++k) {
        wv[k] = wv[k + 1];
        wt[k] = wt[k + 1];
      }
      wv[W - 1] = -1.0;
      if (wv[0] < 0.0) refill(m, lt);
      key = key_hi(wv[0]);
    }
    prefix += m;
    ++rank;
  }

  // 4. mask row and ascending compaction (round t holds blocks 64 t .. 64 t + 63)
  uint8_t* mrow = mask + (size_t)row * Tn;
  int32_t* out = row_idx + (size_t)row * Tn;
  int base = 0;
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    if (t >= tcnt) break;
    const int j = l + 64 * t;
    const bool kb = (kept >> t) & 1;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(kb);
    if (j < Tn) mrow[j] = kb;
    if (kb) {
      const int pos = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
      out[base + pos] = j;
    }
    base += __builtin_popcountll(bal);
  }
  if (l == 0) row_cnt[row] = rank;
}

// Row lists from a caller-filled mask: one wave per row, 64 blocks per step; a ballot of
// the step's bytes (nonzero = kept) places every kept block after those of earlier steps.
__global__ __launch_bounds__(256) void rows_kernel(const uint8_t* __restrict__ mask, int rows,
                                                   int Tn, int32_t* __restrict__ row_cnt,
                                                   int32_t* __restrict__ row_idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves; no barrier below
  const int l = lane_id();
  const uint8_t* mr = mask + (size_t)row * Tn;
  int32_t* out = row_idx + (size_t)row * Tn;
  int base = 0;
  for (int t0 = 0; t0 < Tn; t0 += 64) {
    const int j = t0 + l;
    const bool kb = j < Tn && mr[j] != 0;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(kb);
    if (kb)
      out[base + __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                           __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0))] = j;
    base += __builtin_popcountll(bal);
  }
  if (l == 0) row_cnt[row] = base;
}

// Column lists: a workgroup covers 64 key blocks (columns) of one head, one column per
// lane; its eight waves take contiguous slices of the query blocks (rows), so every row's
// 64 mask bytes are one coalesced load. Each wave counts its slice's kept rows per column,
// the counts are scanned over the slices in LDS, and a second pass over the slice writes
// the kept rows after those of the earlier slices: the lists come out ascending.
__global__ __launch_bounds__(512) void cols_kernel(const uint8_t* __restrict__ mask, int Tm,
                                                   int Tn, int col_groups,
                                                   int32_t* __restrict__ col_cnt,
                                                   int32_t* __restrict__ col_idx) {
  constexpr int NWV = 8;  // waves (row slices) per workgroup
  constexpr int U = 16;   // rows loaded together
  __shared__ int cnts[NWV][64];
  const int bh = blockIdx.x / col_groups;
  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = (blockIdx.x % col_groups) * 64 + l;
  const bool col_ok = j < Tn;
  const int per = (Tm + NWV - 1) / NWV;
  const int i0 = min(Tm, w * per), i1 = min(Tm, i0 + per);
  const uint8_t* mc = mask + (size_t)bh * Tm * Tn + j;  // column j, row 0

  int n = 0;
  if (col_ok) {
    for (int ib = i0; ib < i1; ib += U) {
      // unconditional loads (row clamped into the slice) so all U are in flight together
      uint8_t b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = mc[(size_t)min(ib + u, i1 - 1) * Tn];
#pragma unroll
      for (int u = 0; u < U; ++u) n += (ib + u < i1) & (b[u] != 0);
    }
  }
  cnts[w][l] = n;
  __syncthreads();
  int off = 0;
  for (int v = 0; v < w; ++v) off += cnts[v][l];
  if (col_ok) {
    int32_t* out = col_idx + ((size_t)bh * Tn + j) * Tm;
    for (int ib = i0; ib < i1; ib += U) {
      uint8_t b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = mc[(size_t)min(ib + u, i1 - 1) * Tn];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((ib + u < i1) & (b[u] != 0)) out[off++] = ib + u;
    }
    if (w == NWV - 1) col_cnt[(size_t)bh * Tn + j] = off;
  }
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar,
                       int pitch, hipStream_t st) {
  const dim3 grid(s.BH() * (s.Tm + s.Tn));
#define SPA2_POOL(T, D)                                                                      \
  pool_kernel<T, D><<<grid, 256, 0, st>>>((const T*)q, (const T*)k, qbar, kbar, s.BH(), s.N, \
                                          s.BQ, s.BKV, s.Tm, s.Tn, pitch)
  if (s.dtype == SPA2_BF16) {
    if (s.D == 64) SPA2_POOL(bf16, 64); else SPA2_POOL(bf16, 128);
  } else {
    if (s.D == 64) SPA2_POOL(float, 64); else SPA2_POOL(float, 128);
  }
#undef SPA2_POOL
  return hipGetLastError();
}

hipError_t launch_scores(const Shape& s, const double* qbar, const double* kbar, int pitch,
                         double* scores, hipStream_t st) {
  const int tm = (s.Tm + 63) / 64, tn = (s.Tn + 63) / 64;
  const dim3 grid(s.BH() * tm * tn);  // one workgroup per 64 x 64 tile
  const double sqrt_d = sqrt((double)s.D);
  if (s.D == 64)
    scores_kernel<64><<<grid, 256, 0, st>>>(qbar, kbar, scores, s.Tm, s.Tn, pitch, tm, tn, sqrt_d);
  else
    scores_kernel<128><<<grid, 256, 0, st>>>(qbar, kbar, scores, s.Tm, s.Tn, pitch, tm, tn, sqrt_d);
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const double* src, bool from_scores, double* pbar_out,
                         int n_k, double p_frac, const spa2_blockmask& m, hipStream_t st) {
  const int rows = s.BH() * s.Tm;
  const dim3 grid((rows + 3) / 4);  // four rows (waves) per workgroup
  const int per = (s.Tn + 63) / 64;
#define SPA2_SELECT(P)                                                                   \
  do {                                                                                   \
    if (from_scores)                                                                     \
      select_kernel<P, true><<<grid, 256, 0, st>>>(src, pbar_out, rows, s.Tn, n_k,       \
                                                   p_frac, m.mask, m.row_cnt, m.row_idx); \
    else                                                                                 \
      select_kernel<P, false><<<grid, 256, 0, st>>>(src, nullptr, rows, s.Tn, n_k,       \
                                                    p_frac, m.mask, m.row_cnt, m.row_idx); \
  } while (0)
  if (per <= 8) SPA2_SELECT(8);
  else if (per <= 16) SPA2_SELECT(16);
  else if (per <= 32) SPA2_SELECT(32);
  else SPA2_SELECT(64);
#undef SPA2_SELECT
  return hipGetLastError();
}

// Scheduling order: the item range [0, items) is cut into eight contiguous parts like
// xcd_item() cuts it; workgroup x lists part x by a counting sort. With per_head = 0 the
// key is the kept count, largest first. With per_head > 0 (items per head) the part is
// listed head by head, each head's items largest first, so the workgroups that run at the
// same time on one XCD mostly read one head's tiles (more L2 reuse); if the part spans too
// many heads for the histogram, the plain order is used. With hoist > 0 as well, items
// whose count reaches `hoist` are listed first (largest first) and only the rest head by
// head, so that the few very long lists start at once. Items with equal keys land in the
// order of their atomic increments.
__global__ __launch_bounds__(256) void order_kernel(OrderJob j0, OrderJob j1) {
  constexpr int kBins = 16384;
  static_assert(kBins >= kMaxTn + 1, "the plain order always fits");
  __shared__ int hist[kBins];
  __shared__ int wsum[4];
  // workgroups 0-7 list the parts of the first job, 8-15 those of the second
  const OrderJob& job = blockIdx.x < 8 ? j0 : j1;
  const int32_t* __restrict__ cnt = job.cnt;
  int32_t* __restrict__ order = job.order;
  const int items = job.items, maxc = job.maxc, per_head = job.per_head, hoist = job.hoist;
  const int tid = threadIdx.x, x = blockIdx.x & 7;
  const int q = items >> 3, r = items & 7;
  const int lo = x * q + min(x, r), n = q + (x < r ? 1 : 0);
  const int nb = maxc + 1;
  const int h0 = per_head > 0 ? lo / per_head : 0;
  const int nh = per_head > 0 && n > 0 ? (lo + n - 1) / per_head - h0 + 1 : 1;
  const int top = per_head > 0 && hoist > 0 ? nb : 0;  // bins of the hoisted section
  const bool by_head = top + nh * nb <= kBins;
  const int nbins = by_head ? top + nh * nb : nb;
  // bin of item lo + i: hoisted items by count from the top; the others by head within
  // the part, then count from the top
  auto bin = [&](int i) {
    const int c = min(max(cnt[lo + i], 0), maxc);
    if (!by_head || per_head == 0) return maxc - c;
    if (top > 0 && c >= hoist) return maxc - c;
    return top + ((lo + i) / per_head - h0) * nb + (maxc - c);
  };
  for (int c = tid; c < nbins; c += 256) hist[c] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 256) atomicAdd(&hist[bin(i)], 1);
  __syncthreads();
  // exclusive scan of the bins: thread t owns bins [t per, (t + 1) per)
  const int per = (nbins + 255) / 256;
  int local = 0;
  for (int k = 0; k < per; ++k) {
    const int u = tid * per + k;
    if (u < nbins) local += hist[u];
  }
  int inc = local;  // inclusive scan over the threads
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if ((tid & 63) >= o) inc += y;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = inc;
  __syncthreads();
  int run = inc - local;
  for (int wv = 0; wv < (tid >> 6); ++wv) run += wsum[wv];
  for (int k = 0; k < per; ++k) {
    const int u = tid * per + k;
    if (u < nbins) {
      const int h = hist[u];
      hist[u] = run;
      run += h;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += 256) order[lo + atomicAdd(&hist[bin(i)], 1)] = lo + i;
}

hipError_t launch_orders(const OrderJob* a, const OrderJob* b, hipStream_t st) {
  if (!a && !b) return hipSuccess;
  if (a && b) order_kernel<<<16, 256, 0, st>>>(*a, *b);
  else order_kernel<<<8, 256, 0, st>>>(a ? *a : *b, a ? *a : *b);
  return hipGetLastError();
}

hipError_t launch_rows(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int rows = s.BH() * s.Tm;
  rows_kernel<<<(rows + 3) / 4, 256, 0, st>>>(m.mask, rows, s.Tn, m.row_cnt, m.row_idx);
  return hipGetLastError();
}

hipError_t launch_cols(const Shape& s, const spa2_blockmask& m, hipStream_t st) {
  const int groups = (s.Tn + 63) / 64;
  cols_kernel<<<s.BH() * groups, 512, 0, st>>>(m.mask, s.Tm, s.Tn, groups, m.col_cnt, m.col_idx);
  return hipGetLastError();
}

}  // namespace spa2
