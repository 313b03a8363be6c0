// Block-sparse attention backward on gfx950 (mask held fixed; it carries no gradient).
//
// The pages state that the sparse attention is trainable with its own backward kernel
// (abstract; paper.rainbus.top summary, "核心方法") but give no formulas. With
// P = softmax over the kept keys of S = Q K^T / sqrt(D) and O = P V, the gradients are
//   Dv_r = dO_r . O_r,   dP = dO V^T,   dS = P * (dP - Dv),
//   dQ = dS K / sqrt(D),   dK = dS^T Q / sqrt(D),   dV = P^T dO,
// summed over kept block pairs only. P is rebuilt from the forward's LSE.
//
// Three deterministic kernels:
//   bwd_pre   Dv = rowsum(dO * O) (fp32), one pass over O and dO;
//   bwd_dkdv  one workgroup per key block, looping over the query blocks that keep it
//             (column lists); the four waves split the block 2 x 2 (key halves of 32
//             x query halves), Q_i and dO_i are staged in LDS, and the two query
//             halves' partial dK/dV are summed through LDS at the end;
//   bwd_dq    one workgroup per query block, looping over its kept key blocks (row
//             lists), like the forward; K_j and V_j are staged in LDS.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace spa2 {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* o_f32;  // optional unrounded O (preferred for the row term)
  const float* lse;
  const void* dout;
  const int32_t* row_cnt;  // nullptr: dense
  const int32_t* row_idx;
  const int32_t* col_cnt;
  const int32_t* col_idx;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  int N, Tm, Tn, BH;
  float scale_log2;  // log2(e) / sqrt(D)
  float scale;       // 1 / sqrt(D)
};

// ------------------------------------------------------------------------------------
// Dv_r = sum_d dO[r][d] * O[r][d]; TPR threads per row, each a 16-byte chunk.
// ------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int TPR = D / EPC;
  constexpr int RPB = 256 / TPR;
  const size_t rows = (size_t)a.BH * a.N;
  const size_t r = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 rd = *reinterpret_cast<const u32x4*>((const T*)a.dout + r * D + c * EPC);
    const T* xd = reinterpret_cast<const T*>(&rd);
    if (a.o_f32) {
      const float* of = a.o_f32 + r * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc += of[e] * Elem<T>::to_f32(xd[e]);
    } else {
      const u32x4 ro = *reinterpret_cast<const u32x4*>((const T*)a.o + r * D + c * EPC);
      const T* xo = reinterpret_cast<const T*>(&ro);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc += Elem<T>::to_f32(xo[e]) * Elem<T>::to_f32(xd[e]);
    }
  }
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
  if (r < rows && c == 0) a.dvec[r] = acc;
}

// ------------------------------------------------------------------------------------
// dQ: per query block, over its kept key blocks.
//   S^T = K Q^T, dP^T = V dO^T (A = K, V rows from LDS; B = Q, dO in registers),
//   dS^T = P^T * (dP^T - Dv), dQ^T += K^T dS^T (A = K^T via transpose reads).
// ------------------------------------------------------------------------------------
template <typename T, int D, int BQ, bool DENSE>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BKV = 64;
  constexpr int QT = BQ / 64;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using KV = Tile<T, BKV, D>;
  // two stages in two LDS variables, named statically (see the forward kernel)
  __shared__ __attribute__((aligned(1024))) char stage0[2 * KV::kBytes];
  __shared__ __attribute__((aligned(1024))) char stage1[2 * KV::kBytes];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = xcd_item(blockIdx.x, a.BH * a.Tm);
  const int bh = item / a.Tm, qb = item % a.Tm;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const int q0 = qb * BQ + w * 16 * QT;

  constexpr bool dense = DENSE;
  const int cnt = dense ? a.Tn : a.row_cnt[item];
  ListCursor cur;
  if (!dense) cur.init(a.row_idx + (size_t)item * a.Tn, cnt);
  auto block_of = [&](int t) { return dense ? t : cur.at(t); };
  typename KV::template Plan<4> plan;
  plan.init(w);
  auto issue = [&](char* stage, int j) {
    plan.issue_any(stage, K, j * BKV, N, w);
    plan.issue_any(stage + KV::kBytes, V, j * BKV, N, w);
  };
  if (cnt > 0) issue(stage0, block_of(0));

  F qf[QT][KS], df[QT][KS];
  float lse2[QT], dv[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = q0 + qt * 16 + c16;
    const bool ok = row < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qt][ks] = ok ? load_row8<T>(Q + (size_t)row * D + ks * 32 + 8 * g) : E::zero();
      df[qt][ks] = ok ? load_row8<T>(dO + (size_t)row * D + ks * 32 + 8 * g) : E::zero();
    }
    lse2[qt] = ok ? a.lse[(size_t)bh * N + row] * kLog2e : INFINITY;
    dv[qt] = ok ? a.dvec[(size_t)bh * N + row] : 0.f;
  }

  // bf16 only: rounding corrections (see below). pkc accumulates sum_j P^blk_j c_j, the
  // attention-weighted block centres; tpart the lane's share of sum_k dS_k.
  constexpr bool kCorr = sizeof(T) == 2;
  f32x4 acc[DT][QT], pkc[DT][QT];
  float tpart[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    tpart[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pkc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  auto block = [&](int t, const char* stage, char* next) {
    const int j = block_of(t);
    const int jn = t + 1 < cnt ? block_of(t + 1) : 0;
    wait_vmem();      // this wave's loads of block t have landed
    __syncthreads();  // ... and every other wave's; block t-1 is no longer being read
    if (t + 1 < cnt) issue(next, jn);
    const char* Kb = stage;
    const char* Vb = stage + KV::kBytes;

    f32x4 s[4][QT], dp[4][QT];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const F ka = KV::read_row8(Kb, kt * 16 + c16, ks * 32 + 8 * g);
        const F va = KV::read_row8(Vb, kt * 16 + c16, ks * 32 + 8 * g);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          s[kt][qt] = E::mma(ka, qf[qt][ks], s[kt][qt]);
          dp[kt][qt] = E::mma(va, df[qt][ks], dp[kt][qt]);
        }
      }
    }
    const bool tail = (j + 1) * BKV > N;
    float pblk[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) pblk[qt] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = !tail || (j * BKV + kt * 16 + 4 * g + e < N);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float p =
              valid ? __builtin_amdgcn_exp2f(s[kt][qt][e] * a.scale_log2 - lse2[qt]) : 0.f;
          const float ds = p * (dp[kt][qt][e] - dv[qt]);
          s[kt][qt][e] = ds;  // dS^T
          if (kCorr) {
            pblk[qt] += p;
            tpart[qt] += ds;
          }
        }
      }

#pragma unroll
    for (int u = 0; u < 2; ++u) {
      F pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) pf[qt] = E::pack(s[2 * u][qt], s[2 * u + 1][qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F kt_;
        KV::read_col4(Kb, 32 * u, dt * 16, kt_, 0);
        KV::read_col4(Kb, 32 * u + 16, dt * 16, kt_, 1);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[dt][qt] = E::mma(kt_, pf[qt], acc[dt][qt]);
      }
    }
    if constexpr (kCorr) {
      // Two bf16 error terms grow with a large offset c_j shared by a block's keys (an
      // attention-sink block), because each is multiplied by the keys:
      //  * rounding dS to bf16 leaves sum_k r_k K_k, r = dS - bf16(dS), whose offset part
      //    (sum_k r_k) c_j is added back here;
      //  * the row term Dv carries the rounding of O, which shifts every dS_k by
      //    -P_k dDv. In exact arithmetic sum_k dS_k = 0 over the row, so the measured
      //    T = sum_k dS_k equals -dDv, and the shift's offset part, T sum_j P^blk_j c_j
      //    (P^blk_j = the row's mass on block j), is removed in the epilogue.
      // c_j = the block's first key row; what remains involves only K_k - c_j.
      float rsum[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float r = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) r += s[kt][qt][e] - (float)(bf16)s[kt][qt][e];
        rsum[qt] = sum4(r);
        pblk[qt] = sum4(pblk[qt]);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 c4 = *reinterpret_cast<const bf16x4*>(Kb + KV::offset(0, dt * 16 + 4 * g));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[dt][qt][e] += (float)c4[e] * rsum[qt];
            pkc[dt][qt][e] += (float)c4[e] * pblk[qt];
          }
      }
    }
  };
  for (int t = 0; t < cnt; t += 2) {
    block(t, stage0, stage1);
    if (t + 1 < cnt) block(t + 1, stage1, stage0);
  }

  if constexpr (kCorr) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float tsum = sum4(tpart[qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt][qt] -= tsum * pkc[dt][qt];
    }
  }

  T* dQ = (T*)a.dq + head;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = q0 + qt * 16 + c16;
    if (row < N) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        T outv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) outv[e] = (T)(acc[dt][qt][e] * a.scale);
        T* dst = dQ + (size_t)row * D + dt * 16 + 4 * g;
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{outv[0], outv[1], outv[2], outv[3]};
        else
          *reinterpret_cast<f32x4*>(dst) = f32x4{outv[0], outv[1], outv[2], outv[3]};
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// dK, dV: per key block, over the query blocks that keep it (column lists).
// Wave w owns key half kh = w % 2 (32 keys) and query half qh = w / 2 of every query
// block, so each wave reads only its half of Q_i and dO_i from LDS (in both layouts),
// which halves the LDS traffic per matrix instruction compared with 16 keys per wave
// over all rows. Q_i and dO_i stream into LDS with global_load_lds, one block ahead;
// LSE and Dv of the wave's rows are read straight from global memory.
//   S = Q K^T, dP = dO V^T (A = Q, dO rows from LDS; B = K, V in registers),
//   dS = P * (dP - Dv), dV^T += dO^T P, dK^T += Q^T dS (A via transpose reads).
// At the end the two query halves' partial sums are added through LDS.
// ------------------------------------------------------------------------------------
template <typename T, int D, int BQ, bool DENSE>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BKV = 64;
  constexpr int MT = BQ / 32;  // 16-row query tiles per wave (half of the query block)
  constexpr int KT = 2;        // 16-key tiles per wave (32 keys)
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using QTile = Tile<T, BQ, D>;
  constexpr int kStage = 2 * QTile::kBytes;  // Q_i and dO_i
  constexpr int NS = 2 * kStage <= 160 * 1024 ? 2 : 1;  // one stage only if two do not fit
  __shared__ __attribute__((aligned(1024))) char stage0[kStage];
  __shared__ __attribute__((aligned(1024))) char stage1[NS == 2 ? kStage : 16];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1, qh = w >> 1;
  const int item = xcd_item(blockIdx.x, a.BH * a.Tn);
  const int bh = item / a.Tn, kb = item % a.Tn;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const float* LSE = a.lse + (size_t)bh * N;
  const float* DV = a.dvec + (size_t)bh * N;
  const int k0 = kb * BKV + kh * 32;  // first key of this wave
  const int qrow0 = qh * (BQ / 2);    // first query row of this wave within a query block

  constexpr bool dense = DENSE;
  const int cnt = dense ? a.Tm : a.col_cnt[item];
  ListCursor cur;
  if (!dense) cur.init(a.col_idx + (size_t)item * a.Tm, cnt);
  auto block_of = [&](int t) { return dense ? t : cur.at(t); };
  typename QTile::template Plan<4> plan;
  plan.init(w);
  auto issue = [&](char* stage, int i) {
    plan.issue_any(stage, Q, i * BQ, N, w);
    plan.issue_any(stage + QTile::kBytes, dO, i * BQ, N, w);
  };
  if (cnt > 0) issue(stage0, block_of(0));

  // K, V as B operands: lane -> key k0 + 16 kt + c16, dims 32 ks + 8 g .. +8
  F kf[KT][KS], vf[KT][KS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = k0 + kt * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kt][ks] = key < N ? load_row8<T>(K + (size_t)key * D + ks * 32 + 8 * g) : E::zero();
      vf[kt][ks] = key < N ? load_row8<T>(V + (size_t)key * D + ks * 32 + 8 * g) : E::zero();
    }
  }

  // accumulators, transposed: lane holds [dim 16 dt + 4 g + e][key 16 kt + c16]
  f32x4 dk[DT][KT], dv[DT][KT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      dk[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  auto compute = [&](int i, const char* stage) {
    const char* Qb = stage;
    const char* Db = stage + QTile::kBytes;
    // this lane's rows of the statistics: queries i*BQ + qrow0 + 16 mt + 4 g + e
    f32x4 l4[MT], d4[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = i * BQ + qrow0 + mt * 16 + 4 * g;
      if (r + 3 < N && ((reinterpret_cast<uintptr_t>(LSE + r) | reinterpret_cast<uintptr_t>(DV + r)) & 15) == 0) {
        l4[mt] = *reinterpret_cast<const f32x4*>(LSE + r);
        d4[mt] = *reinterpret_cast<const f32x4*>(DV + r);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l4[mt][e] = r + e < N ? LSE[r + e] : INFINITY;  // rows past N get P = 0
          d4[mt][e] = r + e < N ? DV[r + e] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) l4[mt][e] *= kLog2e;
    }
    // S[query 16 mt + 4 g + e][key 16 kt + c16], dP likewise
    f32x4 s[MT][KT], dp[MT][KT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[mt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const F qa = QTile::read_row8(Qb, qrow0 + mt * 16 + c16, ks * 32 + 8 * g);
        const F da = QTile::read_row8(Db, qrow0 + mt * 16 + c16, ks * 32 + 8 * g);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          s[mt][kt] = E::mma(qa, kf[kt][ks], s[mt][kt]);
          dp[mt][kt] = E::mma(da, vf[kt][ks], dp[mt][kt]);
        }
      }
    }
    // P (kept in s) and dS (kept in dp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][kt][e], a.scale_log2, -l4[mt][e]));
          s[mt][kt][e] = p;
          dp[mt][kt][e] = p * (dp[mt][kt][e] - d4[mt][e]);
        }
    // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over the wave's queries, 32 at a time)
#pragma unroll
    for (int u = 0; u < MT / 2; ++u) {
      F pf[KT], sf[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        pf[kt] = E::pack(s[2 * u][kt], s[2 * u + 1][kt]);
        sf[kt] = E::pack(dp[2 * u][kt], dp[2 * u + 1][kt]);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F dot, qtr;
        QTile::read_col4(Db, qrow0 + 32 * u, dt * 16, dot, 0);
        QTile::read_col4(Db, qrow0 + 32 * u + 16, dt * 16, dot, 1);
        QTile::read_col4(Qb, qrow0 + 32 * u, dt * 16, qtr, 0);
        QTile::read_col4(Qb, qrow0 + 32 * u + 16, dt * 16, qtr, 1);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          dv[dt][kt] = E::mma(dot, pf[kt], dv[dt][kt]);
          dk[dt][kt] = E::mma(qtr, sf[kt], dk[dt][kt]);
        }
      }
    }
  };

  if constexpr (NS == 2) {
    auto block = [&](int t, const char* stage, char* next) {
      const int i = block_of(t);
      const int in = t + 1 < cnt ? block_of(t + 1) : 0;
      wait_vmem();
      __syncthreads();
      if (t + 1 < cnt) issue(next, in);
      compute(i, stage);
    };
    for (int t = 0; t < cnt; t += 2) {
      block(t, stage0, stage1);
      if (t + 1 < cnt) block(t + 1, stage1, stage0);
    }
  } else {
    for (int t = 0; t < cnt; ++t) {
      const int i = block_of(t);
      const int in = t + 1 < cnt ? block_of(t + 1) : 0;
      wait_vmem();
      __syncthreads();
      compute(i, stage0);
      __syncthreads();  // every wave is done with the only stage
      if (t + 1 < cnt) issue(stage0, in);
    }
  }

  // add the query halves: waves with qh = 1 hand their partial sums to qh = 0 via LDS,
  // one tensor at a time (DT * KT * 1 KB per wave)
  f32x4* xfer = reinterpret_cast<f32x4*>(stage0);
  auto reduce = [&](f32x4 (&acc)[DT][KT]) {
    __syncthreads();
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) xfer[((kh * DT + dt) * KT + kt) * 64 + l] = acc[dt][kt];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) acc[dt][kt] += xfer[((kh * DT + dt) * KT + kt) * 64 + l];
    }
  };
  reduce(dk);
  reduce(dv);

  if (qh == 0) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = k0 + kt * 16 + c16;
      if (key >= N) continue;
      T* dK = (T*)a.dk + head + (size_t)key * D;
      T* dV = (T*)a.dv + head + (size_t)key * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        T ko[4], vo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ko[e] = (T)(dk[dt][kt][e] * a.scale);
          vo[e] = (T)dv[dt][kt][e];
        }
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dK + dt * 16 + 4 * g) = bf16x4{ko[0], ko[1], ko[2], ko[3]};
          *reinterpret_cast<bf16x4*>(dV + dt * 16 + 4 * g) = bf16x4{vo[0], vo[1], vo[2], vo[3]};
        } else {
          *reinterpret_cast<f32x4*>(dK + dt * 16 + 4 * g) = f32x4{ko[0], ko[1], ko[2], ko[3]};
          *reinterpret_cast<f32x4*>(dV + dt * 16 + 4 * g) = f32x4{vo[0], vo[1], vo[2], vo[3]};
        }
      }
    }
  }
}

hipError_t launch_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                      const float* o_f32, const float* lse, const void* dout, const spa2_blockmask* m, void* dq,
                      void* dk, void* dv, float* dvec, int stages, hipStream_t st) {
  BwdArgs a{q, k, v, o, o_f32, lse, dout,
            m ? m->row_cnt : nullptr, m ? m->row_idx : nullptr,
            m ? m->col_cnt : nullptr, m ? m->col_idx : nullptr,
            dq, dk, dv, dvec, s.N, s.Tm, s.Tn, s.BH(),
            (float)(1.4426950408889634 / sqrt((double)s.D)), (float)(1.0 / sqrt((double)s.D))};
  const int tpr = s.D * (s.dtype == SPA2_BF16 ? 2 : 4) / 16;
  const int rpb = 256 / tpr;
  const size_t rows = (size_t)s.BH() * s.N;
  const dim3 gpre((unsigned)((rows + rpb - 1) / rpb));
  const dim3 gq(s.BH() * s.Tm), gk(s.BH() * s.Tn);
#define SPA2_BWD(T, D, BQ)                                                       \
  do {                                                                           \
    if (stages & kBwdPrep) bwd_pre_kernel<T, D><<<gpre, 256, 0, st>>>(a);        \
    if (stages & kBwdDkdv) {                                                     \
      if (m) bwd_dkdv_kernel<T, D, BQ, false><<<gk, 256, 0, st>>>(a);           \
      else bwd_dkdv_kernel<T, D, BQ, true><<<gk, 256, 0, st>>>(a);              \
    }                                                                            \
    if (stages & kBwdDq) {                                                       \
      if (m) bwd_dq_kernel<T, D, BQ, false><<<gq, 256, 0, st>>>(a);             \
      else bwd_dq_kernel<T, D, BQ, true><<<gq, 256, 0, st>>>(a);                \
    }                                                                            \
  } while (0)
  if (s.dtype == SPA2_BF16) {
    if (s.D == 64) {
      if (s.BQ == 64) SPA2_BWD(bf16, 64, 64); else SPA2_BWD(bf16, 64, 128);
    } else {
      if (s.BQ == 64) SPA2_BWD(bf16, 128, 64); else SPA2_BWD(bf16, 128, 128);
    }
  } else {
    if (s.D == 64) {
      if (s.BQ == 64) SPA2_BWD(float, 64, 64); else SPA2_BWD(float, 64, 128);
    } else {
      if (s.BQ == 64) SPA2_BWD(float, 128, 64); else SPA2_BWD(float, 128, 128);
    }
  }
#undef SPA2_BWD
  return hipGetLastError();
}

}  // namespace spa2
