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
//             (column lists); wave w owns 16 keys; Q_i and dO_i are staged in LDS;
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
template <typename T, int D, int BQ>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BKV = 64;
  constexpr int QT = BQ / 64;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using KV = Tile<T, BKV, D>;
  constexpr int CPR = KV::kChunks;
  constexpr int CH = BKV * CPR / 256;
  __shared__ __attribute__((aligned(16))) char smem[2][2][KV::kBytes];

  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.x / a.Tm, qb = blockIdx.x % a.Tm;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const int q0 = qb * BQ + w * 16 * QT;

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

  const bool dense = a.row_cnt == nullptr;
  const int cnt = dense ? a.Tn : a.row_cnt[blockIdx.x];
  const int32_t* list = dense ? nullptr : a.row_idx + (size_t)blockIdx.x * a.Tn;

  u32x4 kr[CH], vr[CH];
  auto gload = [&](int j) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int flat = tid + c * 256, row = flat / CPR, ch = flat % CPR;
      const int key = j * BKV + row;
      if (key < N) {
        kr[c] = *reinterpret_cast<const u32x4*>(K + (size_t)key * D + ch * (16 / sizeof(T)));
        vr[c] = *reinterpret_cast<const u32x4*>(V + (size_t)key * D + ch * (16 / sizeof(T)));
      } else {
        kr[c] = u32x4{0, 0, 0, 0};
        vr[c] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int flat = tid + c * 256, row = flat / CPR, ch = flat % CPR;
      KV::store_chunk(smem[buf][0], row, ch, kr[c]);
      KV::store_chunk(smem[buf][1], row, ch, vr[c]);
    }
  };

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

  if (cnt > 0) {
    gload(dense ? 0 : list[0]);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int j = dense ? t : list[t];
    const int buf = t & 1;
    if (t + 1 < cnt) gload(dense ? t + 1 : list[t + 1]);
    const char* Kb = smem[buf][0];
    const char* Vb = smem[buf][1];

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

    if (t + 1 < cnt) lstore(buf ^ 1);
    __syncthreads();
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
// dK, dV: per key block, over the query blocks that keep it.
//   S = Q K^T, dP = dO V^T (A = Q, dO rows from LDS; B = K, V in registers),
//   dS = P * (dP - Dv), dV^T += dO^T P, dK^T += Q^T dS (A via transpose reads).
// ------------------------------------------------------------------------------------
template <typename T, int D, int BQ>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int BKV = 64;
  constexpr int MT = BQ / 16;  // 16-row query tiles in a query block
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using QTile = Tile<T, BQ, D>;
  constexpr int CPR = QTile::kChunks;
  constexpr int CH = BQ * CPR / 256;
  constexpr int kStage = 2 * QTile::kBytes + 2 * BQ * (int)sizeof(float);
  // two stages when they fit in the 160 KB of LDS, else one (fp32, D = BQ = 128)
  constexpr int NBUF = 2 * kStage <= 160 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][kStage];

  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.x / a.Tn, kb = blockIdx.x % a.Tn;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const float* LSE = a.lse + (size_t)bh * N;
  const float* DV = a.dvec + (size_t)bh * N;
  const int key = kb * BKV + w * 16 + c16;  // this lane's key (B operand column)

  F kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = key < N ? load_row8<T>(K + (size_t)key * D + ks * 32 + 8 * g) : E::zero();
    vf[ks] = key < N ? load_row8<T>(V + (size_t)key * D + ks * 32 + 8 * g) : E::zero();
  }

  const bool dense = a.col_cnt == nullptr;
  const int cnt = dense ? a.Tm : a.col_cnt[blockIdx.x];
  const int32_t* list = dense ? nullptr : a.col_idx + (size_t)blockIdx.x * a.Tm;

  u32x4 qr[CH], dr[CH];
  float lr = 0.f, dvr = 0.f;
  auto gload = [&](int i) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int flat = tid + c * 256, row = flat / CPR, ch = flat % CPR;
      const int q = i * BQ + row;
      if (q < N) {
        qr[c] = *reinterpret_cast<const u32x4*>(Q + (size_t)q * D + ch * (16 / sizeof(T)));
        dr[c] = *reinterpret_cast<const u32x4*>(dO + (size_t)q * D + ch * (16 / sizeof(T)));
      } else {
        qr[c] = u32x4{0, 0, 0, 0};
        dr[c] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < BQ) {
      const int q = i * BQ + tid;
      lr = q < N ? LSE[q] * kLog2e : INFINITY;  // rows past N get P = 0
      dvr = q < N ? DV[q] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    char* base = smem[buf];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int flat = tid + c * 256, row = flat / CPR, ch = flat % CPR;
      QTile::store_chunk(base, row, ch, qr[c]);
      QTile::store_chunk(base + QTile::kBytes, row, ch, dr[c]);
    }
    float* stats = reinterpret_cast<float*>(base + 2 * QTile::kBytes);
    if (tid < BQ) {
      stats[tid] = lr;
      stats[BQ + tid] = dvr;
    }
  };

  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (cnt > 0) {
    gload(dense ? 0 : list[0]);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int buf = NBUF == 2 ? (t & 1) : 0;
    if (t + 1 < cnt) gload(dense ? t + 1 : list[t + 1]);
    const char* Qb = smem[buf];
    const char* Db = Qb + QTile::kBytes;
    const float* stats = reinterpret_cast<const float*>(Qb + 2 * QTile::kBytes);

    // S[query 16 mt + 4 g + e][key c16], dP likewise
    f32x4 s[MT], dp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const F qa = QTile::read_row8(Qb, mt * 16 + c16, ks * 32 + 8 * g);
        const F da = QTile::read_row8(Db, mt * 16 + c16, ks * 32 + 8 * g);
        s[mt] = E::mma(qa, kf[ks], s[mt]);
        dp[mt] = E::mma(da, vf[ks], dp[mt]);
      }
    }
    // P and dS (P kept in s, dS in dp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(stats + mt * 16 + 4 * g);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(stats + BQ + mt * 16 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(s[mt][e] * a.scale_log2 - l4[e]);
        s[mt][e] = p;
        dp[mt][e] = p * (dp[mt][e] - d4[e]);
      }
    }
    // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over the block's queries, 32 at a time)
#pragma unroll
    for (int u = 0; u < MT / 2; ++u) {
      const F pf = E::pack(s[2 * u], s[2 * u + 1]);
      const F sf = E::pack(dp[2 * u], dp[2 * u + 1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F dot, qtr;
        QTile::read_col4(Db, 32 * u, dt * 16, dot, 0);
        QTile::read_col4(Db, 32 * u + 16, dt * 16, dot, 1);
        QTile::read_col4(Qb, 32 * u, dt * 16, qtr, 0);
        QTile::read_col4(Qb, 32 * u + 16, dt * 16, qtr, 1);
        dv[dt] = E::mma(dot, pf, dv[dt]);
        dk[dt] = E::mma(qtr, sf, dk[dt]);
      }
    }

    if (t + 1 < cnt) {
      if (NBUF == 1) __syncthreads();  // every wave is done with the only stage
      lstore(NBUF == 2 ? (buf ^ 1) : 0);
    }
    __syncthreads();
  }

  if (key < N) {
    T* dK = (T*)a.dk + head + (size_t)key * D;
    T* dV = (T*)a.dv + head + (size_t)key * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      T ko[4], vo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ko[e] = (T)(dk[dt][e] * a.scale);
        vo[e] = (T)dv[dt][e];
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
    if (stages & kBwdDkdv) bwd_dkdv_kernel<T, D, BQ><<<gk, 256, 0, st>>>(a);     \
    if (stages & kBwdDq) bwd_dq_kernel<T, D, BQ><<<gq, 256, 0, st>>>(a);         \
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
