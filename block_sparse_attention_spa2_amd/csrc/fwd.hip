// Block-sparse attention forward on gfx950.
//
// Method (SpargeAttention2, paper.rainbus.top summary, "方法步骤详情" step 4; "前置知识",
// block-sparse attention): for each kept block pair (i, j), S_ij = Q_i K_j^T / sqrt(D),
// the softmax is taken online over the kept key blocks of row i only, and O_i
// accumulates P_ij V_j. Masked pairs are skipped entirely: their K/V tiles are never
// fetched.
//
// One workgroup (4 waves) per query tile of 64 or 128 rows (a 256-row block is two
// tiles); two to four workgroups share a CU (one wave's softmax overlaps the others'
// matrix work). Wave w owns a quarter of the tile's rows. Key tiles of 32 or 64 rows (a
// larger key block is two or four tiles) of K and V stream from global memory straight
// into a double-buffered, swizzled LDS tile (global_load_lds), issued one tile ahead,
// with one barrier per tile. Scores are computed transposed, S^T = K Q^T (operand A = K
// rows from LDS, operand B = Q held in registers), so each lane owns one query column and the
// online-softmax state is lane local (the row max needs the 4 lanes that share the
// column, combined with VALU lane swaps, but only when it is raised). P^T leaves the
// accumulators directly as the B operand of O^T = V^T P^T; V^T comes from row-major LDS
// through transpose reads.
// The running max is only raised (and O rescaled) when a row's block max exceeds it by
// more than 2^8, so most blocks skip the rescale; the final normalisation is exact.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace spa2 {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* o_f32;  // optional unrounded copy of O
  const int32_t* row_cnt;  // nullptr: dense
  const int32_t* row_idx;
  const int32_t* row_order;  // optional scheduling order of the query blocks
  int N, Tm, Tn, items;  // items: workgroups = query blocks x query tiles per block
  int bq_block;          // rows of a mask query block (a multiple of the kernel's tile)
  int qsub;              // log2 of the query tiles per block
  float scale_log2;  // log2(e) / sqrt(D)
};

// Rescale threshold in log2 units: probabilities stay below 2^8 between rescales.
constexpr float kRescaleSlack = 8.0f;

// Maxima of scores (finite, or -inf for keys past N) as plain v_max3_f32 / v_max_f32 in
// inline asm: fmaxf would first canonicalise every operand that the compiler cannot prove
// canonical (all matrix-unit results), doubling the instruction count of the block maximum.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum of a lane's 16 (or 8) scores of one column as two interleaved v_max3 chains in
// one asm block (separate asm statements get a wait state between each pair). The scores
// come straight from matrix instructions: a vector instruction may read an MFMA result
// only 8 wait states after the MFMA issues (16x16x32 bf16 on gfx950), and the compiler
// inserts those wait states for its own instructions but not for inline asm, so each
// block starts with s_nop 7.
__device__ __forceinline__ float lane_max16(const f32x4& a, const f32x4& b, const f32x4& c,
                                            const f32x4& d) {
  float r, t;
  asm("s_nop 7\n\t"
      "v_max3_f32 %0, %2, %3, %4\n\t"
      "v_max3_f32 %1, %5, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %1, %1, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %1, %1, %14, %15\n\t"
      "v_max3_f32 %0, %0, %16, %17\n\t"
      "v_max_f32 %0, %0, %1"
      : "=&v"(r), "=&v"(t)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]),
        "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]));
  return r;
}
__device__ __forceinline__ float lane_max8(const f32x4& a, const f32x4& b) {
  float r, t;
  asm("s_nop 7\n\t"
      "v_max3_f32 %0, %2, %3, %4\n\t"
      "v_max3_f32 %1, %5, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max_f32 %0, %0, %1"
      : "=&v"(r), "=&v"(t)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
  return r;
}
// max over the four lanes that share a query column (l, l^16, l^32, l^48)
__device__ __forceinline__ float max4_raw(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = max_raw(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  u = __builtin_bit_cast(unsigned, x);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max_raw(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// Workgroups per CU that the launch bounds ask for. bf16 at D = 128 steps through 32-key
// tiles: 32 KB of LDS and at most 168 registers per 4-wave workgroup of 128 query rows
// (128 for 64 rows) let three (four) workgroups share a CU, which hides more of each
// wave's dependent S -> softmax -> P.V chain than two workgroups with 64-key tiles (64 KB
// of LDS each).
template <typename T, int D, int BQ, int BKV>
constexpr int fwd_wgs_per_cu() {
  return sizeof(T) == 2 && D == 128 && BKV == 32 ? (BQ == 128 ? 3 : 4) : 2;
}

// Tiles: BQ query rows per workgroup, BKV keys per step (32 or 64). A mask block of 256
// rows runs as two workgroups (query tiles), a mask block of more keys than BKV as 2^KSUB
// key steps.
template <typename T, int D, int BQ, int BKV, int KSUB, bool DENSE, int NW>
__global__ __launch_bounds__(64 * NW, (fwd_wgs_per_cu<T, D, BQ, BKV>())) void fwd_kernel(FwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int QT = BQ / (16 * NW);  // 16-row query tiles per wave
  constexpr int KS = D / 32;   // reduction steps over the head dimension
  constexpr int DT = D / 16;   // 16-wide output column tiles
  constexpr int KTN = BKV / 16;  // 16-key score tiles per step
  constexpr int UPV = BKV / 32;  // 32-key reduction steps of O^T += V^T P^T
  using KV = Tile<T, BKV, D>;
  // Two stages in two separate LDS variables: every access names one of them statically
  // (the loop below is unrolled by two), so the compiler can tell that the loads into one
  // stage do not alias the reads of the other and does not wait for them early. The
  // epilogue passes the fp32 O tile through the two stages.
  constexpr int kStageBytes = 2 * KV::kBytes;
  __shared__ __attribute__((aligned(1024))) char stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char stage1[kStageBytes];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // paired XCDs; the tiles of one block stay on one XCD, sharing its L2
  const int pos = xcd_item_paired_tiles(blockIdx.x, a.items, a.qsub);
  const int ppos = pos >> a.qsub;  // this query tile's block, in scheduling order
  const int item = a.row_order ? __builtin_amdgcn_readfirstlane(a.row_order[ppos]) : ppos;
  const int bh = item / a.Tm, qb = item % a.Tm;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const int r0 = qb * a.bq_block + (pos & ((1 << a.qsub) - 1)) * BQ;  // first row of the tile
  const int q0 = r0 + w * 16 * QT;

  constexpr bool dense = DENSE;  // dense: every key tile, no list
  const int cnt = dense ? (N + BKV - 1) / BKV : a.row_cnt[item] << KSUB;  // key steps
  TileQueue<KSUB> bq;  // key tiles t, t + 1 (next tile load) and t + 2 (being read)
  if (!dense) bq.init(a.row_idx + (size_t)item * a.Tn, a.row_cnt[item]);
  auto block_at = [&](int t, int i) { return dense ? t + i : bq.tile(t, i); };
  typename KV::template Plan<NW> plan;
  plan.init(w);
  auto issue = [&](char* stage, int j) {
    plan.issue_any(stage, K, j * BKV, N, w);
    plan.issue_any(stage + KV::kBytes, V, j * BKV, N, w);
  };
  if (cnt > 0) issue(stage0, block_at(0, 0));

  // Q as the B operand: lane -> query q0 + 16 qt + c16, dims 32 ks + 8 g .. +8
  F qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = q0 + qt * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qt][ks] = row < N ? load_row8_stream<T>(Q + (size_t)row * D + ks * 32 + 8 * g) : E::zero();
  }

  f32x4 oacc[DT][QT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max (log2 units) and its finite stand-in for the exponent (0 while no key of
  // the column has been seen), both changed only when the max is raised
  float mrow[QT], mref[QT], lrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrow[qt] = -INFINITY;
    mref[qt] = 0.f;
    lrow[qt] = 0.f;
  }

  auto block = [&](int t, const char* stage, char* next) {
    const int j = block_at(t, 0);
    const int jn = block_at(t, 1);
    if (!dense) bq.advance(t);
    wait_vmem();      // this wave's loads of block t have landed
    lds_barrier();  // ... and every other wave's; block t-1 is no longer being read
    if (t + 1 < cnt) issue(next, jn);
    const char* Kb = stage;
    const char* Vb = stage + KV::kBytes;

    // S^T = K Q^T : s[kt][qt] lane holds S^T[key 16 kt + 4 g + e][query 16 qt + c16]
    f32x4 s[KTN][QT];
#pragma unroll
    for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) {
        const F ka = KV::read_row8(Kb, kt * 16 + c16, ks * 32 + 8 * g);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[kt][qt] = E::mma(ka, qf[qt][ks], s[kt][qt]);
      }
    }
    // keys past N exist only in the last, partial key block
    if ((j + 1) * BKV > N) {
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j * BKV + kt * 16 + 4 * g + e >= N)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[kt][qt][e] = -INFINITY;
    }

    // online softmax, per query column (base-2 exponent with the scale folded in). Whether
    // some column's block max exceeds its running max by the slack is decided from each
    // lane's own maximum (a column exceeds it iff one of its four lanes does); the column
    // max over the four lanes is formed only when the running max is raised.
    float mx[QT];
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // this lane's KTN x 4 scores of the column
      float m;
      if constexpr (KTN == 4) m = lane_max16(s[0][qt], s[1][qt], s[2][qt], s[3][qt]);
      else m = lane_max8(s[0][qt], s[1][qt]);
      mx[qt] = m;
      raise |= m * a.scale_log2 > mrow[qt] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform: some row needs a new max
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mnew = fmaxf(mrow[qt], max4_raw(mx[qt]) * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(mrow[qt] - mnew);  // 0 on the first block
        mrow[qt] = mnew;
        mref[qt] = mnew == -INFINITY ? 0.f : mnew;
        lrow[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][qt][e], a.scale_log2, -mref[qt]));
          s[kt][qt][e] = p;
          ls += p;
        }
      lrow[qt] += ls;
    }

    // O^T += V^T P^T over the step's keys, 32 at a time
#pragma unroll
    for (int u = 0; u < UPV; ++u) {
      F pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) pf[qt] = E::pack(s[2 * u][qt], s[2 * u + 1][qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F va;
        KV::read_col4(Vb, 32 * u, dt * 16, va, 0);
        KV::read_col4(Vb, 32 * u + 16, dt * 16, va, 1);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = E::mma(va, pf[qt], oacc[dt][qt]);
      }
    }
  };
  for (int t = 0; t < cnt; t += 2) {
    block(t, stage0, stage1);
    if (t + 1 < cnt) block(t + 1, stage1, stage0);
  }

  // epilogue: normalise, then store O (and the unrounded copy) through LDS, so that every
  // global store writes whole 16-byte chunks of consecutive columns of a row (full cache
  // lines) instead of 4 columns of 16 rows. The fp32 tile (BQ x D) passes through the two
  // stages in as many passes of kPassRows rows as they need (one for 64-key tiles, two
  // for 32-key tiles): the first half of a pass's rows into stage0, the rest into
  // stage1, with the 16-byte chunks of row r XOR-swizzled by r mod 32 (conflict-free
  // writes of 16 rows at a time).
  float* lse = a.lse + (size_t)bh * N;
  constexpr int kRowChunks = D / 4;               // 16-byte fp32 chunks per row
  constexpr int kFit = 2 * (kStageBytes / (D * 4));  // rows that the two stages hold
  constexpr int kPassRows = kFit < BQ ? kFit : BQ;
  constexpr int kHalfRows = kPassRows / 2;
  static_assert(BQ % kPassRows == 0 && kPassRows % (16 * QT) == 0, "whole waves per pass");
  auto chunk_at = [&](int r, int c) -> f32x4* {  // row r of the pass, chunk c
    char* base = r < kHalfRows ? stage0 : stage1;
    const int rr = r % kHalfRows;
    return reinterpret_cast<f32x4*>(base + rr * D * 4 + ((c ^ (rr & (kRowChunks - 1) & 31)) << 4));
  };
  float inv[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = r0 + w * 16 * QT + qt * 16 + c16;
    const float lt = sum4(lrow[qt]);
    inv[qt] = lt > 0.f ? 1.f / lt : 0.f;
    if (g == 0 && row < N) lse[row] = lt > 0.f ? (mrow[qt] + __log2f(lt)) * kLn2 : -INFINITY;
  }
  constexpr int kEpc = 16 / (int)sizeof(T);        // elements per 16-byte output chunk
  for (int pr0 = 0; pr0 < BQ; pr0 += kPassRows) {
    lds_barrier();  // the K/V stages, or the previous pass, are no longer read
    if (w * 16 * QT >= pr0 && w * 16 * QT < pr0 + kPassRows) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int rl = w * 16 * QT + qt * 16 + c16 - pr0;  // row within the pass
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *chunk_at(rl, dt * 4 + g) = oacc[dt][qt] * inv[qt];
      }
    }
    lds_barrier();
    const int rows_here = min(kPassRows, N - r0 - pr0);
    T* O = (T*)a.o + head + (size_t)(r0 + pr0) * D;
    for (int f = tid; f < kPassRows * D / kEpc; f += 64 * NW) {
      const int r = f / (D / kEpc), c = f % (D / kEpc);
      if (r >= rows_here) break;  // chunks are in row order
      if constexpr (sizeof(T) == 2) {
        const f32x4 lo = *chunk_at(r, 2 * c), hi = *chunk_at(r, 2 * c + 1);
        bf16x8 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ob[e] = (bf16)lo[e];
          ob[4 + e] = (bf16)hi[e];
        }
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ob),
                                    reinterpret_cast<u32x4*>(O + (size_t)r * D + c * kEpc));
      } else {
        __builtin_nontemporal_store(*chunk_at(r, c), reinterpret_cast<f32x4*>(O + (size_t)r * D + c * kEpc));
      }
    }
    if (a.o_f32) {
      float* Of = a.o_f32 + head + (size_t)(r0 + pr0) * D;
      for (int f = tid; f < kPassRows * kRowChunks; f += 64 * NW) {
        const int r = f / kRowChunks, c = f % kRowChunks;
        if (r >= rows_here) break;
        __builtin_nontemporal_store(*chunk_at(r, c), reinterpret_cast<f32x4*>(Of + (size_t)r * D + c * 4));
      }
    }
  }
}

// Waves per workgroup. Four (32 query rows each for 128-row blocks) measured faster than
// eight waves of 16 rows, which read every K/V tile from LDS twice as often per matrix
// instruction.
template <typename T, int BQ>
constexpr int fwd_waves() { return 4; }

template <typename T, int D, int BQ, int BK>
void launch_fwd_tile(const Shape& s, const FwdArgs& a, hipStream_t st) {
  constexpr int nw = fwd_waves<T, BQ>();
  const dim3 grid(a.items), block(64 * nw);
  const int steps = s.BKV / BK;  // key steps per mask block: 1, 2 or 4
  if (!a.row_cnt) {
    fwd_kernel<T, D, BQ, BK, 0, true, nw><<<grid, block, 0, st>>>(a);
  } else if constexpr (BK == 32) {
    if (steps == 4) fwd_kernel<T, D, BQ, BK, 2, false, nw><<<grid, block, 0, st>>>(a);
    else if (steps == 2) fwd_kernel<T, D, BQ, BK, 1, false, nw><<<grid, block, 0, st>>>(a);
    else fwd_kernel<T, D, BQ, BK, 0, false, nw><<<grid, block, 0, st>>>(a);
  } else {
    if (steps == 2) fwd_kernel<T, D, BQ, BK, 1, false, nw><<<grid, block, 0, st>>>(a);
    else fwd_kernel<T, D, BQ, BK, 0, false, nw><<<grid, block, 0, st>>>(a);
  }
}

template <typename T, int D, int BQ>
void launch_fwd_bq(const Shape& s, const FwdArgs& a, hipStream_t st) {
  if constexpr (fwd_wgs_per_cu<T, D, BQ, 32>() > 2) launch_fwd_tile<T, D, BQ, 32>(s, a, st);
  else if (s.bkv_tile() == 32) launch_fwd_tile<T, D, BQ, 32>(s, a, st);
  else launch_fwd_tile<T, D, BQ, 64>(s, a, st);
}

template <typename T, int D>
void launch_fwd_d(const Shape& s, const FwdArgs& a, hipStream_t st) {
  if (s.bq_tile() == 64) launch_fwd_bq<T, D, 64>(s, a, st);
  else launch_fwd_bq<T, D, 128>(s, a, st);
}

hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const int32_t* row_cnt, const int32_t* row_idx, const int32_t* row_order,
                      void* o, float* lse, float* o_f32, hipStream_t st) {
  const int items = (s.BH() * s.Tm) << s.qsub();
  const FwdArgs a{q, k, v, o, lse, o_f32, row_cnt, row_idx, row_cnt ? row_order : nullptr, s.N,
                  s.Tm, s.Tn, items, s.BQ, s.qsub(),
                  (float)(1.4426950408889634 / sqrt((double)s.D))};
  if (s.dtype == SPA2_BF16) {
    if (s.D == 64) launch_fwd_d<bf16, 64>(s, a, st); else launch_fwd_d<bf16, 128>(s, a, st);
  } else {
    if (s.D == 64) launch_fwd_d<float, 64>(s, a, st); else launch_fwd_d<float, 128>(s, a, st);
  }
  return hipGetLastError();
}

}  // namespace spa2
