// Block-sparse attention backward on gfx950 (mask held fixed; it carries no gradient).
//
// The pages state that the sparse attention is trainable with its own backward kernel
// (abstract; paper.rainbus.top summary, "核心方法") but give no formulas. With
// P = softmax over the kept keys of S = Q K^T / sqrt(D) and O = P V, the gradients are
//   Dv_r = dO_r . O_r,   dP = dO V^T,   dS = P * (dP - Dv),
//   dQ = dS K / sqrt(D),   dK = dS^T Q / sqrt(D),   dV = P^T dO,
// summed over kept block pairs only. P is rebuilt from the forward's LSE.
//
// Deterministic kernels (spa2_bwd runs the dQ pass with the row term, then dK/dV):
//   bwd_pre   Dv = rowsum(dO * O) (fp32), one pass over O and dO (the staged call only);
//   bwd_dq    one workgroup per query tile, looping over its kept key tiles (row lists),
//             like the forward; K_j and V_j are staged in LDS; optionally computes Dv of
//             its rows first (the row term) and writes it for the dK/dV pass;
//   bwd_dkdv  one workgroup per key tile, looping over the query tiles that keep it
//             (column lists); the waves split the pair into key groups (x query groups
//             for fp32, whose partial dK/dV are summed through LDS at the end); Q_i and
//             dO_i are staged in LDS.
// bf16 runs both passes on 64-row query tiles with four waves, small enough in LDS for two
// workgroups to share a CU, so that one hides the other's fixed cost (list lookups, first
// tile, fragment loads, epilogue). Tiles are at most 128 query rows and 64 keys; a larger
// mask block is two or four consecutive tiles over the same list entry (TileQueue).
#include <math.h>

#include <type_traits>

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
  const int32_t* row_order;  // optional scheduling orders (query blocks, key blocks)
  const int32_t* col_order;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  const bf16* kmean;  // bf16 dQ pass: mean key of every key tile [BH, tiles, D]
  int N, Tm, Tn, BH;
  int bq_block, bkv_block;  // rows / keys of a mask block (multiples of the kernels' tiles)
  int qsub, ksub;           // log2 of the query tiles per block and key tiles per key block
                            // (the loops over lists take them as template parameters)
  int rowterm;  // dQ pass: compute Dv = rowsum(dO * O) itself and store it in dvec
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
// Mean key of every key tile of BKVT keys (the last tile over its valid keys), fp32
// sums rounded once to bf16: the reference vectors of the bf16 dQ pass's corrections,
// formed once per call instead of in every query block that keeps the tile.
// One workgroup per (head, tile); TPR threads per row move 16-byte chunks.
// ------------------------------------------------------------------------------------
template <int D, int BKVT>
__global__ __launch_bounds__(256) void kmean_kernel(const bf16* __restrict__ k, bf16* __restrict__ out,
                                                    int N, int tiles) {
  constexpr int TPR = D / 8;    // threads per row
  constexpr int RP = 256 / TPR; // rows in flight
  __shared__ float red[RP][D];
  const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int lo = tile * BKVT, hi = min(N, lo + BKVT);
  const bf16* base = k + (size_t)bh * N * D;
  const int c = threadIdx.x % TPR, r0 = threadIdx.x / TPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r = lo + r0; r < hi; r += RP) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(base + (size_t)r * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
    for (int r = 0; r < RP; ++r) sum += red[r][threadIdx.x];
    out[((size_t)bh * tiles + tile) * D + threadIdx.x] = (bf16)(hi > lo ? sum / (float)(hi - lo) : 0.f);
  }
}

// ------------------------------------------------------------------------------------
// dQ: per query block, over its kept key blocks.
//   S^T = K Q^T, dP^T = V dO^T (A = K, V rows from LDS; B = Q, dO in registers),
//   dS^T = P^T * (dP^T - Dv), dQ^T += K^T dS^T (A = K^T via transpose reads).
//
// bf16 only: two rounding errors grow with a large component c_j shared by a block's keys
// (an attention-sink block, or keys with a smooth positional component), because each is
// multiplied by the keys:
//  * rounding dS to bf16 leaves sum_k r_k K_k, r = dS - bf16(dS), whose c_j part
//    (sum_k r_k) c_j is added back;
//  * the row term Dv carries the rounding of O, which shifts every dS_k by -P_k dDv. In
//    exact arithmetic sum_k dS_k = 0 over the row, so the measured T = sum_k dS_k equals
//    -dDv, and the shift's c_j part T sum_j P^blk_j c_j (P^blk_j = the row's mass on
//    block j) is removed at the end.
// What remains involves only K_k - c_j, so c_j is the block's mean key: it removes the
// shared part whatever its shape (a first-key reference also carries that key's own
// noise, which on keys with a smooth positional component left more error than no
// correction at all). The means come from kmean_kernel, once per call; wave 0 reads the
// next block's mean with the tile loads and copies it into LDS after the next barrier.
// Both terms are rank-one updates per block, w_j (x) c_j with
// w_j = sum_k r_k or P^blk_j. They are batched on the matrix unit, eight blocks at a
// time: each lane group g (16 lanes, a quarter of the block's keys) keeps its partial
// weights of the last eight blocks as the eight reduction slots 8g .. 8g + 7 of an MFMA
// operand W, and an LDS matrix C holds c_j of those blocks so that slot 8g + i of the
// other operand is c_i for every g. One MFMA per output tile then sums the partials over
// the groups and the blocks: acc += C^T W, pkc += C^T W'. The groups' partials of
// sum_k bf16(dS_k) come from the matrix unit too (a 0/1 operand times the packed dS), so
// sum_k r_k costs one add per element.
// ------------------------------------------------------------------------------------
template <typename T, int D, int BQ, int BKV, int KSUB, bool DENSE, int NW>
__global__ __launch_bounds__(64 * NW, sizeof(T) == 2 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int KTN = BKV / 16;  // 16-key tiles per key step (BQ x BKV tiles)
  constexpr int UPV = BKV / 32;  // 32-key reduction steps of the dQ product
  constexpr int QT = BQ / (16 * NW);  // 16-row query tiles per wave
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using KV = Tile<T, BKV, D>;
  constexpr bool kCorr = sizeof(T) == 2;
  using CM = Tile<T, 32, D>;  // c_j of one batch of eight blocks, four copies (bf16 only)
  // K/V stages in separate LDS variables, named statically (see the forward kernel). The
  // code also runs three stages (loads issued two blocks ahead, partial vmcnt waits), which
  // measured slower than two (with eight-wave workgroups, one per CU).
  constexpr int kStageBytes = 2 * KV::kBytes;
  constexpr int NS = 2;
  __shared__ __attribute__((aligned(1024))) char stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char stage1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char stage2[NS == 3 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) char cm0[kCorr ? CM::kBytes : 16];
  __shared__ __attribute__((aligned(1024))) char cm1[kCorr ? CM::kBytes : 16];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // paired XCDs; the tiles of one block stay on one XCD, sharing its L2
  const int pos = xcd_item_paired_tiles(blockIdx.x, (a.BH * a.Tm) << a.qsub, a.qsub);
  const int ppos = pos >> a.qsub;  // this query tile's block, in scheduling order
  const int item = a.row_order ? __builtin_amdgcn_readfirstlane(a.row_order[ppos]) : ppos;
  const int bh = item / a.Tm, qb = item % a.Tm;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const int q0 = qb * a.bq_block + (pos & ((1 << a.qsub) - 1)) * BQ + w * 16 * QT;

  constexpr bool dense = DENSE;
  const int cnt = dense ? (N + BKV - 1) / BKV : a.row_cnt[item] << KSUB;  // key steps
  static_assert(NS <= 3, "TileQueue reads two positions ahead");
  TileQueue<KSUB> bq;  // key tiles t .. t + NS - 1 (tile loads) and t + NS (being read)
  if (!dense) bq.init(a.row_idx + (size_t)item * a.Tn, a.row_cnt[item]);
  auto block_at = [&](int t, int i) { return dense ? t + i : bq.tile(t, i); };
  typename KV::template Plan<NW> plan;
  plan.init(w);
  auto issue = [&](char* stage, int j) {
    plan.issue_any(stage, K, j * BKV, N, w);
    plan.issue_any(stage + KV::kBytes, V, j * BKV, N, w);
  };
  if (cnt > 0) issue(stage0, block_at(0, 0));
  if (NS == 3 && cnt > 1) issue(stage1, block_at(0, 1));
  // mean key rows: lane c of each 16-lane group of wave 0 holds 16-byte chunk c of the
  // mean of the block whose C row is written next (read one block ahead, with the tiles)
  static_assert(!kCorr || CM::kChunks <= 16, "a bf16 key row is at most 16 chunks");
  const bf16* KM = kCorr ? a.kmean + (size_t)bh * ((size_t)a.Tn << a.ksub) * D : nullptr;
  const int mc = l & 15;
  u32x4 mrow{0u, 0u, 0u, 0u};
  auto load_mean = [&](int j) {
    if (kCorr && w == 0 && mc < CM::kChunks)
      mrow = *reinterpret_cast<const u32x4*>(KM + (size_t)j * D + mc * 8);
  };
  if (cnt > 0) load_mean(block_at(0, 0));
  if constexpr (kCorr) {  // C starts at zero: unfilled rows meet zero weights
    const u32x4 z{0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < CM::kBytes; o += 64 * NW * 16) {
      *reinterpret_cast<u32x4*>(cm0 + o) = z;
      *reinterpret_cast<u32x4*>(cm1 + o) = z;
    }
  }

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
    if (a.rowterm) {
      // Dv = rowsum(dO * O) from the dO fragments already held (lane: 8 columns per ks)
      // and the same columns of O (o_f32 when given), summed over the 4 lanes of the row
      float part = 0.f;
      if (ok) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const size_t off = (size_t)row * D + ks * 32 + 8 * g;
          if (a.o_f32) {
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(a.o_f32 + head + off);
            const f32x4 o1 = *reinterpret_cast<const f32x4*>(a.o_f32 + head + off + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              part += E::to_f32(df[qt][ks][e]) * o0[e];
              part += E::to_f32(df[qt][ks][4 + e]) * o1[e];
            }
          } else {
            const F of = load_row8<T>((const T*)a.o + head + off);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += E::to_f32(df[qt][ks][e]) * E::to_f32(of[e]);
          }
        }
      }
      dv[qt] = sum4(part);
      if (ok && g == 0) a.dvec[(size_t)bh * N + row] = dv[qt];
    } else {
      dv[qt] = ok ? a.dvec[(size_t)bh * N + row] : 0.f;
    }
  }

  f32x4 acc[DT][QT], pkc[DT][QT];
  float tpart[QT];
  // correction weights: wr / wp hold this lane group's partial sum_k r_k / P^blk of the
  // last eight blocks (bf16, the newest in element 7): at the end of a batch of eight,
  // element i is block i of the batch.
  u32x4 wr[QT], wp[QT];
  // the last block's sums, taken into the weights at the start of the next block (so the
  // wait for the 0/1-operand MFMA is off the block's critical path)
  float pend_tb[QT], pend_pb[QT];
  f32x4 pend_cs[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    tpart[qt] = 0.f;
    wr[qt] = wp[qt] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pkc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // A operand with ones where the reduction slot belongs to lane group m % 4 (row m): row
  // m of C sums the column over the slots of lane group m % 4 only, so element g of lane
  // group g receives the sum over its own 16 keys
  F ones = E::zero();
  if constexpr (kCorr) {
    if (g == (c16 & 3))
#pragma unroll
      for (int e = 0; e < 8; ++e) ones[e] = (T)1.0f;
  }

  auto shift_in = [&](u32x4& r, float x) {  // drop element 0, append bf16(x) as element 7
    const unsigned b = __builtin_bit_cast(unsigned short, (bf16)x);
    r = u32x4{__builtin_amdgcn_alignbit(r[1], r[0], 16), __builtin_amdgcn_alignbit(r[2], r[1], 16),
              __builtin_amdgcn_alignbit(r[3], r[2], 16), __builtin_amdgcn_alignbit(b, r[3], 16)};
  };
  auto take_pending = [&]() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      tpart[qt] += pend_tb[qt];
      const float bsum = g == 0 ? pend_cs[qt][0] : g == 1 ? pend_cs[qt][1] : g == 2 ? pend_cs[qt][2] : pend_cs[qt][3];
      shift_in(wr[qt], pend_tb[qt] - bsum);
      shift_in(wp[qt], pend_pb[qt]);
    }
  };
  // C rows: block i of a batch at rows 4 g' + i (i < 4) or 16 + 4 g' + (i - 4), g' = 0..3,
  // so that the transpose reads of every lane group see c_0 .. c_7 in slots 0..7
  auto flush = [&](const char* cmb) {
    if constexpr (kCorr) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F ca;
        CM::read_col4(cmb, 0, dt * 16, ca, 0);
        CM::read_col4(cmb, 16, dt * 16, ca, 1);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          acc[dt][qt] = E::mma(ca, __builtin_bit_cast(F, wr[qt]), acc[dt][qt]);
          pkc[dt][qt] = E::mma(ca, __builtin_bit_cast(F, wp[qt]), pkc[dt][qt]);
        }
      }
    }
  };

  // Per-wave direct-to-LDS loads of one block (K and V), for the partial waits below.
  constexpr int kBlockLoads = 2 * KV::template Plan<NW>::kLoads;
  // block t: its stage is `stage`; the loads of block t + NS - 1 go to `next`
  auto block = [&](int t, const char* stage, char* next) {
    const int j = block_at(t, 0);
    const int ahead = t + NS - 1;
    const int jn = block_at(t, NS - 1);
    const int jm = NS == 2 ? jn : block_at(t, 1);  // the next block, for its mean key
    if (!dense) bq.advance(t);
    // this wave's loads of block t have landed: with three stages the loads of block
    // t + 1 (issued later; loads complete in order) may still be in flight
    if (NS == 3 && t + 1 < cnt) wait_vmem_below<kBlockLoads>();
    else wait_vmem();
    lds_barrier();  // ... and every other wave's; block t-1 is no longer being read
    if constexpr (kCorr) {
      // this block's mean key (loaded during the previous block), four copies (one per
      // lane group of wave 0): rows 4 g' + i (i = t mod 8 < 4) or 16 + 4 g' + (i - 4)
      if (w == 0 && mc < CM::kChunks) {
        const int i = t & 7;
        CM::store_chunk(((t >> 3) & 1) ? cm1 : cm0, (i < 4 ? i : 12 + i) + 4 * (l >> 4), mc, mrow);
      }
    }
    if (ahead < cnt) issue(next, jn);
    if (t + 1 < cnt) load_mean(jm);
    const char* Kb = stage;
    const char* Vb = stage + KV::kBytes;
    if constexpr (kCorr) {
      // the previous batch's C rows are now visible to every wave; its weights are the
      // shift registers' contents (this block has not shifted in yet)
      if (t > 0) take_pending();  // the previous block's weights
      if ((t & 7) == 0 && t > 0) flush(((t >> 3) & 1) ? cm0 : cm1);
    }

    f32x4 s[KTN][QT], dp[KTN][QT];
#pragma unroll
    for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) {
        const F ka = KV::read_row8(Kb, kt * 16 + c16, ks * 32 + 8 * g);
        const F va = KV::read_row8(Vb, kt * 16 + c16, ks * 32 + 8 * g);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          s[kt][qt] = E::mma(ka, qf[qt][ks], s[kt][qt]);
          dp[kt][qt] = E::mma(va, df[qt][ks], dp[kt][qt]);
        }
      }
    }
    // keys past N exist only in the last, partial key block: P = 0 there
    if ((j + 1) * BKV > N) {
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j * BKV + kt * 16 + 4 * g + e >= N)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[kt][qt][e] = -INFINITY;
    }
    float pb[QT], tb[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) pb[qt] = tb[qt] = 0.f;
#pragma unroll
    for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][qt][e], a.scale_log2, -lse2[qt]));
          const float ds = p * (dp[kt][qt][e] - dv[qt]);
          s[kt][qt][e] = ds;  // dS^T
          if (kCorr) {
            pb[qt] += p;
            tb[qt] += ds;
          }
        }

    f32x4 cs[QT];  // element g: sum of bf16(dS_k) over this lane group's keys
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) cs[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < UPV; ++u) {
      F pf[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        pf[qt] = E::pack(s[2 * u][qt], s[2 * u + 1][qt]);
        if (kCorr) cs[qt] = E::mma(ones, pf[qt], cs[qt]);
      }
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
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // this group's share of sum_k r_k: its fp32 partial of sum_k dS_k minus its partial
        // of sum_k bf16(dS_k) (small: bf16 keeps the weight's own rounding negligible);
        // taken into the weights at the start of the next block
        pend_tb[qt] = tb[qt];
        pend_pb[qt] = pb[qt];
        pend_cs[qt] = cs[qt];
      }
    }
  };
  if constexpr (NS == 3) {
    for (int t = 0; t < cnt; t += 3) {
      block(t, stage0, stage2);
      if (t + 1 < cnt) block(t + 1, stage1, stage0);
      if (t + 2 < cnt) block(t + 2, stage2, stage1);
    }
  } else {
    for (int t = 0; t < cnt; t += 2) {
      block(t, stage0, stage1);
      if (t + 1 < cnt) block(t + 1, stage1, stage0);
    }
  }

  if constexpr (kCorr) {
    if (cnt > 0) {
      take_pending();  // the last block's weights
      // complete the last batch with zero weights, then apply it
      const int last = cnt - 1;
      for (int t = last + 1; (t & 7) != 0; ++t)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          shift_in(wr[qt], 0.f);
          shift_in(wp[qt], 0.f);
        }
      __syncthreads();  // the last C rows written are visible
      flush(((last >> 3) & 1) ? cm1 : cm0);
    }
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
// NW waves split each (key block, query tile) pair into KW key groups of 16 KT keys
// times QW = NW / KW query groups, so each wave reads only its rows of Q_i and dO_i from
// LDS (in both layouts). bf16: four waves of 16 keys over 64-row query tiles (QW = 1),
// 246 registers and 65.5 KB of LDS, two workgroups per CU (two waves per SIMD); 32 keys
// per wave would halve the LDS traffic per matrix instruction but needs more registers
// than two waves per SIMD allow. Q_i, dO_i and the row statistics stream into LDS with
// direct-to-LDS loads, one tile ahead.
//   S = Q K^T, dP = dO V^T (A = Q, dO rows from LDS; B = K, V in registers),
//   dS = P * (dP - Dv), dV^T += dO^T P, dK^T += Q^T dS (A via transpose reads).
// With QW > 1 (fp32) the query groups' partial sums are added through LDS at the end.
// ------------------------------------------------------------------------------------
template <typename T, int D, int BQ, int BKV, int QSUB, bool DENSE, int NW, int KT>
__global__ __launch_bounds__(64 * NW, sizeof(T) == 2 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int KW = BKV / (16 * KT);    // key groups (KT 16-key tiles per wave)
  constexpr int QW = NW / KW;            // query groups
  constexpr int MT = BQ / QW / 16;       // 16-row query tiles per wave
  static_assert(MT % 2 == 0, "the dV/dK products reduce over 32 query rows at a time");
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  using QTile = Tile<T, BQ, D>;
  // A stage holds Q_i, dO_i and the statistics of its rows (LSE_i, then Dv_i, fp32), all
  // streamed in by direct-to-LDS loads one block ahead.
  constexpr int kStats = 2 * BQ * 4;
  constexpr int kStage = 2 * QTile::kBytes + kStats;
  constexpr int NS = 2 * kStage <= 160 * 1024 ? 2 : 1;  // one stage only if two do not fit
  __shared__ __attribute__((aligned(1024))) char stage0[kStage];
  __shared__ __attribute__((aligned(1024))) char stage1[NS == 2 ? kStage : 16];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w % KW, qh = w / KW;
  const int pos = xcd_item(blockIdx.x, (a.BH * a.Tn) << a.ksub);
  const int ppos = pos >> a.ksub;  // this key tile's block, in scheduling order
  const int item = a.col_order ? __builtin_amdgcn_readfirstlane(a.col_order[ppos]) : ppos;
  const int bh = item / a.Tn, kb = item % a.Tn;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* dO = (const T*)a.dout + head;
  const float* LSE = a.lse + (size_t)bh * N;
  const float* DV = a.dvec + (size_t)bh * N;
  const int k0 = kb * a.bkv_block + (pos & ((1 << a.ksub) - 1)) * BKV + kh * 16 * KT;  // first key of this wave
  const int qrow0 = qh * (BQ / QW);        // first query row of this wave within a block

  constexpr bool dense = DENSE;
  const int cnt = dense ? (N + BQ - 1) / BQ : a.col_cnt[item] << QSUB;  // query tiles
  TileQueue<QSUB> bq;  // query tiles t, t + 1 (next tile load) and t + 2 (being read)
  if (!dense) bq.init(a.col_idx + (size_t)item * a.Tm, a.col_cnt[item]);
  auto block_at = [&](int t, int i) { return dense ? t + i : bq.tile(t, i); };
  typename QTile::template Plan<NW> plan;
  plan.init(w);
  auto issue = [&](char* stage, int i) {
    plan.issue_any(stage, Q, i * BQ, N, w);
    plan.issue_any(stage + QTile::kBytes, dO, i * BQ, N, w);
    // statistics: 2 BQ floats, 64 per load (4 bytes per lane), wave w issues load w;
    // rows past N are clamped here and given P = 0 in compute()
    if (w < 2 * BQ / 64) {
      const int e = w * 64 + l;
      const int r = min(i * BQ + (e % BQ), N - 1);
      const float* src = (e < BQ ? LSE : DV) + r;
      lds_dma4(src, __builtin_amdgcn_readfirstlane(lds_address(stage + 2 * QTile::kBytes + w * 256)));
    }
  };
  if (cnt > 0) issue(stage0, block_at(0, 0));

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
    const char* St = stage + 2 * QTile::kBytes;
    // this lane's rows of the statistics: queries i*BQ + qrow0 + 16 mt + 4 g + e
    f32x4 l4[MT], d4[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int rl = qrow0 + mt * 16 + 4 * g;  // row within the block
      l4[mt] = *reinterpret_cast<const f32x4*>(St + rl * 4);
      d4[mt] = *reinterpret_cast<const f32x4*>(St + (BQ + rl) * 4);
      if ((i + 1) * BQ > N) {  // last, partial query block: rows past N get P = 0
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i * BQ + rl + e >= N) {
            l4[mt][e] = INFINITY;
            d4[mt][e] = 0.f;
          }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) l4[mt][e] *= kLog2e;
    }
    // Two halves of the wave's rows (u): S, dP, P, dS of half u (scores), then the dV/dK
    // products of half u; the products of half 0 are issued after the scores of half 1,
    // which do not depend on them.
    F pf[MT / 2][KT], sf[MT / 2][KT];
    auto scores = [&](int u) __attribute__((always_inline)) {
      f32x4 s[2][KT], dp[2][KT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          s[h][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int mt = 2 * u + h;
          const F qa = QTile::read_row8(Qb, qrow0 + mt * 16 + c16, ks * 32 + 8 * g);
          const F da = QTile::read_row8(Db, qrow0 + mt * 16 + c16, ks * 32 + 8 * g);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            s[h][kt] = E::mma(qa, kf[kt][ks], s[h][kt]);
            dp[h][kt] = E::mma(da, vf[kt][ks], dp[h][kt]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int mt = 2 * u + h;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][kt][e], a.scale_log2, -l4[mt][e]));
            s[h][kt][e] = p;
            dp[h][kt][e] = p * (dp[h][kt][e] - d4[mt][e]);
          }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        pf[u][kt] = E::pack(s[0][kt], s[1][kt]);
        sf[u][kt] = E::pack(dp[0][kt], dp[1][kt]);
      }
    };
    // dV^T += dO^T P ; dK^T += Q^T dS over the 32 queries of half u
    auto products = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        F dot, qtr;
        QTile::read_col4(Db, qrow0 + 32 * u, dt * 16, dot, 0);
        QTile::read_col4(Db, qrow0 + 32 * u + 16, dt * 16, dot, 1);
        QTile::read_col4(Qb, qrow0 + 32 * u, dt * 16, qtr, 0);
        QTile::read_col4(Qb, qrow0 + 32 * u + 16, dt * 16, qtr, 1);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          dv[dt][kt] = E::mma(dot, pf[u][kt], dv[dt][kt]);
          dk[dt][kt] = E::mma(qtr, sf[u][kt], dk[dt][kt]);
        }
      }
    };
    scores(0);
#pragma unroll
    for (int u = 1; u < MT / 2; ++u) {
      scores(u);
      products(u - 1);
    }
    products(MT / 2 - 1);
  };

  if constexpr (NS == 2) {
    auto block = [&](int t, const char* stage, char* next) {
      const int i = block_at(t, 0);
      const int in = block_at(t, 1);
      if (!dense) bq.advance(t);
      wait_vmem();
      lds_barrier();
      if (t + 1 < cnt) issue(next, in);
      compute(i, stage);
    };
    for (int t = 0; t < cnt; t += 2) {
      block(t, stage0, stage1);
      if (t + 1 < cnt) block(t + 1, stage1, stage0);
    }
  } else {
    for (int t = 0; t < cnt; ++t) {
      const int i = block_at(t, 0);
      const int in = block_at(t, 1);
      if (!dense) bq.advance(t);
      wait_vmem();
      lds_barrier();
      compute(i, stage0);
      lds_barrier();  // every wave is done with the only stage
      if (t + 1 < cnt) issue(stage0, in);
    }
  }

  // add the query groups: waves with qh = r > 0 hand their partial sums to qh = 0 via
  // LDS, one group and one tensor at a time (DT * KT * 1 KB per wave)
  f32x4* xfer = reinterpret_cast<f32x4*>(stage0);
  auto reduce = [&](f32x4 (&acc)[DT][KT]) {
#pragma unroll
    for (int r = 1; r < QW; ++r) {
      __syncthreads();
      if (qh == r) {
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

// dK/dV work split: bf16 runs four waves of one 16-key tile each over 64-row query tiles
// (launch_bwd); fp32 runs waves of two 16-key tiles.
template <typename T, int BQ>
constexpr int dkdv_key_tiles() { return sizeof(T) == 2 ? 1 : 2; }
// dK/dV waves of the 128-row-tile form (fp32): 2 x 16-row query tiles per wave at least
// (the products reduce over 32 rows)
template <typename T, int BQ, int BKV>
constexpr int dkdv_waves() {
  return (sizeof(T) == 2 ? 8 : 4) / (BKV == 32 && BQ == 64 ? 2 : 1);
}
// dQ waves: 16 rows each (bf16), except with 32-key tiles at D = 64, where a K/V tile is only
// four 1 KB loads (32 rows each then); fp32: four waves
template <typename T, int D, int BQ, int BKV>
constexpr int dq_waves() {
  return sizeof(T) == 2 ? (D == 64 && BKV == 32 ? BQ / 32 : BQ / 16) : 4;
}

hipError_t launch_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                      const float* o_f32, const float* lse, const void* dout, const spa2_blockmask* m, void* dq,
                      void* dk, void* dv, float* dvec, void* kmean, int stages, hipStream_t st) {
  BwdArgs a{q, k, v, o, o_f32, lse, dout,
            m ? m->row_cnt : nullptr, m ? m->row_idx : nullptr,
            m ? m->col_cnt : nullptr, m ? m->col_idx : nullptr,
            m ? m->row_order : nullptr, m ? m->col_order : nullptr,
            dq, dk, dv, dvec, (const bf16*)kmean, s.N, s.Tm, s.Tn, s.BH(), s.BQ, s.BKV, s.qsub(), s.ksub(), 0,
            (float)(1.4426950408889634 / sqrt((double)s.D)), (float)(1.0 / sqrt((double)s.D))};
  const int tpr = s.D * (s.dtype == SPA2_BF16 ? 2 : 4) / 16;
  const int rpb = 256 / tpr;
  const size_t rows = (size_t)s.BH() * s.N;
  const dim3 gpre((unsigned)((rows + rpb - 1) / rpb));
  const dim3 gq((s.BH() * s.Tm) << s.qsub()), gk((s.BH() * s.Tn) << s.ksub());
  const int tiles = bwd_key_tiles(s);
#define SPA2_BWD(T, D, BQ, BK)                                                       \
  do {                                                                               \
    auto launch_dq = [&](auto bqt, auto nqt, dim3 grid) {                            \
      constexpr int BQT = decltype(bqt)::value, NQ = decltype(nqt)::value;           \
      if constexpr (sizeof(T) == 2)                                                  \
        kmean_kernel<D, BK><<<dim3((unsigned)(s.BH() * tiles)), 256, 0, st>>>(       \
            (const bf16*)k, (bf16*)kmean, s.N, tiles);                                \
      if (!m) bwd_dq_kernel<T, D, BQT, BK, 0, true, NQ><<<grid, 64 * NQ, 0, st>>>(a); \
      else if (s.ksub()) bwd_dq_kernel<T, D, BQT, BK, 1, false, NQ><<<grid, 64 * NQ, 0, st>>>(a); \
      else bwd_dq_kernel<T, D, BQT, BK, 0, false, NQ><<<grid, 64 * NQ, 0, st>>>(a);  \
    };                                                                               \
    auto run_dq = [&]() {                                                            \
      if constexpr (sizeof(T) == 2) { /* 64-row tiles: two workgroups share a CU */  \
        a.qsub = a.bq_block == 256 ? 2 : a.bq_block == 128 ? 1 : 0;                  \
        launch_dq(std::integral_constant<int, 64>{},                                 \
                  std::integral_constant<int, dq_waves<T, D, 64, BK>()>{},           \
                  dim3((unsigned)((s.BH() * s.Tm) << a.qsub)));                      \
        a.qsub = s.qsub();                                                           \
      } else {                                                                       \
        launch_dq(std::integral_constant<int, BQ>{},                                 \
                  std::integral_constant<int, dq_waves<T, D, BQ, BK>()>{}, gq);      \
      }                                                                              \
    };                                                                               \
    if (stages & kBwdPrep) bwd_pre_kernel<T, D><<<gpre, 256, 0, st>>>(a);            \
    if (stages & kBwdDqRow) { /* dQ and the row term first: dK/dV reads dvec */      \
      a.rowterm = 1;                                                                 \
      run_dq();                                                                      \
      a.rowterm = 0;                                                                 \
    }                                                                                \
    if (stages & kBwdDkdv) {                                                         \
      constexpr int kt = dkdv_key_tiles<T, BQ>();                                    \
      if constexpr (sizeof(T) == 2) {                                                \
        /* 64-row query tiles, 4 waves: two workgroups share a CU */                 \
        constexpr int nw = 4;                                                        \
        if (!m) bwd_dkdv_kernel<T, D, 64, BK, 0, true, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
        else if (a.bq_block == 128) bwd_dkdv_kernel<T, D, 64, BK, 1, false, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
        else if (a.bq_block == 64) bwd_dkdv_kernel<T, D, 64, BK, 0, false, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
        else bwd_dkdv_kernel<T, D, 64, BK, 2, false, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
      } else {                                                                       \
        constexpr int nw = dkdv_waves<T, BQ, BK>();                                  \
        if (!m) bwd_dkdv_kernel<T, D, BQ, BK, 0, true, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
        else if (s.qsub()) bwd_dkdv_kernel<T, D, BQ, BK, 1, false, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
        else bwd_dkdv_kernel<T, D, BQ, BK, 0, false, nw, kt><<<gk, 64 * nw, 0, st>>>(a); \
      }                                                                              \
    }                                                                                \
    if (stages & kBwdDq) run_dq();                                                   \
  } while (0)
#define SPA2_BWD_BK(T, D, BQ)                                                        \
  do {                                                                               \
    if (s.bkv_tile() == 32) SPA2_BWD(T, D, BQ, 32); else SPA2_BWD(T, D, BQ, 64);     \
  } while (0)
#define SPA2_BWD_BQ(T, D)                                                            \
  do {                                                                               \
    if (s.bq_tile() == 64) SPA2_BWD_BK(T, D, 64); else SPA2_BWD_BK(T, D, 128);       \
  } while (0)
  if (s.dtype == SPA2_BF16) {
    if (s.D == 64) SPA2_BWD_BQ(bf16, 64); else SPA2_BWD_BQ(bf16, 128);
  } else {
    if (s.D == 64) SPA2_BWD_BQ(float, 64); else SPA2_BWD_BQ(float, 128);
  }
#undef SPA2_BWD_BQ
#undef SPA2_BWD_BK
#undef SPA2_BWD
  return hipGetLastError();
}

}  // namespace spa2
