// Device-side building blocks shared by the gfx950 kernels.
//
// MFMA layout facts used throughout (checked on the device with an in-bounds probe):
//   v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32 / v_mfma_f64_16x16x4_f64:
//     operand A: lane l supplies row (l % 16), operand B: lane l supplies column (l % 16);
//     lane group g = l / 16 supplies its own slice of the reduction dimension.
//     fp32 result C: lane l holds C[4 * g + e][l % 16] for e = 0..3;
//     fp64 result C: lane l holds C[g + 4 * e][l % 16] for e = 0..3.
//   The reduction slots only have to agree between A and B, so every "fragment" below
//   is 8 values per lane whose slot s in group g means the same k in A and B.
//   ds_read_b64_tr_b16: within each 16-lane group, source lane s that points at row
//     (s / 4), columns 4 * (s % 4) .. +3 of a row-major 16-bit tile makes output lane j
//     receive column j of those 4 rows (element e = row e). This yields transposed MFMA
//     operands directly from row-major LDS tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define SPA2_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(size_t)(const SPA2_LDS char*)p;
}
// Direct-to-LDS loads (global_load_lds): lane l's 16 (or 4) bytes from g land at
// lds + 16 l (4 l); lds must be wave-uniform. They are written as inline asm on purpose:
// the compiler's wait-count pass treats an outstanding builtin direct-to-LDS load as an
// LDS access that completes out of order, and then waits for every LDS read with
// lgkmcnt(0) until the load is done (which serialises the operand reads of the block
// being computed with the matrix instructions). The asm writes no register (M0 aside), so
// nothing the compiler allocates can be overwritten in flight; completion is waited for
// explicitly with wait_vmem() (vmcnt(0)) before the barrier that publishes the tile, and
// extra outstanding loads only make the compiler's own vmcnt waits stricter.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// Cross-lane exchange without LDS: v_permlane16_swap / v_permlane32_swap applied to two
// copies of x leave, in every lane l, the values of lanes {l, l^16} (resp. {l, l^32}).
__device__ __forceinline__ float xchg16(float x, bool take_max) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float a = __builtin_bit_cast(float, (unsigned)r[0]);
  const float b = __builtin_bit_cast(float, (unsigned)r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xchg32(float x, bool take_max) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __builtin_bit_cast(float, (unsigned)r[0]);
  const float b = __builtin_bit_cast(float, (unsigned)r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
// Max / sum over the four lanes that share (l % 16): lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float max4(float x) { return xchg32(xchg16(x, true), true); }
__device__ __forceinline__ float sum4(float x) { return xchg32(xchg16(x, false), false); }

// Work item for workgroup `bid` of `items`: consecutive items go to the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs), so the query blocks of one
// head share that XCD's L2 for their K/V tiles.
__device__ __forceinline__ int xcd_item(int bid, int items) {
  const int q = items >> 3, r = items & 7, x = bid & 7, slot = bid >> 3;
  return x * q + min(x, r) + slot;
}

// The same ranges, but XCDs 2k and 2k + 1 walk the union of their two ranges together,
// alternating items (a bijection: the first XCD of a pair never holds fewer items than the
// second). The query-block passes (forward, dQ) use it: each XCD still runs one head's
// blocks at a time, while only four heads' K/V tiles are live across the GPU instead of
// eight, which the memory-side cache keeps better at long sequence lengths (forward
// 2.5% faster at 75,600 tokens, 1.8% at 32,760; dQ 2.6%; the key-block dK/dV pass is 2.4%
// slower this way and keeps xcd_item).
__device__ __forceinline__ int xcd_item_paired(int bid, int items) {
  const int q = items >> 3, r = items & 7, x = bid & 7, slot = bid >> 3;
  const int x0 = x & ~1;
  return x0 * q + min(x0, r) + 2 * slot + (x & 1);
}

// The paired walk for work items that are 2^sub consecutive tiles of one block (items =
// blocks << sub): the two XCDs of a pair alternate whole blocks, so a block's tiles run on
// one XCD and share its L2. A bijection when items is a multiple of 8 << sub (each XCD's
// range is then whole blocks); otherwise the plain contiguous ranges of xcd_item.
__device__ __forceinline__ int xcd_item_paired_tiles(int bid, int items, int sub) {
  if (sub == 0) return xcd_item_paired(bid, items);
  if (items & ((8 << sub) - 1)) return xcd_item(bid, items);
  const int q = items >> 3, x = bid & 7, slot = bid >> 3;
  const int x0 = x & ~1;
  return x0 * q + ((2 * (slot >> sub) + (x & 1)) << sub) + (slot & ((1 << sub) - 1));
}

// The kept-block list of one work item, read ahead with scalar loads. The lists are not
// written while a kernel runs, so they are read through the constant address space: the
// wait for an entry is an lgkmcnt wait, never a wait for the direct-to-LDS tile loads in
// flight (a vector load of the entry would complete only after those, since vector memory
// operations complete in issue order). q[i] is the block at position t + i of the list
// (i <= AHEAD; 0 past the end); advance() moves from t to t + 1 and starts reading the
// entry AHEAD + 1 positions ahead. t must be wave-uniform.
template <int AHEAD>
struct BlockQueue {
  const __attribute__((address_space(4))) int32_t* list;
  int cnt;
  int q[AHEAD + 1];
  __device__ __forceinline__ void init(const int32_t* l, int cnt_) {
    list = (const __attribute__((address_space(4))) int32_t*)l;
    cnt = cnt_;
#pragma unroll
    for (int i = 0; i <= AHEAD; ++i) q[i] = i < cnt ? list[i] : 0;
  }
  __device__ __forceinline__ void advance(int t) {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) q[i] = q[i + 1];
    const int n = t + 1 + AHEAD;
    q[AHEAD] = n < cnt ? list[n] : 0;
  }
};

// Tiles of a kept-block list when every kept block covers 2^S consecutive tiles of the
// kernel (S = 0, 1 or 2; e.g. S = 1 for 128-key blocks run as two 64-key tiles, S = 2 for
// 256-row blocks run as four 64-row tiles): tile t is sub-tile (t mod 2^S) of list entry
// t >> S. tile(t, i) is the tile at position t + i (i <= 2; entries past the list read as
// block 0); advance(t) moves from t to t + 1. t must be wave-uniform. S is a template
// parameter so that the plain case (S = 0) is exactly BlockQueue, with no branch in the
// loop.
template <int S>
struct TileQueue {
  static_assert(S >= 0 && S <= 2, "up to four tiles per block");
  BlockQueue<2> bq;
  __device__ __forceinline__ void init(const int32_t* l, int blocks) { bq.init(l, blocks); }
  __device__ __forceinline__ int tile(int t, int i) const {
    if constexpr (S == 0) {
      return bq.q[i];
    } else {
      const int u = (t & ((1 << S) - 1)) + i;  // at most 2^S + 1: entry index u >> S <= 1
      return (bq.q[u >> S] << S) + (u & ((1 << S) - 1));
    }
  }
  __device__ __forceinline__ void advance(int t) {
    if constexpr (S == 0) bq.advance(t);
    else if ((t & ((1 << S) - 1)) == (1 << S) - 1) bq.advance(t >> S);
  }
};

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left unconstrained): this wave's outstanding
// vector memory operations, including direct-to-LDS loads, have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0xF70); }
// Workgroup barrier for LDS tiles filled by direct-to-LDS loads. __syncthreads() (and a
// workgroup fence on LDS) makes every wave wait for all of its outstanding direct-to-LDS
// loads, including those issued ahead for later blocks; here the caller first waits for
// the loads it needs (vmcnt), this wave's own LDS accesses are completed (lgkmcnt(0)),
// and the barrier is an s_barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): at most the N most recent vector memory operations of this wave are
// still outstanding (loads complete in issue order), so everything issued earlier is done.
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// ------------------------------------------------------------------------------------
// Element traits: fragment type, MFMA step, conversions.
// ------------------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  using frag = bf16x8;  // 8 bf16 per lane = one 16x16x32 MFMA operand
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag pack(f32x4 lo, f32x4 hi) {
    frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (bf16)lo[e];
      r[4 + e] = (bf16)hi[e];
    }
    return r;
  }
  __device__ static __forceinline__ frag zero() {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)0.0f;
    return r;
  }
  __device__ static __forceinline__ float to_f32(bf16 x) { return (float)x; }
};

template <>
struct Elem<float> {
  using frag = f32x8;  // 8 fp32 per lane = eight 16x16x4 MFMA steps
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ frag pack(f32x4 lo, f32x4 hi) {
    frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = lo[e];
      r[4 + e] = hi[e];
    }
    return r;
  }
  __device__ static __forceinline__ frag zero() {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 0.0f;
    return r;
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
};

// ------------------------------------------------------------------------------------
// Global memory: 8 consecutive elements (one fragment's worth along the row).
// ------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag load_row8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::frag*>(p);
}

// Streaming accesses (read or written once per kernel): non-temporal, so they do not push
// the K/V tiles that many workgroups re-read out of the caches.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag load_row8_stream(const T* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(q));
  } else {
    const u32x4 lo = __builtin_nontemporal_load(q), hi = __builtin_nontemporal_load(q + 1);
    return Elem<float>::pack(__builtin_bit_cast(f32x4, lo), __builtin_bit_cast(f32x4, hi));
  }
}
__device__ __forceinline__ void store4_stream(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store4_stream(bf16* p, f32x4 v) {
  const bf16x4 b{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, b),
                              reinterpret_cast<unsigned long long*>(p));
}

// ------------------------------------------------------------------------------------
// Row-major LDS tile of ROWS x D elements, 16-byte chunks XOR-swizzled per row so that
// both the 16-lane row reads (16 rows, one chunk) and the transpose reads (4 rows, two
// chunks per group) hit distinct banks.
// ------------------------------------------------------------------------------------
template <typename T, int ROWS, int D>
struct Tile {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
  static constexpr int kBytes = ROWS * kRowBytes;

  __device__ static __forceinline__ int swz(int row) {
    return ((((row & 7) << 1) | ((row >> 3) & 1))) & (kChunks - 1);
  }
  // byte offset of element column `col` in row `row`
  __device__ static __forceinline__ int offset(int row, int col) {
    const int byte = col * (int)sizeof(T);
    return row * kRowBytes + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
  }
  __device__ static __forceinline__ void store_chunk(char* base, int row, int chunk, u32x4 v) {
    *reinterpret_cast<u32x4*>(base + row * kRowBytes + ((chunk ^ swz(row)) << 4)) = v;
  }
  // Fill the tile straight from global memory (global_load_lds, 16 bytes per lane) with
  // rows row0 .. row0 + ROWS - 1 of a row-major [nrows, D] matrix; rows past nrows - 1 are
  // clamped to the last row (finite data that the callers mask or weight by zero). Every
  // wave of the workgroup (nwaves of them) issues kChunks * ROWS / (64 * nwaves) loads;
  // lane l of a load lands at its 16-byte slot, so the swizzle is applied to the source
  // address. Completion: wait_vmem() in each wave, then a workgroup barrier.
  __device__ static __forceinline__ void load_async(char* base, const T* src, int row0, int nrows,
                                                    int wave, int nwaves) {
    constexpr int kPerWave = kChunks * ROWS / 64;  // 16-byte loads per wave if one wave
    const int l = lane_id();
    for (int i = wave; i < kPerWave; i += nwaves) {
      const int f = i * 64 + l;  // flat 16-byte slot in the tile
      const int row = f / kChunks, pc = f % kChunks;
      const int grow = min(row0 + row, nrows - 1);
      const T* g = src + (size_t)grow * D + ((pc ^ swz(row)) * (16 / (int)sizeof(T)));
      lds_dma16(g, __builtin_amdgcn_readfirstlane(lds_address(base + i * 1024)));
    }
  }

  // The same fill for NW waves with the lane part of the source offsets computed once:
  // off[n] = element offset of this lane's slot for load n (wave-relative) within a
  // whole tile of ROWS valid rows.
  template <int NW>
  struct Plan {
    static constexpr int kLoads = kChunks * ROWS / 64 / NW;  // loads per wave per tile
    static_assert(kLoads * NW * 64 == kChunks * ROWS, "every wave issues the same loads");
    int off[kLoads];
    __device__ __forceinline__ void init(int wave) {
      const int l = lane_id();
#pragma unroll
      for (int n = 0; n < kLoads; ++n) {
        const int f = (n * NW + wave) * 64 + l;
        const int row = f / kChunks, pc = f % kChunks;
        off[n] = row * D + (pc ^ swz(row)) * (16 / (int)sizeof(T));
      }
    }
    // rows row0 .. row0 + ROWS - 1 all exist
    __device__ __forceinline__ void issue(char* base, const T* src, int row0, int wave) const {
      const T* tile = src + (size_t)row0 * D;
#pragma unroll
      for (int n = 0; n < kLoads; ++n)
        lds_dma16(tile + off[n],
                  __builtin_amdgcn_readfirstlane(lds_address(base + (n * NW + wave) * 1024)));
    }
    // general case: rows past nrows - 1 clamped
    __device__ __forceinline__ void issue_any(char* base, const T* src, int row0, int nrows,
                                              int wave) const {
      if (row0 + ROWS <= nrows) issue(base, src, row0, wave);
      else load_async(base, src, row0, nrows, wave, NW);
    }
  };
  // 8 consecutive elements [col, col+8) of one row (col multiple of 8)
  __device__ static __forceinline__ typename Elem<T>::frag read_row8(const char* base, int row, int col);
  // 4 elements down column `col`, rows r0 .. r0+3 (the transposed operand half)
  __device__ static __forceinline__ void read_col4(const char* base, int row0_of_group, int col0,
                                                    typename Elem<T>::frag& f, int half);
};

// Generic definitions (specialised by element size through if constexpr).
template <typename T, int ROWS, int D>
__device__ __forceinline__ typename Elem<T>::frag Tile<T, ROWS, D>::read_row8(const char* base,
                                                                              int row, int col) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(base + offset(row, col));
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(base + offset(row, col));
    const f32x4 hi = *reinterpret_cast<const f32x4*>(base + offset(row, col + 4));
    return Elem<float>::pack(lo, hi);
  }
}

// Transposed half-fragment. For lane (j = l % 16, g = l / 16) this fills slots
// [4*half, 4*half+4) with T[row0 + 4*g + e][col0 + j], e = 0..3.
template <typename T, int ROWS, int D>
__device__ __forceinline__ void Tile<T, ROWS, D>::read_col4(const char* base, int row0, int col0,
                                                           typename Elem<T>::frag& f, int half) {
  const int l = lane_id();
  const int g = l >> 4, s = l & 15;
  if constexpr (sizeof(T) == 2) {
    // source lane s points at row (row0 + 4g + s/4), columns col0 + 4*(s%4) .. +3
    const int row = row0 + 4 * g + (s >> 2);
    const int col = col0 + 4 * (s & 3);
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (SPA2_LDS s16x4*)(base + offset(row, col)));
    const bf16x4 b = __builtin_bit_cast(bf16x4, r);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * half + e] = b[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      f[4 * half + e] = *reinterpret_cast<const float*>(base + offset(row0 + 4 * g + e, col0 + s));
  }
}

}  // namespace spa2
