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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define SPA2_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Max over the four lanes that share (l % 16): lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
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
