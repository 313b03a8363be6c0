// Error decomposition of a sparse forward against the dense forward (diagnostics).
//
// rainbus summary, "技术新颖性": O_dense - O_sparse splits into the dropped mass
// (p * (1 - m)) V and the renormalisation (1 - 1/tau)(p * m) V, tau = the dense mass on
// the kept keys. With (p * m) V = tau O_sparse and tau = exp(LSE_sparse - LSE_dense), the
// per-element terms are O_dense - tau O_sparse and (tau - 1) O_sparse.
//
// One workgroup per (head, 64-row slice): each thread walks whole 16-byte chunks of the
// slice's rows (D/4 chunks per row), accumulates the four absolute sums in double, the
// workgroup reduces them and adds them to the head's four totals.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace spa2 {

namespace {

constexpr int kRowsPerGroup = 64;

__global__ __launch_bounds__(64) void zero_terms_kernel(double* terms, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < n) terms[i] = 0.0;
}

template <int D>
__global__ __launch_bounds__(256) void error_terms_kernel(const float* __restrict__ os,
                                                          const float* __restrict__ ls,
                                                          const float* __restrict__ od,
                                                          const float* __restrict__ ld,
                                                          double* __restrict__ terms,
                                                          float* __restrict__ tau_out, int N,
                                                          int slices) {
  constexpr int kChunks = D / 4;
  const int bh = blockIdx.x / slices, slice = blockIdx.x % slices;
  const int r0 = slice * kRowsPerGroup, rows = min(kRowsPerGroup, N - r0);
  const size_t base = (size_t)bh * N + r0;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int f = threadIdx.x; f < rows * kChunks; f += 256) {
    const int r = f / kChunks, c = f % kChunks;
    const float lsp = ls[base + r];
    const float tau = lsp == -INFINITY ? 0.f : __expf(lsp - ld[base + r]);
    if (c == 0 && tau_out) tau_out[base + r] = tau;
    const f32x4 s = *reinterpret_cast<const f32x4*>(os + (base + r) * D + 4 * c);
    const f32x4 d = *reinterpret_cast<const f32x4*>(od + (base + r) * D + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double sv = s[e], dv = d[e], t = tau;
      acc[0] += fabs(dv);
      acc[1] += fabs(dv - sv);
      acc[2] += fabs(dv - t * sv);
      acc[3] += fabs((t - 1.0) * sv);
    }
  }
  __shared__ double red[4][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double x = acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    if (lane == 0) red[w][i] = x;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const double t = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] +
                     red[3][threadIdx.x];
    atomicAdd(&terms[(size_t)bh * 4 + threadIdx.x], t);
  }
}

}  // namespace

hipError_t launch_error_terms(const Shape& s, const float* os, const float* ls, const float* od,
                              const float* ld, double* terms, float* tau, hipStream_t st) {
  const int n = s.BH() * 4;
  zero_terms_kernel<<<(n + 63) / 64, 64, 0, st>>>(terms, n);
  const int slices = (s.N + kRowsPerGroup - 1) / kRowsPerGroup;
  const dim3 grid(s.BH() * slices);
  if (s.D == 64) error_terms_kernel<64><<<grid, 256, 0, st>>>(os, ls, od, ld, terms, tau, s.N, slices);
  else error_terms_kernel<128><<<grid, 256, 0, st>>>(os, ls, od, ld, terms, tau, s.N, slices);
  return hipGetLastError();
}

}  // namespace spa2
