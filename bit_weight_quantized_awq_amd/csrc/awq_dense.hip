// Unquantised float16 skinny linear: the baseline that the W4A16 decode is
// measured against.  y[m, n] = sum_k x[m, k] * w[n, k] (+ bias[n]), w of
// shape (N, K) row-major as F.linear takes it -- the page "Predibase Lorax
// Linear Layer Factory" (Description: FastLinear, whose ROCm variant sends
// single-token products at K = 8192, N = 1280 or 7168 to a custom skinny
// kernel).  1 <= M <= 4.
//
// Bound: HBM (2 bytes per weight, read once).  Work-group = 8 waves, one
// output row n per wave: the wave streams w[n, :] with 16-byte loads (64
// lanes x 8 halves = 512 consecutive weights, 1 KiB per load, four loads in
// flight per lane), takes x from LDS (staged once per work-group), and
// accumulates packed float16 dot products in fp32; the lanes' partial sums
// meet through a cross-lane reduction and lane 0 writes y.  Deterministic:
// the summation order is fixed.
#include "awq_device.h"

namespace awq {
namespace {

constexpr int kDenseWaves = 8;

__device__ __forceinline__ float dot8(half8_t a, half8_t b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t pa = {a[2 * i], a[2 * i + 1]};
    const half2_t pb = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pa, pb, acc, false);
  }
  return acc;
}

template <int MR>
__global__ __launch_bounds__(64 * kDenseWaves) void dense_gemv_kernel(
    const _Float16* __restrict__ x, const _Float16* __restrict__ w,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y, int K, int N) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  _Float16* xs = reinterpret_cast<_Float16*>(smem);
  // Stage x (MR x K halves, K % 8 == 0) in LDS.
  for (int i = threadIdx.x; i < MR * K / 8; i += 64 * kDenseWaves)
    reinterpret_cast<half8_t*>(xs)[i] = reinterpret_cast<const half8_t*>(x)[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kDenseWaves + static_cast<int>(threadIdx.x >> 6);
  if (n >= N) return;
  const half8_t* wr = reinterpret_cast<const half8_t*>(w + static_cast<size_t>(n) * K);
  const int chunks = K / 8;   // 16-byte chunks per row
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
  int c = lane;
  for (; c + 192 < chunks; c += 256) {
    half8_t wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) wv[u] = __builtin_nontemporal_load(wr + c + 64 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int m = 0; m < MR; ++m)
        acc[m] = dot8(wv[u], reinterpret_cast<const half8_t*>(xs + m * K)[c + 64 * u], acc[m]);
  }
  for (; c < chunks; c += 64) {
    const half8_t wv = __builtin_nontemporal_load(wr + c);
#pragma unroll
    for (int m = 0; m < MR; ++m)
      acc[m] = dot8(wv, reinterpret_cast<const half8_t*>(xs + m * K)[c], acc[m]);
  }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
  if (lane == 0) {
    const float b = bias ? static_cast<float>(bias[n]) : 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m) y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(acc[m] + b);
  }
}

}  // namespace

hipError_t launch_dense_gemv(const _Float16* x, const _Float16* w, const _Float16* bias,
                             _Float16* y, int M, int K, int N, hipStream_t stream) {
  const dim3 grid((N + kDenseWaves - 1) / kDenseWaves);
  const dim3 block(64 * kDenseWaves);
  const size_t lds = static_cast<size_t>(M) * K * 2;
  switch (M) {
    case 1: hipLaunchKernelGGL(dense_gemv_kernel<1>, grid, block, lds, stream, x, w, bias, y, K, N); break;
    case 2: hipLaunchKernelGGL(dense_gemv_kernel<2>, grid, block, lds, stream, x, w, bias, y, K, N); break;
    case 3: hipLaunchKernelGGL(dense_gemv_kernel<3>, grid, block, lds, stream, x, w, bias, y, K, N); break;
    case 4: hipLaunchKernelGGL(dense_gemv_kernel<4>, grid, block, lds, stream, x, w, bias, y, K, N); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace awq
