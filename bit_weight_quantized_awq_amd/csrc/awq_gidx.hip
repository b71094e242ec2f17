// Reorders behind the activation-order forward (awq_gemm_act_order).
//
// A row-to-group map (the g_idx of the GPTQ tuple on the page "Predibase
// Lorax Linear Layer Factory", Description) that gives every group the same
// number of rows is a grouped weight whose input rows were shuffled.  Sorting
// the rows by group once, at load time, turns it back into contiguous groups,
// which the grouped kernels run at full speed; each forward then only has to
// apply the same order to the columns of x, since
//   sum_k x[m, k] w[k, n] = sum_j x[m, perm[j]] w[perm[j], n].
// Both reorders are pure data movement (HBM-bound): 16-byte stores, and the
// reads of x go to one row of x at a time, which stays in L2.
#include "awq_device.h"

namespace awq {
namespace {

// dst[j, :] = src[perm[j], :] for a row-major (K, NW) matrix of 32-bit
// words; VEC moves 4 words (16 bytes) per thread.  An entry of perm outside
// [0, K) writes a row of zeros.
template <bool VEC>
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint32_t* __restrict__ src,
                                                           const int32_t* __restrict__ perm,
                                                           uint32_t* __restrict__ dst, int K,
                                                           int NW) {
  const int per_row = VEC ? NW / 4 : NW;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(K) * per_row) return;
  const int j = static_cast<int>(idx / per_row);
  const int c = static_cast<int>(idx - static_cast<long long>(j) * per_row);
  const int r = perm[j];
  const bool ok = r >= 0 && r < K;
  if (VEC) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (ok) v = reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r) * NW)[c];
    reinterpret_cast<u32x4*>(dst + static_cast<size_t>(j) * NW)[c] = v;
  } else {
    dst[static_cast<size_t>(j) * NW + c] = ok ? src[static_cast<size_t>(r) * NW + c] : 0u;
  }
}

// xp[m, j] = x[m, perm[j]] for a row-major (M, K) float16 matrix; VEC forms
// 8 consecutive outputs (one 16-byte store) per thread.  An entry of perm
// outside [0, K) gives 0.
template <bool VEC>
__global__ __launch_bounds__(256) void gather_cols_kernel(const _Float16* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          _Float16* __restrict__ xp, int M,
                                                          int K) {
  const int per_row = VEC ? K / 8 : K;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(M) * per_row) return;
  const int m = static_cast<int>(idx / per_row);
  const int c = static_cast<int>(idx - static_cast<long long>(m) * per_row);
  const _Float16* xrow = x + static_cast<size_t>(m) * K;
  if (VEC) {
    const u32x4 p0 = reinterpret_cast<const u32x4*>(perm)[2 * c];
    const u32x4 p1 = reinterpret_cast<const u32x4*>(perm)[2 * c + 1];
    half8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = static_cast<int>(i < 4 ? p0[i] : p1[i - 4]);
      v[i] = (r >= 0 && r < K) ? xrow[r] : static_cast<_Float16>(0.f);
    }
    *reinterpret_cast<half8_t*>(xp + static_cast<size_t>(m) * K + 8 * c) = v;
  } else {
    const int r = perm[c];
    xp[static_cast<size_t>(m) * K + c] = (r >= 0 && r < K) ? xrow[r] : static_cast<_Float16>(0.f);
  }
}

int blocks_for(long long items) { return static_cast<int>((items + 255) / 256); }

}  // namespace

hipError_t launch_permute_rows(const uint32_t* src, const int32_t* perm, uint32_t* dst, int K,
                               int NW, hipStream_t stream) {
  const bool vec = NW % 4 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  const long long items = static_cast<long long>(K) * (vec ? NW / 4 : NW);
  if (vec)
    hipLaunchKernelGGL(permute_rows_kernel<true>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       src, perm, dst, K, NW);
  else
    hipLaunchKernelGGL(permute_rows_kernel<false>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       src, perm, dst, K, NW);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const _Float16* x, const int32_t* perm, _Float16* xp, int M, int K,
                              hipStream_t stream) {
  const bool vec = K % 8 == 0 && reinterpret_cast<uintptr_t>(perm) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(xp) % 16 == 0;
  const long long items = static_cast<long long>(M) * (vec ? K / 8 : K);
  if (vec)
    hipLaunchKernelGGL(gather_cols_kernel<true>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       x, perm, xp, M, K);
  else
    hipLaunchKernelGGL(gather_cols_kernel<false>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       x, perm, xp, M, K);
  return hipGetLastError();
}

}  // namespace awq
