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

// The same reorder for many rows.  ROWS consecutive rows of x and all of
// perm are copied into LDS with asynchronous 16-byte direct-to-LDS loads
// (all in flight at once, one wait), then every thread forms 8 consecutive
// outputs of each row from LDS.  Scattered 2-byte reads from global memory
// cost one cache-line lookup per lane; from LDS a few bank cycles per
// instruction.  Needs K % 8 == 0, x, perm and xp 16-byte aligned and
// lds_gather_bytes(ROWS, K) bytes of LDS.
constexpr uint32_t kDmaChunk = 1024;   // bytes one wave's direct-to-LDS load moves
__host__ __device__ constexpr uint32_t round_chunk(uint32_t b) {
  return (b + kDmaChunk - 1) / kDmaChunk * kDmaChunk;
}
__host__ __device__ constexpr uint32_t lds_gather_bytes(int rows, int K) {
  return round_chunk(static_cast<uint32_t>(rows) * K * 2u) + round_chunk(static_cast<uint32_t>(K) * 4u);
}

__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t bytes,
                                            int wave, int lane) {
  for (uint32_t off = static_cast<uint32_t>(wave) * kDmaChunk; off < bytes; off += 4 * kDmaChunk)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(lds + off), 16,
        off + static_cast<uint32_t>(lane) * 16u, 0, 0, 0);
}

template <int ROWS>
__global__ __launch_bounds__(256) void gather_cols_lds_kernel(const _Float16* __restrict__ x,
                                                              const int32_t* __restrict__ perm,
                                                              _Float16* __restrict__ xp, int M,
                                                              int K) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int m0 = blockIdx.x * ROWS;
  const int rows = min(ROWS, M - m0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t xbytes = static_cast<uint32_t>(rows) * K * 2u;
  const uint32_t pbytes = static_cast<uint32_t>(K) * 4u;
  const uint32_t xregion = round_chunk(static_cast<uint32_t>(ROWS) * K * 2u);
  // Loads past each range read zero (the LDS regions are whole chunks).
  copy_to_lds(make_rsrc(x + static_cast<size_t>(m0) * K, xbytes), smem, xbytes, wave, lane);
  copy_to_lds(make_rsrc(perm, pbytes), smem + xregion, pbytes, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const _Float16* xs = reinterpret_cast<const _Float16*>(smem);
  const u32x4* ps = reinterpret_cast<const u32x4*>(smem + xregion);
  const int chunks = K / 8;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 p0 = ps[2 * c];
    const u32x4 p1 = ps[2 * c + 1];
    int src[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      src[i] = static_cast<int>(i < 4 ? p0[i] : p1[i - 4]);
      ok[i] = src[i] >= 0 && src[i] < K;
      if (!ok[i]) src[i] = 0;
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (r < rows) {
        half8_t v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ok[i] ? xs[r * K + src[i]] : static_cast<_Float16>(0.f);
        *reinterpret_cast<half8_t*>(xp + static_cast<size_t>(m0 + r) * K + 8 * c) = v;
      }
    }
  }
}

constexpr uint32_t kLdsMax = 160 * 1024;
constexpr int kGatherLdsMinRows = 32;   // below this the direct form is as fast

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
  // Rows per work-group: 4 while the stage leaves room for a second
  // work-group per CU, else fewer; rows past the LDS size take the direct form.
  int rows = 0;
  if (lds_gather_bytes(4, K) <= 96 * 1024) rows = 4;
  else if (lds_gather_bytes(2, K) <= 128 * 1024) rows = 2;
  else if (lds_gather_bytes(1, K) <= kLdsMax) rows = 1;
  if (vec && reinterpret_cast<uintptr_t>(x) % 16 == 0 && M >= kGatherLdsMinRows && rows > 0) {
    const size_t lds = lds_gather_bytes(rows, K);
    const dim3 grid((M + rows - 1) / rows);
    switch (rows) {
      case 4:
        hipLaunchKernelGGL(gather_cols_lds_kernel<4>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, K);
        break;
      case 2:
        hipLaunchKernelGGL(gather_cols_lds_kernel<2>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, K);
        break;
      default:
        hipLaunchKernelGGL(gather_cols_lds_kernel<1>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, K);
        break;
    }
    return hipGetLastError();
  }
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
