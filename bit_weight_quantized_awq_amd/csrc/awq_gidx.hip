// Reorders behind the sorted-weight forward (awq_gemm_sorted).
//
// A row-to-group map (the g_idx of the GPTQ tuple on the page "Predibase
// Lorax Linear Layer Factory", Description) becomes an ordinary grouped
// weight once, at load time: its rows are sorted by group and cut into
// blocks that each lie in one group (null rows pad a group's last block
// when the groups are uneven), and every block gets its group's zero and
// scale row.  The grouped kernels then run at full speed; each forward only
// has to bring the columns of x into the same order, since
//   sum_k x[m, k] w[k, n] = sum_j x[m, perm[j]] w[perm[j], n]
// with x read as 0 for a null row (perm entry -1).  Both reorders are pure
// data movement (HBM-bound): 16-byte stores, and the reads of x go to one
// row of x at a time, which stays in L2.
#include "awq_device.h"

namespace awq {
namespace {

// dst[j, :] = src[idx[j], :] for row-major matrices of row_words 32-bit
// words (src_rows rows in, dst_rows out); VEC moves 4 words (16 bytes) per
// thread.  An index outside [0, src_rows) writes a row of zeros.
template <bool VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t* __restrict__ src,
                                                          int src_rows,
                                                          const int32_t* __restrict__ idx,
                                                          uint32_t* __restrict__ dst,
                                                          int dst_rows, int row_words) {
  const int per_row = VEC ? row_words / 4 : row_words;
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(dst_rows) * per_row) return;
  const int j = static_cast<int>(i / per_row);
  const int c = static_cast<int>(i - static_cast<long long>(j) * per_row);
  const int r = idx[j];
  const bool ok = r >= 0 && r < src_rows;
  if (VEC) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (ok) v = reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r) * row_words)[c];
    reinterpret_cast<u32x4*>(dst + static_cast<size_t>(j) * row_words)[c] = v;
  } else {
    dst[static_cast<size_t>(j) * row_words + c] =
        ok ? src[static_cast<size_t>(r) * row_words + c] : 0u;
  }
}

// xp[m, j] = x[m, perm[j]] for x (M, Kin) and xp (M, Kout), row-major
// float16; VEC forms 8 consecutive outputs (one 16-byte store) per thread.
// An entry of perm outside [0, Kin) gives 0.
template <bool VEC>
__global__ __launch_bounds__(256) void gather_cols_kernel(const _Float16* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          _Float16* __restrict__ xp, int M,
                                                          int Kin, int Kout) {
  const int per_row = VEC ? Kout / 8 : Kout;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(M) * per_row) return;
  const int m = static_cast<int>(idx / per_row);
  const int c = static_cast<int>(idx - static_cast<long long>(m) * per_row);
  const _Float16* xrow = x + static_cast<size_t>(m) * Kin;
  if (VEC) {
    const u32x4 p0 = reinterpret_cast<const u32x4*>(perm)[2 * c];
    const u32x4 p1 = reinterpret_cast<const u32x4*>(perm)[2 * c + 1];
    half8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = static_cast<int>(i < 4 ? p0[i] : p1[i - 4]);
      v[i] = (r >= 0 && r < Kin) ? xrow[r] : static_cast<_Float16>(0.f);
    }
    *reinterpret_cast<half8_t*>(xp + static_cast<size_t>(m) * Kout + 8 * c) = v;
  } else {
    const int r = perm[c];
    xp[static_cast<size_t>(m) * Kout + c] =
        (r >= 0 && r < Kin) ? xrow[r] : static_cast<_Float16>(0.f);
  }
}

// The same reorder for many rows.  ROWS consecutive rows of x and all of
// perm are copied into LDS with asynchronous 16-byte direct-to-LDS loads
// (all in flight at once, one wait), then every thread forms 8 consecutive
// outputs of each row from LDS.  Scattered 2-byte reads from global memory
// cost one cache-line lookup per lane; from LDS a few bank cycles per
// instruction.  Needs Kin % 8 == 0, Kout % 8 == 0, x, perm and xp 16-byte
// aligned and lds_gather_bytes(ROWS, Kin, Kout) bytes of LDS.
constexpr uint32_t kDmaChunk = 1024;   // bytes one wave's direct-to-LDS load moves
__host__ __device__ constexpr uint32_t round_chunk(uint32_t b) {
  return (b + kDmaChunk - 1) / kDmaChunk * kDmaChunk;
}
__host__ __device__ constexpr uint32_t lds_gather_bytes(int rows, int Kin, int Kout) {
  return round_chunk(static_cast<uint32_t>(rows) * Kin * 2u) +
         round_chunk(static_cast<uint32_t>(Kout) * 4u);
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
                                                              int Kin, int Kout) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int m0 = blockIdx.x * ROWS;
  const int rows = min(ROWS, M - m0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t xbytes = static_cast<uint32_t>(rows) * Kin * 2u;
  const uint32_t pbytes = static_cast<uint32_t>(Kout) * 4u;
  const uint32_t xregion = round_chunk(static_cast<uint32_t>(ROWS) * Kin * 2u);
  // Loads past each range read zero (the LDS regions are whole chunks).
  copy_to_lds(make_rsrc(x + static_cast<size_t>(m0) * Kin, xbytes), smem, xbytes, wave, lane);
  copy_to_lds(make_rsrc(perm, pbytes), smem + xregion, pbytes, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const _Float16* xs = reinterpret_cast<const _Float16*>(smem);
  const u32x4* ps = reinterpret_cast<const u32x4*>(smem + xregion);
  const int chunks = Kout / 8;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 p0 = ps[2 * c];
    const u32x4 p1 = ps[2 * c + 1];
    int src[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      src[i] = static_cast<int>(i < 4 ? p0[i] : p1[i - 4]);
      ok[i] = src[i] >= 0 && src[i] < Kin;
      if (!ok[i]) src[i] = 0;
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (r < rows) {
        half8_t v;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = ok[i] ? xs[r * Kin + src[i]] : static_cast<_Float16>(0.f);
        *reinterpret_cast<half8_t*>(xp + static_cast<size_t>(m0 + r) * Kout + 8 * c) = v;
      }
    }
  }
}

constexpr uint32_t kLdsMax = 160 * 1024;
constexpr int kGatherLdsMinRows = 32;   // below this the direct form is as fast

int blocks_for(long long items) { return static_cast<int>((items + 255) / 256); }

}  // namespace

hipError_t launch_gather_rows(const uint32_t* src, int src_rows, const int32_t* idx,
                              uint32_t* dst, int dst_rows, int row_words, hipStream_t stream) {
  const bool vec = row_words % 4 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  const long long items = static_cast<long long>(dst_rows) * (vec ? row_words / 4 : row_words);
  if (vec)
    hipLaunchKernelGGL(gather_rows_kernel<true>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       src, src_rows, idx, dst, dst_rows, row_words);
  else
    hipLaunchKernelGGL(gather_rows_kernel<false>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       src, src_rows, idx, dst, dst_rows, row_words);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const _Float16* x, const int32_t* perm, _Float16* xp, int M,
                              int Kin, int Kout, hipStream_t stream) {
  const bool vec = Kout % 8 == 0 && reinterpret_cast<uintptr_t>(perm) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(xp) % 16 == 0;
  // Rows per work-group: 4 while the stage leaves room for a second
  // work-group per CU, else fewer; rows past the LDS size take the direct form.
  int rows = 0;
  if (lds_gather_bytes(4, Kin, Kout) <= 96 * 1024) rows = 4;
  else if (lds_gather_bytes(2, Kin, Kout) <= 128 * 1024) rows = 2;
  else if (lds_gather_bytes(1, Kin, Kout) <= kLdsMax) rows = 1;
  if (vec && Kin % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
      M >= kGatherLdsMinRows && rows > 0) {
    const size_t lds = lds_gather_bytes(rows, Kin, Kout);
    const dim3 grid((M + rows - 1) / rows);
    switch (rows) {
      case 4:
        hipLaunchKernelGGL(gather_cols_lds_kernel<4>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, Kin, Kout);
        break;
      case 2:
        hipLaunchKernelGGL(gather_cols_lds_kernel<2>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, Kin, Kout);
        break;
      default:
        hipLaunchKernelGGL(gather_cols_lds_kernel<1>, grid, dim3(256), lds, stream, x, perm, xp,
                           M, Kin, Kout);
        break;
    }
    return hipGetLastError();
  }
  const long long items = static_cast<long long>(M) * (vec ? Kout / 8 : Kout);
  if (vec)
    hipLaunchKernelGGL(gather_cols_kernel<true>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       x, perm, xp, M, Kin, Kout);
  else
    hipLaunchKernelGGL(gather_cols_kernel<false>, dim3(blocks_for(items)), dim3(256), 0, stream,
                       x, perm, xp, M, Kin, Kout);
  return hipGetLastError();
}

}  // namespace awq
