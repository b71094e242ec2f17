// General W4A16 GEMM for any legal shape and alignment (any group size, K not
// a multiple of 8, unaligned x or scales).  Plain fp32 FMA, no matrix cores:
// this is the correctness fallback, not a fast path.
//
// It also runs the forward under an arbitrary row-to-group map (awq_gemm_gidx:
// the g_idx of the GPTQ tuple on the page "Predibase Lorax Linear Layer
// Factory", Description), looking row k's group up instead of k / g.
//
// Work-group tile: 16 rows x 256 columns, one output column per thread.  A
// 16 x 64 slab of x is staged in LDS as fp32; each thread dequantises its
// column's weights exactly (float16_RNE((q - z) * s)) and accumulates the 16
// rows in fp32.  The epilogue adds the bias in fp32 and rounds once.
#include "awq_device.h"

namespace awq {
namespace {

constexpr int kRows = 16;
constexpr int kKChunk = 64;

__global__ __launch_bounds__(256) void generic_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    int M, int K, int N, int g, const int32_t* __restrict__ gidx, int G, int n_tiles) {
  __shared__ float xs[kRows][kKChunk];
  const int NW = N / 8;
  const int mt = blockIdx.x / n_tiles;
  const int n = (blockIdx.x - mt * n_tiles) * 256 + threadIdx.x;
  const int m0 = mt * kRows;
  const int c = n >> 3;
  const int shift = 4 * (n & 7);
  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kKChunk) {
    for (int i = threadIdx.x; i < kRows * kKChunk; i += 256) {
      const int r = i / kKChunk, kk = i - r * kKChunk;
      const int m = m0 + r, k = k0 + kk;
      xs[r][kk] = (m < M && k < K) ? static_cast<float>(x[m * K + k]) : 0.f;
    }
    __syncthreads();
    if (n < N) {
      const int kend = min(kKChunk, K - k0);
      for (int kk = 0; kk < kend; ++kk) {
        const int k = k0 + kk;
        // An entry of the map outside [0, G) reads zero point 0 and scale 0.
        const int grp = gidx ? gidx[k] : k / g;
        const bool gok = grp >= 0 && grp < G;
        const int q = (qw[k * NW + c] >> shift) & 0xF;
        const int z = gok ? (qz[grp * NW + c] >> shift) & 0xF : 0;
        const float s = gok ? static_cast<float>(sc[grp * N + n]) : 0.f;
        const float w = static_cast<float>(static_cast<_Float16>(static_cast<float>(q - z) * s));
#pragma unroll
        for (int r = 0; r < kRows; ++r) acc[r] = fmaf(xs[r][kk], w, acc[r]);
      }
    }
    __syncthreads();
  }
  if (n < N) {
    const float b = bias ? static_cast<float>(bias[n]) : 0.f;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int m = m0 + r;
      if (m < M) y[m * N + n] = static_cast<_Float16>(acc[r] + b);
    }
  }
}

}  // namespace

hipError_t launch_generic(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, const _Float16* bias, _Float16* y,
                          int M, int K, int N, int g, const int32_t* gidx, int G,
                          hipStream_t stream) {
  const int n_tiles = (N + 255) / 256;
  const int m_tiles = (M + kRows - 1) / kRows;
  hipLaunchKernelGGL(generic_kernel, dim3(n_tiles * m_tiles), dim3(256), 0, stream,
                     x, qweight, qzeros, scales, bias, y, M, K, N, g, gidx, G, n_tiles);
  return hipGetLastError();
}

}  // namespace awq
