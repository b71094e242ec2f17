// awq_dequant: W[K, N] float16 = float16_RNE((q - z) * s), bit-exact.
// awq_dequant_gidx: the same with row k's zero/scale row taken from a
// row-to-group map (the g_idx of the GPTQ tuple on the page "Predibase
// Lorax Linear Layer Factory", Description) instead of k / g.
//
// Per-group dequantisation of the page "Predibase Lorax AWQ WQLinear"
// (Description: eight 4-bit values per int32 along the output dimension,
// group_size rows per scale/zero row).  Memory-bound: 0.5 byte in and 2 bytes
// out per weight, plus the (cached) group rows.  One thread per packed word;
// consecutive threads take consecutive words of a row, so loads of qweight
// and the 16-byte stores of W are fully coalesced.
#include "awq_device.h"

namespace awq {
namespace {

template <bool VEC>
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const _Float16* __restrict__ sc, _Float16* __restrict__ w,
    int K, int NW, int N, int g, const int32_t* __restrict__ gidx, int G) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= K * NW) return;
  const int k = idx / NW;
  const int c = idx - k * NW;
  // Contiguous groups, or the map's entry; an entry outside [0, G) reads
  // zero points and scales of zero (that row dequantises to zeros).
  int grp = gidx ? gidx[k] : k / g;
  const bool gok = grp >= 0 && grp < G;
  if (!gok) grp = 0;
  const uint32_t word = qw[idx];
  const uint32_t zw = gok ? qz[grp * NW + c] : 0u;
  const _Float16* srow = sc + grp * N + 8 * c;
  half8_t s = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  if (gok) {
    if (VEC) {
      s = *reinterpret_cast<const half8_t*>(srow);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] = srow[j];
    }
  }
  half8_t out;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (word >> (4 * j)) & 0xF;
    const int z = (zw >> (4 * j)) & 0xF;
    // q - z is an integer in [-15, 15]; its product with a float16 is exact
    // in float32, so the conversion is the only rounding.
    out[j] = static_cast<_Float16>(static_cast<float>(q - z) * static_cast<float>(s[j]));
  }
  _Float16* dst = w + k * N + 8 * c;
  if (VEC) {
    *reinterpret_cast<half8_t*>(dst) = out;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = out[j];
  }
}

}  // namespace

hipError_t launch_dequant(const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, _Float16* w, int K, int N, int g,
                          const int32_t* gidx, int G, hipStream_t stream) {
  const int NW = N / 8;
  const long long words = static_cast<long long>(K) * NW;
  const int blocks = static_cast<int>((words + 255) / 256);
  const bool vec = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(w) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                       qweight, qzeros, scales, w, K, NW, N, g, gidx, G);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                       qweight, qzeros, scales, w, K, NW, N, g, gidx, G);
  return hipGetLastError();
}

}  // namespace awq
