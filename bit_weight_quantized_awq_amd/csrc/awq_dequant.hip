// awq_dequant: W[K, N] float16 = float16_RNE((q - z) * s), bit-exact.
// awq_dequant_gidx: the same with row k's zero/scale row taken from a
// row-to-group map (the g_idx of the GPTQ tuple on the page "Predibase
// Lorax Linear Layer Factory", Description) instead of k / g.
//
// Per-group dequantisation of the page "Predibase Lorax AWQ WQLinear"
// (Description: eight 4-bit values per int32 along the output dimension,
// group_size rows per scale/zero row).  HBM-bound: 0.5 byte in and 2 bytes
// out per weight, plus the (cached) group rows.  Consecutive lanes take
// consecutive words, so every load of qweight and every 16-byte store of W
// covers consecutive memory.  With scales and W 16-byte aligned each thread
// takes four words, with all its loads in flight before one wait.
//
// The store form depends on the size of W.  A W that fits well inside the
// 256 MB last-level cache is written with ordinary stores.  The GEMM that
// usually reads W next then finds it there: dequantisation followed by a
// float16 GEMM ran 10-17 us faster at K = 8192, N = 7168 (W = 117 MB) than
// with nontemporal stores.  A larger W cannot stay there anyway, so it is
// streamed out with nontemporal stores.  That is the faster form on its own
// (30 vs 37.5 us at 117 MB; 109 vs 134 us at 470 MB), and it also won the
// GEMM pipeline at 235 MB and above.
#include "awq_device.h"

namespace awq {
namespace {

// Eight outputs of one packed word: q - z is an integer in [-15, 15] and
// the scale a float16, both exact in float16, so one IEEE float16 multiply
// rounds the exact product once, signed zeros included (q = z with a
// negative scale gives -0).  A float32 product converted to float16 is the
// same value, but the compiler may fuse that multiply and conversion into a
// mixed-precision FMA with a +0 addend, which turns -0 into +0.
__device__ __forceinline__ half8_t dequant_word(uint32_t word, uint32_t zw, half8_t s) {
  half8_t out;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (word >> (4 * j)) & 0xF;
    const int z = (zw >> (4 * j)) & 0xF;
    out[j] = static_cast<_Float16>(q - z) * s[j];
  }
  return out;
}

// One word per thread, element-aligned operands (the form for scales or W
// that are not 16-byte aligned).
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const _Float16* __restrict__ sc, _Float16* __restrict__ w,
    int K, int NW, int N, int g, const int32_t* __restrict__ gidx, int G) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= K * NW) return;
  const int k = idx / NW;
  const int c = idx - k * NW;
  // Contiguous groups, or the map's entry; an entry outside [0, G) reads
  // zero points and scales of zero (that row dequantises to +0).
  int grp = gidx ? gidx[k] : k / g;
  const bool gok = grp >= 0 && grp < G;
  if (!gok) grp = 0;
  const uint32_t zw = gok ? qz[grp * NW + c] : 0u;
  half8_t s = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  if (gok) {
    const _Float16* srow = sc + grp * N + 8 * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = srow[j];
  }
  const half8_t out = dequant_word(qw[idx], zw, s);
  _Float16* dst = w + k * N + 8 * c;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = out[j];
}

// Four words per thread, interleaved: work-group b takes the 1024 words
// starting at 1024*b of the flattened (K, NW) array, and its thread t the
// words 256*u + t (u = 0..3), so each load and store instruction of a wave
// covers consecutive memory.  Loads are unconditional (indices clamped into
// range, the out-of-range group cases selected away after the load), and a
// whole work-group (all but possibly the last) stores unconditionally too,
// so the twelve loads of a thread are all in flight before one wait.
// K * N < 2^31, so 32-bit indices suffice.  Needs scales and w 16-byte
// aligned.
constexpr int kWordsPerThread = 4;
constexpr uint32_t kWordsPerGroup = 256u * kWordsPerThread;

template <bool GIDX, bool WHOLE, bool NT>
__device__ __forceinline__ void dequant4_body(
    const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const _Float16* __restrict__ sc, _Float16* __restrict__ w, uint32_t total, uint32_t nw,
    uint32_t N, int g, const int32_t* __restrict__ gidx, int G) {
  constexpr int U = kWordsPerThread;
  const uint32_t base = blockIdx.x * kWordsPerGroup + threadIdx.x;
  uint32_t word[U], zw[U], k[U], c[U];
  int grp[U];
  half8_t s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t idx = WHOLE ? base + 256u * u : min(base + 256u * u, total - 1u);
    k[u] = idx / nw;
    c[u] = idx - k[u] * nw;
    word[u] = qw[idx];
    grp[u] = GIDX ? gidx[k[u]] : static_cast<int>(k[u]) / g;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t gr = (grp[u] >= 0 && grp[u] < G) ? static_cast<uint32_t>(grp[u]) : 0u;
    zw[u] = qz[gr * nw + c[u]];
    s[u] = *reinterpret_cast<const half8_t*>(sc + gr * N + 8u * c[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!WHOLE && base + 256u * u >= total) break;
    if (!(grp[u] >= 0 && grp[u] < G)) {     // an entry outside [0, G): zero point 0, scale 0
      zw[u] = 0u;
      s[u] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
    half8_t* dst = reinterpret_cast<half8_t*>(w + k[u] * N + 8u * c[u]);
    if (NT) __builtin_nontemporal_store(dequant_word(word[u], zw[u], s[u]), dst);
    else *dst = dequant_word(word[u], zw[u], s[u]);
  }
}

template <bool GIDX, bool NT>
__global__ __launch_bounds__(256) void dequant4_kernel(
    const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const _Float16* __restrict__ sc, _Float16* __restrict__ w,
    int K, int NW, int N, int g, const int32_t* __restrict__ gidx, int G) {
  const uint32_t total = static_cast<uint32_t>(K) * static_cast<uint32_t>(NW);
  if ((blockIdx.x + 1u) * kWordsPerGroup <= total)
    dequant4_body<GIDX, true, NT>(qw, qz, sc, w, total, static_cast<uint32_t>(NW),
                              static_cast<uint32_t>(N), g, gidx, G);
  else
    dequant4_body<GIDX, false, NT>(qw, qz, sc, w, total, static_cast<uint32_t>(NW),
                               static_cast<uint32_t>(N), g, gidx, G);
}

// W larger than this (three quarters of the last-level cache) is written
// with nontemporal stores.
constexpr long long kStreamOutBytes = 192ll << 20;

}  // namespace

hipError_t launch_dequant(const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, _Float16* w, int K, int N, int g,
                          const int32_t* gidx, int G, hipStream_t stream) {
  const int NW = N / 8;
  const long long words = static_cast<long long>(K) * NW;
  if (words == 0) return hipSuccess;
  const bool vec = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(w) % 16 == 0);
  if (vec) {
    const dim3 grid(static_cast<unsigned>((words + kWordsPerGroup - 1) / kWordsPerGroup));
    const bool stream_out = static_cast<long long>(K) * N * 2 > kStreamOutBytes;
    auto kernel = gidx ? (stream_out ? dequant4_kernel<true, true> : dequant4_kernel<true, false>)
                       : (stream_out ? dequant4_kernel<false, true> : dequant4_kernel<false, false>);
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, qweight, qzeros, scales, w, K, NW, N,
                       g, gidx, G);
  } else {
    hipLaunchKernelGGL(dequant_kernel, dim3(static_cast<unsigned>((words + 255) / 256)),
                       dim3(256), 0, stream, qweight, qzeros, scales, w, K, NW, N, g, gidx, G);
  }
  return hipGetLastError();
}

}  // namespace awq
