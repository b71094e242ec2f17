// Prefill W4A16 GEMM (large M): LDS-tiled matrix-core GEMM whose weight tile
// is dequantised into LDS, with the bias epilogue fused in.
//
// The product of the page "Predibase Lorax AWQ WQLinear" (Description, forward
// step 2) is compute-bound at prefill sizes, so the dequantisation must be
// amortised over many rows of x: each 256 x 128 output tile dequantises its
// 64 x 128 weight slab once per K step into LDS and feeds it to all 256 rows.
//
// * Work-group: 256 threads = 4 waves in a 2 x 2 grid; each wave owns a
//   128 x 64 sub-tile = 4 x 2 blocks of v_mfma_f32_32x32x16_f16 (fp32
//   accumulators, 128 per lane).
// * LDS: x tile [256][64] and weight tile [128 columns][64 k], both with the
//   k index contiguous and rows padded to 144 bytes so the 16-byte operand
//   reads of a wave hit distinct banks; double-buffered (108 KiB).
// * Global loads for the next K step are issued before the matrix-core work
//   on the current one; x moves as 16-byte loads, packed words as one word per
//   thread for four consecutive rows (64-byte row segments per 16 threads).
// * Dequantisation (exact, per weight): byte-shuffle two rows' words so
//   nibble j of both sits in the halves of one register, OR into float16
//   1024.0, subtract (1024 + z) and multiply by s with packed float16
//   arithmetic: float16_RNE((q - z) * s), the same value awq_dequant writes.
// * Tile order: work-group ids are remapped so that each of the 8 XCDs (which
//   receive ids round-robin) works on a contiguous range of tiles that share
//   rows of x, keeping that slab resident in the XCD's L2.
#include "awq_device.h"
#include "awq_plan.h"

namespace awq {
namespace {

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr int BK = kPrefillBK;
constexpr int LDA = BK + 8;  // halfs per LDS row (144 bytes)

__global__ __launch_bounds__(256) void prefill_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    int M, int K, int N, int g, int n_tiles) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * LDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int mt = bid / n_tiles;
  const int nt = bid - mt * n_tiles;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  const int NW = N >> 3;
  const int nkt = (K + BK - 1) / BK;

  // Weight loader: word column bwc of the tile, rows 4*brb .. 4*brb+3.
  const int bwc = tid & 15;
  const int brb = tid >> 4;
  const int bc = (n0 >> 3) + bwc;
  const bool bcvalid = bc < NW;

  uint4 areg[8];
  uint32_t breg[4];
  uint32_t bz;
  half8_t bs;

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3;
      const int kc = idx & 7;
      const int m = m0 + row;
      const int k = k0 + 8 * kc;
      areg[i] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(x + m * K + k)
                                 : make_uint4(0u, 0u, 0u, 0u);
    }
    const int kr = k0 + 4 * brb;
    const bool rv = bcvalid && kr < K;
    if (rv) {
      const uint32_t* src = qw + kr * NW + bc;
#pragma unroll
      for (int r = 0; r < 4; ++r) breg[r] = src[r * NW];
      const int grp = kr / g;
      bz = qz[grp * NW + bc];
      bs = *reinterpret_cast<const half8_t*>(sc + grp * N + 8 * bc);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) breg[r] = 0u;
      bz = 0u;
      bs = half8_t{};
    }
  };

  auto store_tile = [&](int buf) {
    _Float16* Ab = As[buf];
    _Float16* Bb = Bs[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3;
      const int kc = idx & 7;
      *reinterpret_cast<uint4*>(Ab + row * LDA + 8 * kc) = areg[i];
    }
    const uint32_t lo0 = pair_bytes_lo(breg[0], breg[1]);
    const uint32_t hi0 = pair_bytes_hi(breg[0], breg[1]);
    const uint32_t lo1 = pair_bytes_lo(breg[2], breg[3]);
    const uint32_t hi1 = pair_bytes_hi(breg[2], breg[3]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t s0 = (j < 4) ? lo0 : hi0;
      const uint32_t s1 = (j < 4) ? lo1 : hi1;
      const int sh = 4 * (j & 3);
      const half2_t z2 = as_h2(zero_pair(bz, j));
      const half2_t s2 = half2_t{bs[j], bs[j]};
      const half2_t d0 = (as_h2(magic_pair(s0, sh)) - z2) * s2;
      const half2_t d1 = (as_h2(magic_pair(s1, sh)) - z2) * s2;
      *reinterpret_cast<uint2*>(Bb + (8 * bwc + j) * LDA + 4 * brb) =
          make_uint2(as_u32(d0), as_u32(d1));
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int frow = lane & 31;
  const int fk = 8 * (lane >> 5);

  auto compute = [&](int buf) {
    const _Float16* Ab = As[buf];
    const _Float16* Bb = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      half8_t af[4], bf[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const half8_t*>(Ab + (128 * wm + 32 * mi + frow) * LDA +
                                                   16 * ks + fk);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *reinterpret_cast<const half8_t*>(Bb + (64 * wn + 32 * ni + frow) * LDA +
                                                   16 * ks + fk);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt + 1);
    compute(kt & 1);
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: 32x32 block output, lane holds column (lane % 32) and rows
  // 8*(r/4) + 4*(lane/32) + r%4 of register r.
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int col = n0 + 64 * wn + 32 * ni + frow;
    if (col >= N) continue;
    const float b = bias ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 128 * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) y[row * N + col] = static_cast<_Float16>(acc[mi][ni][r] + b);
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, const _Float16* bias, _Float16* y,
                          int M, int K, int N, int g, int m_tiles, int n_tiles,
                          hipStream_t stream) {
  hipLaunchKernelGGL(prefill_kernel, dim3(m_tiles * n_tiles), dim3(256), 0, stream,
                     x, qweight, qzeros, scales, bias, y, M, K, N, g, n_tiles);
  return hipGetLastError();
}

}  // namespace awq
