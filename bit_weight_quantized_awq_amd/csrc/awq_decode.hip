// Decode W4A16 skinny GEMM (M <= 16): split-K over the input dimension,
// matrix cores for the multiply-accumulate, deterministic cross-work-group
// reduction with the bias epilogue fused in.
//
// The page "Predibase Lorax AWQ WQLinear" (Description, forward step 2) runs
// this product in one extension call; at decode sizes the whole cost is the
// stream of packed weights from HBM (0.5 byte per weight), so the kernel is
// built around keeping that stream saturated:
//
// * Work-group = 4 waves covering 256 output columns (32 packed words per row,
//   128 contiguous bytes) and 2 x 32*STEPS input rows.  Waves 0/2 take words
//   0..15 of the tile, waves 1/3 words 16..31; waves 0/1 take the first half
//   of the rows, 2/3 the second.
// * Lane l of a wave owns word column (l % 16) and the 8-row block (l / 16) of
//   each 32-row step: it loads 8 words (one per row) of its column.  Each
//   row's 16 words are one 64-byte contiguous segment, and the two waves on
//   a row make it a full 128-byte line.  All loads of a wave are issued
//   before any arithmetic.
// * Unpack: two rows' words are byte-shuffled so that nibble j of both sits
//   in the two halves of one register; OR-ing into float16 1024.0 gives the
//   exact pair (1024 + q_k, 1024 + q_k+1), and a packed subtraction of
//   (1024 + z) gives the exact integers q - z as float16.
// * MFMA v_mfma_f32_16x16x32_f16: A = 16 rows of x (rows >= M are zero),
//   B = (q - z) for 16 columns x 32 rows, one MFMA per nibble position j, so
//   MFMA j covers columns 8*word + j.  Accumulation is fp32.
// * The scale is applied once per group to the fp32 group partial:
//   sum_k x*(q - z)*s = s * sum_k x*(q - z) exactly in real arithmetic; this
//   differs from rounding each dequantised weight to float16 only by that
//   rounding (relative 2^-11 per term).  A one-hot row still reproduces the
//   float16 dequantised weight exactly.
// * Reduction: the two K-halves of a work-group meet in LDS; work-groups write
//   fp32 partials to the workspace, take a ticket on their column tile, and
//   the last one sums the partials in split order (deterministic), adds the
//   bias, rounds to float16 and resets the ticket.
#include "awq_device.h"
#include "awq_plan.h"

namespace awq {
namespace {

template <int STEPS>
__global__ __launch_bounds__(256) void decode_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    float* __restrict__ partial, uint32_t* __restrict__ tickets,
    int M, int K, int N, int g, int G, int splits) {
  extern __shared__ float red[];  // [2][M][256] fp32
  __shared__ int s_last;

  const int NW = N >> 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1;
  const int wk = wave >> 1;
  const int n_tile = blockIdx.x / splits;
  const int split = blockIdx.x - n_tile * splits;
  const int col16 = lane & 15;  // MFMA column (B) / row (A) of this lane
  const int kb = lane >> 4;     // 8-row block within a 32-row step
  const int c = n_tile * 32 + wn * 16 + col16;
  const bool cvalid = c < NW;
  const int kw0 = split * (64 * STEPS) + wk * (32 * STEPS);
  const bool wave_has_rows = kw0 < K;

  // Group parameters of the wave's first step, fetched first.
  int cur = (G == 1) ? 0 : kw0 / g;
  uint32_t zw = 0;
  half8_t sv = {};
  if (wave_has_rows && cvalid) {
    zw = qz[cur * NW + c];
    sv = *reinterpret_cast<const half8_t*>(sc + cur * N + 8 * c);
  }

  // All x fragments and packed words of this wave.
  half8_t xa[STEPS];
  uint32_t wv[STEPS][8];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int kr = kw0 + 32 * s + 8 * kb;
    xa[s] = (col16 < M && kr < K) ? *reinterpret_cast<const half8_t*>(x + col16 * K + kr)
                                  : half8_t{};
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int kr = kw0 + 32 * s + 8 * kb;
    const bool rv = cvalid && kr < K;
    const uint32_t* src = qw + kr * NW + c;
#pragma unroll
    for (int r = 0; r < 8; ++r) wv[s][r] = rv ? src[r * NW] : 0u;
  }

  floatx4 acc[8], tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    tot[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t zp[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zp[j] = zero_pair(zw, j);

#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int k0 = kw0 + 32 * s;
    if (k0 >= K) break;
    const int grp = (G == 1) ? 0 : k0 / g;
    if (grp != cur) {
      // Close the previous group: scale its fp32 partial into the total.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot[j] += static_cast<float>(sv[j]) * acc[j];
        acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      cur = grp;
      zw = cvalid ? qz[grp * NW + c] : 0u;
      sv = cvalid ? *reinterpret_cast<const half8_t*>(sc + grp * N + 8 * c) : half8_t{};
#pragma unroll
      for (int j = 0; j < 8; ++j) zp[j] = zero_pair(zw, j);
    }
    uint32_t plo[4], phi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      plo[p] = pair_bytes_lo(wv[s][2 * p], wv[s][2 * p + 1]);
      phi[p] = pair_bytes_hi(wv[s][2 * p], wv[s][2 * p + 1]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t b;
      const half2_t z2 = as_h2(zp[j]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t src = (j < 4) ? plo[p] : phi[p];
        const half2_t d = as_h2(magic_pair(src, 4 * (j & 3))) - z2;
        b[2 * p] = d[0];
        b[2 * p + 1] = d[1];
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[s], b, acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) tot[j] += static_cast<float>(sv[j]) * acc[j];

  // tot[j][i] is row 4*kb + i, column 8*c + j.  Meet the other K-half in LDS.
  const int lcol = 8 * (wn * 16 + col16);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < M) red[(wk * M + m) * kDecodeCols + lcol + j] = tot[j][i];
    }
  }
  __syncthreads();

  const int n = n_tile * kDecodeCols + tid;
  const bool nvalid = n < N;
  if (splits == 1) {
    if (nvalid) {
      const float b = bias ? static_cast<float>(bias[n]) : 0.f;
      for (int m = 0; m < M; ++m) {
        const float v = red[m * kDecodeCols + tid] + red[(M + m) * kDecodeCols + tid];
        y[m * N + n] = static_cast<_Float16>(v + b);
      }
    }
    return;
  }

  if (nvalid) {
    for (int m = 0; m < M; ++m) {
      const float v = red[m * kDecodeCols + tid] + red[(M + m) * kDecodeCols + tid];
      partial[(split * M + m) * N + n] = v;
    }
  }
  __threadfence();  // release this work-group's partials device-wide
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&tickets[n_tile], 1u) == static_cast<unsigned>(splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire every other work-group's partials

  if (nvalid) {
    const float b = bias ? static_cast<float>(bias[n]) : 0.f;
    for (int m = 0; m < M; ++m) {
      const float* p = partial + m * N + n;
      const int stride = M * N;
      float sum = 0.f;
      int sp = 0;
      for (; sp + 8 <= splits; sp += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(sp + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      for (; sp < splits; ++sp) sum += p[sp * stride];
      y[m * N + n] = static_cast<_Float16>(sum + b);
    }
  }
  if (tid == 0) atomicExch(&tickets[n_tile], 0u);
}

template <int STEPS>
hipError_t launch_steps(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                        const _Float16* scales, const _Float16* bias, _Float16* y,
                        int M, int K, int N, int g, int G, int splits, int n_tiles,
                        float* partial, uint32_t* tickets, hipStream_t stream) {
  const size_t shmem = 2 * static_cast<size_t>(M) * kDecodeCols * sizeof(float);
  hipLaunchKernelGGL(decode_kernel<STEPS>, dim3(n_tiles * splits), dim3(256), shmem, stream,
                     x, qweight, qzeros, scales, bias, y, partial, tickets, M, K, N, g, G,
                     splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                         const _Float16* scales, const _Float16* bias, _Float16* y,
                         int M, int K, int N, int g, int G, int steps, int splits,
                         int n_tiles, void* workspace, size_t ticket_bytes,
                         hipStream_t stream) {
  uint32_t* tickets = static_cast<uint32_t*>(workspace);
  float* partial = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                        ticket_bytes)
                             : nullptr;
  switch (steps) {
    case 1: return launch_steps<1>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, partial, tickets, stream);
    case 2: return launch_steps<2>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, partial, tickets, stream);
    case 4: return launch_steps<4>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, partial, tickets, stream);
    case 8: return launch_steps<8>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, partial, tickets, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
