// Decode W4A16 skinny GEMM (M <= 32): split-K over the input dimension,
// matrix cores for the multiply-accumulate, deterministic cross-work-group
// reduction with the bias epilogue fused in.
//
// The page "Predibase Lorax AWQ WQLinear" (Description, forward step 2) runs
// this product in one extension call; at decode sizes the whole cost is the
// stream of packed weights from HBM (0.5 byte per weight), so the kernel is
// built around keeping that stream saturated:
//
// * Two variants.  Streaming (N % 32 == 0, decode_lds_kernel): 4 or 8 waves
//   over the same 256 output columns (32 packed words, 128 contiguous bytes
//   per row) and consecutive 32*STEPS-row K ranges; each wave copies its rows
//   HBM -> LDS with 16-byte direct-to-LDS loads, all issued before any
//   arithmetic, and reads back per 32-row step the 8 rows of its word column.
//   Register (other N, decode_kernel): 2 x 2 waves, each lane loading the 8
//   words of its column and 8-row block per step into registers.
// * Unpack: the streaming variant forms exact normal float16 operands from
//   byte pairs of two rows with four VALU ops per four weights (see
//   decode_lds_kernel); the register variant ORs nibble pairs into float16
//   1024.0 and subtracts (1024 + z), giving the exact integers q - z.
// * MFMA v_mfma_f32_16x16x32_f16: A = 16 rows of x (rows >= M are zero),
//   B = dequantised weights for 16 columns x 32 rows.  Accumulation is fp32.
//   Batches of 17-32 rows (streaming variant, one group per wave) take two
//   16-row blocks of x, each multiplied with the same dequantised operands.
// * The scale is applied once per group to the fp32 group partial:
//   sum_k x*(q - z)*s = s * sum_k x*(q - z) exactly in real arithmetic; this
//   differs from rounding each dequantised weight to float16 only by that
//   rounding (relative 2^-11 per term).  A one-hot row still reproduces the
//   float16 dequantised weight exactly.
// * Reduction: the K-ranges of a work-group meet in LDS; the work-groups of a
//   column tile then meet in the workspace, deterministically in either of
//   two ways, chosen by the planner.  For M <= 4 and few enough atomics per
//   call, one 64-bit device-scope atomic per output element
//   (splitk_atomic): each adds its partial as a 2^-24 fixed-point integer
//   with a contribution count, and the one whose returned sum shows every
//   split has arrived writes y -- one atomic round trip.  Past that, the
//   atomic count outgrows what the memory-side atomic units sustain, so
//   each work-group stores its partials with plain stores and a second
//   kernel on the same stream sums them in split order (decode_sum_kernel).
//   The accumulator region of the workspace is zero again when the atomic
//   exchange ends.
// * Activation order (a row-to-group map whose groups were made contiguous
//   by reordering the packed rows at load time): the LDS variant reads x
//   through the same row order, gathering x[m, perm[k]] itself, so the
//   forward stays one launch.
#include <type_traits>

#include "awq_device.h"
#include "awq_plan.h"

namespace awq {
namespace {

// Split-K exchange state in the workspace (acc and mask are zero between
// calls; partials are overwritten by every call that uses them).
struct SplitK {
  unsigned long long* acc;   // [M][N]: fixed-point sum, contribution count (atomic exchange)
  unsigned long long* mask;  // [M][N]: splits that sent a float partial (atomic exchange)
  float* partial;            // [splits][M][N]: partials (all of them for the two-launch
                             // exchange, the float ones for the atomic exchange)
  int atomic;                // the planner's exchange: 1 atomic, 0 two launches
};
// acc layout: bits 0-51 sum of (v + 2^45) over fixed-point contributions,
// v = rint(p * 2^24) with |p| < 2^21 (so each term is below 2^46 and up to
// 63 of them stay below 2^52); bits 52-57 number of contributions; bits
// 58-62 number of float contributions.  A partial outside the fixed-point
// range (huge, infinite or NaN) is published as a float and flagged instead.
constexpr unsigned long long kFxUnit = 1ull << 52;
constexpr unsigned long long kFxFloat = 1ull << 58;
constexpr long long kFxBias = 1ll << 45;
constexpr float kFxScale = 16777216.0f;   // 2^24
constexpr float kFxLimit = 2097152.0f;    // 2^21
static_assert(kDecodeMaxSplits <= 63, "six-bit contribution counts");

// Cross-wave reduction in LDS.  Each wave's region (`stride` floats apart)
// is laid out [row group of 4][column][4 rows] (row groups below M only):
// the lane holding rows 4*kb .. 4*kb+3 of a column writes them as one
// 16-byte store, and the thread of a column reads each row group of each
// wave as one 16-byte load.  Columns are XOR-swizzled within groups of 16
// (bits 1-3 ^= bits 4-6): the 16 lanes of one store instruction (columns 8
// apart) then spread over 8 bank groups instead of 2, and 16 consecutive
// columns still cover 16 distinct bank groups for the loads.
__device__ __forceinline__ int red_col(int col) { return col ^ (((col >> 4) & 7) << 1); }
__device__ __forceinline__ void red_store(float* red, int stride, int wave, int kb, int col,
                                          floatx4 v) {
  *reinterpret_cast<floatx4*>(red + wave * stride + (kb * kDecodeCols + red_col(col)) * 4) = v;
}
// Sums one pass of M <= kDecodeBlockM rows into part[0 .. M), waves in order.
template <int WAVES>
__device__ __forceinline__ void red_sum(const float* red, int stride, int M, int col, float* part) {
  const int pc = red_col(col);
  if (M == 1) {
    float v = red[pc * 4];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += red[w * stride + pc * 4];
    part[0] = v;
    return;
  }
#pragma unroll
  for (int c4 = 0; c4 < kDecodeBlockM / 4; ++c4) {
    if (4 * c4 < M) {
      floatx4 v = *reinterpret_cast<const floatx4*>(red + (c4 * kDecodeCols + pc) * 4);
#pragma unroll
      for (int w = 1; w < WAVES; ++w)
        v += *reinterpret_cast<const floatx4*>(red + w * stride + (c4 * kDecodeCols + pc) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[4 * c4 + i] = v[i];
    }
  }
}
// Output of a work-group that covers all of K (no exchange).
template <int MM>
__device__ __forceinline__ void store_rows(const float (&part)[MM],
                                           const _Float16* __restrict__ bias,
                                           _Float16* __restrict__ y, int M, int N, int n) {
  const float b = bias ? static_cast<float>(bias[n]) : 0.f;
#pragma unroll
  for (int m = 0; m < MM; ++m)
    if (m < M) y[m * N + n] = static_cast<_Float16>(part[m] + b);
}

// Called by the thread that owns column n of this work-group, with part[m]
// the work-group's partial for row m < M.  All atomics of the thread are issued
// before any result is used.  Partials are exact multiples of 2^-24 whenever
// the scales are (every float16 is), so a one-hot row stays exact.
template <int MM>
__device__ __forceinline__ void splitk_atomic(const float (&part)[MM], const SplitK& sk,
                                              const _Float16* __restrict__ bias,
                                              _Float16* __restrict__ y, int M, int N, int n,
                                              int split, int splits) {
  constexpr int R = MM < kDecodeAtomicMaxM ? MM : kDecodeAtomicMaxM;   // M <= R
  unsigned long long add[R], old[R];
  bool published = false;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    if (m < M) {
      const float p = part[m];
      if (fabsf(p) < kFxLimit) {   // false for NaN
        const long long v = static_cast<long long>(__builtin_rintf(p * kFxScale));
        add[m] = static_cast<unsigned long long>(v + kFxBias) + kFxUnit;
      } else {
        const size_t e = static_cast<size_t>(m) * N + n;
        __hip_atomic_store(sk.partial + static_cast<size_t>(split) * M * N + e, p,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(sk.mask + e, 1ull << split, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        add[m] = kFxUnit + kFxFloat;
        published = true;
      }
    }
  }
  // A published float partial is acknowledged before its count is added, so
  // whoever completes the count sees it (device-coherent accesses throughout).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (published) __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int m = 0; m < R; ++m)
    if (m < M)
      old[m] = __hip_atomic_fetch_add(sk.acc + static_cast<size_t>(m) * N + n, add[m],
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float b = bias ? static_cast<float>(bias[n]) : 0.f;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    if (m >= M) continue;
    const unsigned long long tot = old[m] + add[m];
    if (static_cast<int>((tot >> 52) & 63u) != splits) continue;
    const size_t e = static_cast<size_t>(m) * N + n;
    const int nf = static_cast<int>((tot >> 58) & 63u);
    const long long fx = static_cast<long long>(tot & (kFxUnit - 1)) -
                         static_cast<long long>(splits - nf) * kFxBias;
    float r = static_cast<float>(static_cast<double>(fx) * (1.0 / 16777216.0));
    if (nf) {
      const unsigned long long msk =
          __hip_atomic_load(sk.mask + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int sp = 0; sp < splits; ++sp)
        if ((msk >> sp) & 1ull)
          r += __hip_atomic_load(sk.partial + static_cast<size_t>(sp) * M * N + e,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sk.mask + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    y[e] = static_cast<_Float16>(r + b);
    // Every split has been counted, so nothing else touches this word in
    // this call, and the next call on the stream sees the zero through the
    // kernel boundary: a plain store resets it (a device-scope store would
    // go out to memory and hold up the end of the kernel).
    sk.acc[e] = 0ull;
  }
}

// Two-launch exchange (above the atomic exchange's rows): the thread of
// column n stores the work-group's partial of each row with plain stores;
// decode_sum_kernel, next on the stream, sums them.
template <int MM>
__device__ __forceinline__ void store_partials(const float (&part)[MM],
                                               float* __restrict__ partial, int M, int N, int n,
                                               int split) {
#pragma unroll
  for (int m = 0; m < MM; ++m)
    if (m < M) partial[(static_cast<size_t>(split) * M + m) * N + n] = part[m];
}

// SINGLE_GROUP: every row a wave reads lies in one quantisation group (the
// group size is a multiple of the wave's 32*STEPS rows, or there is one
// group), so the scale is applied once after all steps.  Otherwise each
// 32-row step (which never straddles a group) is scaled on its own.
// Four waves per SIMD cap a wave at 128 registers; the plans that hold
// more words in flight (eight steps, or four steps scaled per step) take
// two, which keeps them from spilling.
template <int STEPS, bool SINGLE_GROUP>
constexpr int decode_kernel_min_waves() {
  return (STEPS >= 8 || (STEPS >= 4 && !SINGLE_GROUP)) ? 2 : 4;
}

template <int STEPS, bool SINGLE_GROUP>
__global__ __launch_bounds__(256) __attribute__((
    amdgpu_waves_per_eu(decode_kernel_min_waves<STEPS, SINGLE_GROUP>(), 8))) void decode_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    SplitK sk, int M, int K, int N, int g, int G, int splits) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // see red_store
  pin_arg(y);
  pin_arg(bias);
  pin_arg(sk.acc);
  pin_arg(sk.mask);
  pin_arg(sk.partial);
  pin_arg(sk.atomic);

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

  // Buffer resources: every load below is range-checked by the hardware and
  // reads zero outside its tensor, so tails need no branches.  Steps at or
  // past K read x == 0 and contribute exact zeros.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(M) * K * 2u);

  // Group parameters first (one group, or one per step).
  constexpr int NG = SINGLE_GROUP ? 1 : STEPS;
  uint32_t zw[NG];
  half8_t sv[NG];
#pragma unroll
  for (int s = 0; s < NG; ++s) {
    const int k0 = kw0 + 32 * s;
    const int grp = (G == 1) ? 0 : k0 / g;
    const bool ok = cvalid && k0 < K;
    zw[s] = buf_load_u32(rz, ok ? static_cast<uint32_t>(grp * NW + c) * 4u : kOutOfRange);
    sv[s] = __builtin_bit_cast(
        half8_t, buf_load_u32x4(rs, ok ? static_cast<uint32_t>(grp * N + 8 * c) * 2u
                                       : kOutOfRange));
  }

  // x fragments, then every packed word of this wave, all in flight at once.
  half8_t xa[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int kr = kw0 + 32 * s + 8 * kb;
    const uint32_t xoff = (col16 < M && kr < K) ? static_cast<uint32_t>(col16 * K + kr) * 2u
                                                : kOutOfRange;
    xa[s] = __builtin_bit_cast(half8_t, buf_load_u32x4(rx, xoff));
  }
  uint32_t wv[STEPS][8];
  const uint32_t row_bytes = static_cast<uint32_t>(NW) * 4u;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int kr = kw0 + 32 * s + 8 * kb;
    const uint32_t off = cvalid ? static_cast<uint32_t>(kr * NW + c) * 4u : kOutOfRange;
#pragma unroll
    for (int r = 0; r < 8; ++r) wv[s][r] = buf_load_u32(rq, off + r * row_bytes);
  }

  floatx4 acc[8], tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    tot[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int gi = SINGLE_GROUP ? 0 : s;
    uint32_t plo[4], phi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      plo[p] = pair_bytes_lo(wv[s][2 * p], wv[s][2 * p + 1]);
      phi[p] = pair_bytes_hi(wv[s][2 * p], wv[s][2 * p + 1]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t b;
      const half2_t z2 = as_h2(zero_pair(zw[gi], j));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t src = (j < 4) ? plo[p] : phi[p];
        const half2_t d = as_h2(magic_pair(src, 4 * (j & 3))) - z2;
        b[2 * p] = d[0];
        b[2 * p + 1] = d[1];
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[s], b, acc[j], 0, 0, 0);
    }
    if (!SINGLE_GROUP) {
      // Scale this step's fp32 partial by its group's scales.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot[j] += static_cast<float>(sv[s][j]) * acc[j];
        acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  if (SINGLE_GROUP) {
#pragma unroll
    for (int j = 0; j < 8; ++j) tot[j] = static_cast<float>(sv[0][j]) * acc[j];
  }

  // tot[j][i] is row 4*kb + i, column 8*c + j.  Meet the other K-half in LDS.
  const int Mq = (M + 3) >> 2;
  const int lcol = 8 * (wn * 16 + col16);
  const int stride = Mq * kDecodeCols * 4;
  if (4 * kb < M) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red_store(red, stride, wk, kb, lcol + j, tot[j]);
  }
  __syncthreads();

  const int n = n_tile * kDecodeCols + tid;
  const bool nvalid = n < N;
  float part[kDecodeBlockM];
  red_sum<2>(red, stride, M, tid, part);
  if (splits == 1) {
    if (nvalid) store_rows(part, bias, y, M, N, n);
    return;
  }

  if (!nvalid) return;
  if (sk.atomic)
    splitk_atomic(part, sk, bias, y, M, N, n, split, splits);
  else
    store_partials(part, sk.partial, M, N, n, split);
}

// ---------------------------------------------------------------------------
// Streaming variant for N % 32 == 0 (rows are 16-byte aligned).  Each wave
// copies its rows straight from HBM into a private LDS region with 16-byte
// buffer loads (8 lanes cover one 128-byte row segment, one instruction moves
// 8 rows), then every lane reads back, per 32-row step, the 8 rows of its
// word column -- the transposition the MFMA operand layout needs -- without
// the packed words ever occupying registers in flight.
//
// Work-group: 4 or 8 waves (WAVES) over the same 256 columns (two MFMA
// column sets of 16 words per wave) and consecutive 32*STEPS-row ranges; the
// K-ranges meet in LDS, the work-groups of a column tile meet through the
// split-K exchange.  The 8-row blocks sit 1088 bytes apart in LDS so that the 64
// lanes of a transposed read (16 word columns x 4 row blocks) hit 64 distinct
// banks.
constexpr int kLdsBlockPitch = 1088;  // 8 rows x 128 bytes + 64-byte skew
constexpr uint32_t kPairTwo15 = 0x78007800u;  // float16 pair (2^15, 2^15)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most n (a multiple of 4 below 64) vector-memory loads are
// outstanding.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n >> 2) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<4>(); break;
    case 2: wait_vmcnt<8>(); break;
    case 3: wait_vmcnt<12>(); break;
    case 4: wait_vmcnt<16>(); break;
    case 5: wait_vmcnt<20>(); break;
    case 6: wait_vmcnt<24>(); break;
    case 7: wait_vmcnt<28>(); break;
    case 8: wait_vmcnt<32>(); break;
    case 9: wait_vmcnt<36>(); break;
    case 10: wait_vmcnt<40>(); break;
    case 11: wait_vmcnt<44>(); break;
    case 12: wait_vmcnt<48>(); break;
    case 13: wait_vmcnt<52>(); break;
    case 14: wait_vmcnt<56>(); break;
    case 15: wait_vmcnt<60>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// GATHER: x (M rows of Kx columns) is read through a column order,
// x[m, perm[k]] in place of x[m, k], and as 0 where perm[k] is outside
// [0, Kx) (the sorted-weight forward; its null rows have perm -1).  Each lane then gathers its eight
// values per step one by one; the perm entries are loaded first and the
// packed-word copies are split in two halves around the gathers, so the
// dependent perm -> x round trip overlaps the first half of the weight
// stream instead of delaying all of it.
//
// RB: MFMA row blocks of 16 rows (2 for 17-32 rows): the dequantised weight
// operands of a step feed one MFMA per block, and the LDS reduction runs
// once per block.
template <int STEPS, bool SINGLE_GROUP, bool GATHER, int WAVES, int RB>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 8))) void
decode_lds_kernel(const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
                  const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
                  const _Float16* __restrict__ bias, _Float16* __restrict__ y,
                  SplitK sk, int M, int K, int N, int g, int G, int splits,
                  const int32_t* __restrict__ perm, int Kx) {
  static_assert(!GATHER || STEPS <= 4, "gather loads must fit the load counter");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves along K");
  static_assert(RB == 1 || (RB == 2 && SINGLE_GROUP && !GATHER),
                "two row blocks only for one group per wave, without a gather");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  pin_arg(y);
  pin_arg(bias);
  pin_arg(sk.acc);
  pin_arg(sk.mask);
  pin_arg(sk.partial);
  pin_arg(sk.atomic);
  constexpr int kWaveBytes = STEPS * 4 * kLdsBlockPitch;

  const int NW = N >> 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Consecutive work-groups take the same rows of neighbouring column tiles,
  // so the 128-byte segments requested together make up whole rows.
  const int n_tiles = gridDim.x / splits;
  const int split = blockIdx.x / n_tiles;
  const int n_tile = blockIdx.x - split * n_tiles;
  const int col16 = lane & 15;  // MFMA column (B) / row (A) of this lane
  const int kb = lane >> 4;     // 8-row block within a 32-row step
  const int c0 = n_tile * 32;   // first word column of the tile
  const int kw0 = split * (32 * WAVES * STEPS) + wave * (32 * STEPS);

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(M) * K * 2u);

  // Group parameters for the lane's two word columns c0 + col16 and
  // c0 + 16 + col16 (one group, or one per step).
  constexpr int NG = SINGLE_GROUP ? 1 : STEPS;
  uint32_t zw[NG][2];
  half8_t sv[NG][2];
#pragma unroll
  for (int s = 0; s < NG; ++s) {
    const int k0 = kw0 + 32 * s;
    const int grp = (G == 1) ? 0 : k0 / g;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + 16 * h + col16;
      const bool ok = c < NW && k0 < K;
      zw[s][h] = buf_load_u32(rz, offset_or_oob(ok, static_cast<uint32_t>(grp * NW + c) * 4u));
      sv[s][h] = __builtin_bit_cast(
          half8_t, buf_load_u32x4(rs, offset_or_oob(ok, static_cast<uint32_t>(grp * N + 8 * c) * 2u)));
    }
  }
  // Packed words: HBM -> LDS, 4 instructions (4 x 8 rows) per step, issued
  // after the x loads so that waiting for step s leaves later steps in flight.
  char* wlds = smem + wave * kWaveBytes;
  const int lrow = lane >> 3;   // row within an 8-row block
  const int lword = c0 + 4 * (lane & 7);
  const uint32_t row_bytes = static_cast<uint32_t>(NW) * 4u;
  const bool cok = lword < NW;
  auto copy_steps = [&](int s_begin, int s_end) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (s < s_begin || s >= s_end) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = kw0 + 32 * s + 8 * b + lrow;
        const uint32_t off = offset_or_oob(
            cok, static_cast<uint32_t>(row) * row_bytes + static_cast<uint32_t>(lword) * 4u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(wlds + (4 * s + b) * kLdsBlockPitch),
            16, off, 0, 0, 0);
      }
    }
  };
  // Steps whose copies precede the x gathers (GATHER only).
  constexpr int kEarly = GATHER ? (STEPS + 1) / 2 : 0;

  // xa[rb][s]: rows 16 * rb + col16 of x (zero past M), k 8 * kb .. +7 of step s.
  half8_t xa[RB][STEPS];
  if (!GATHER) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int kr = kw0 + 32 * s + 8 * kb;
        const int row = kDecodeBlockM * rb + col16;
        const uint32_t xoff =
            offset_or_oob(row < M && kr < K, static_cast<uint32_t>(row * K + kr) * 2u);
        xa[rb][s] = __builtin_bit_cast(half8_t, buf_load_u32x4(rx, xoff));
      }
    // Nothing may be scheduled between here and the waits below except the
    // LDS copies: the waits count outstanding copies.
    __builtin_amdgcn_sched_barrier(0);
    copy_steps(0, STEPS);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    // perm entries of the lane's eight rows per step (rows past K read 0 and
    // are never used), then the first half of the copies, then the gathers
    // (each needs its perm entry: the compiler waits for the perm loads
    // only), then the rest of the copies.
    // Only the lanes of rows below M load (the others' operands are zero),
    // so a gather instruction touches M x 4 addresses, not 64.
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(perm, static_cast<uint32_t>(K) * 4u);
    const bool row_lane = col16 < M;
    u32x4 pv[STEPS][2];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      pv[s][0] = u32x4{0u, 0u, 0u, 0u};
      pv[s][1] = u32x4{0u, 0u, 0u, 0u};
      xa[0][s] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (row_lane) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int kr = kw0 + 32 * s + 8 * kb;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pv[s][h] = buf_load_u32x4(rp, offset_or_oob(kr < K, static_cast<uint32_t>(kr + 4 * h) * 4u));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    copy_steps(0, kEarly);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t kmax = static_cast<uint32_t>(Kx);
    const __amdgpu_buffer_rsrc_t rxg = make_rsrc(x, static_cast<uint32_t>(M) * Kx * 2u);
    if (row_lane) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int kr = kw0 + 32 * s + 8 * kb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t src = pv[s][i >> 2][i & 3];
          const uint32_t off = offset_or_oob(kr < K && src < kmax,
                                             static_cast<uint32_t>(col16) * kmax * 2u + src * 2u);
          xa[0][s][i] =
              __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rxg, off, 0, 0));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    copy_steps(kEarly, STEPS);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Byte-pair contraction.  For byte b of a word (nibbles 2b and 2b+1,
  // columns 8c+2b and 8c+2b+1), one byte shuffle per row pair places that
  // byte of both rows, zero-extended, in the two halves of a register; read
  // as float16 that is the subnormal byte * 2^-24, and masking the high
  // nibble gives q_e * 2^-24.  One packed fused multiply-add by 2^15 with the
  // group's -(zero byte) * 2^-9 (or -z_e * 2^-9) turns each into the exact
  // normal float16
  //   f = ((q_e - z_e) + 16*(q_o - z_o)) * 2^-9,  e = (q_e - z_e) * 2^-9,
  // so the MFMAs sum acc_f[b] = sum_k x*f and acc_e[b] = sum_k x*e, and the
  // odd column is (acc_f - acc_e) / 16.  Four VALU ops per four weights.
  // The operands are kept normal because the matrix cores align subnormal
  // products without normalising them, which costs bits next to a large
  // activation.  q == z and one-hot rows stay exact.
  floatx4 acc_e[RB][2][4], acc_f[RB][2][4];
  floatx4 tot[RB][2][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc_e[rb][h][q] = floatx4{0.f, 0.f, 0.f, 0.f};
        acc_f[rb][h][q] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      if (!SINGLE_GROUP) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tot[rb][h][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }

  // -(zero byte) * 2^-9 and -(low zero nibble) * 2^-9 pairs of byte b of zero
  // word zw (exact: the subnormal byte times -2^15).
  const half2_t up = as_h2(kPairTwo15);
  auto zero_pairs = [up](uint32_t zw, int b, half2_t& zf, half2_t& ze) {
    const uint32_t dup = __builtin_amdgcn_perm(zw, zw, 0x0C000C00u | ((4u + b) << 16) | b);
    zf = -(as_h2(dup) * up);
    ze = -(as_h2(dup & kNibblePairMask) * up);
  };
  // Scale the group partials of set h into the totals, elements 0..R-1 (rows
  // 4*kb + i): added for one group per step, assigned for one group per wave.
  auto fold = [&](int rb, int h, half8_t svh, auto rows) {
    constexpr int R = decltype(rows)::value;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float se = static_cast<float>(svh[2 * q]) * 0x1p9f;
      const float so = static_cast<float>(svh[2 * q + 1]) * 0x1p5f;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float ve = se * acc_e[rb][h][q][i];
        const float vo = so * (acc_f[rb][h][q][i] - acc_e[rb][h][q][i]);
        if (SINGLE_GROUP) {
          tot[rb][h][2 * q][i] = ve;
          tot[rb][h][2 * q + 1][i] = vo;
        } else {
          tot[rb][h][2 * q][i] += ve;
          tot[rb][h][2 * q + 1][i] += vo;
        }
      }
    }
  };
  using OneRow = std::integral_constant<int, 1>;
  using FourRows = std::integral_constant<int, 4>;
  // Only row 0 exists when M == 1 (element 0 of the kb == 0 lanes).
  const bool one_row = M == 1;

  half2_t zf[NG][2][4], ze[NG][2][4];
#pragma unroll
  for (int s = 0; s < NG; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) zero_pairs(zw[s][h], q, zf[s][h][q], ze[s][h][q]);

#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    // Step s's four LDS copies are done once at most 4*(STEPS-1-s) loads
    // (the later steps' copies) are outstanding; with GATHER the early
    // steps' copies precede the gathers and the late copies, so they are
    // done once only the late copies remain.
    wait_vmcnt_upto(s < kEarly ? 4 * (STEPS - kEarly) : 4 * (STEPS - 1 - s));
    const int gi = SINGLE_GROUP ? 0 : s;
    const char* blk = wlds + (4 * s + kb) * kLdsBlockPitch;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        w[r] = *reinterpret_cast<const uint32_t*>(blk + r * 128 + (16 * h + col16) * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // [row 2p byte q, 0, row 2p+1 byte q, 0] for the four row pairs.
        const uint32_t sel = 0x0C000C00u | ((4u + q) << 16) | q;
        half8_t bf, be;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t pb = __builtin_amdgcn_perm(w[2 * p + 1], w[2 * p], sel);
          const half2_t f = __builtin_elementwise_fma(as_h2(pb), up, zf[gi][h][q]);
          const half2_t e = __builtin_elementwise_fma(as_h2(pb & kNibblePairMask), up, ze[gi][h][q]);
          bf[2 * p] = f[0];
          bf[2 * p + 1] = f[1];
          be[2 * p] = e[0];
          be[2 * p + 1] = e[1];
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc_e[rb][h][q] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rb][s], be, acc_e[rb][h][q], 0, 0, 0);
          acc_f[rb][h][q] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rb][s], bf, acc_f[rb][h][q], 0, 0, 0);
        }
      }
      if (!SINGLE_GROUP) {   // RB == 1
        if (one_row)
          fold(0, h, sv[s][h], OneRow{});
        else
          fold(0, h, sv[s][h], FourRows{});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc_e[0][h][q] = floatx4{0.f, 0.f, 0.f, 0.f};
          acc_f[0][h][q] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  // The WAVES K-ranges meet in LDS, one pass per row block.  tot[rb][h][j][i]
  // is row 16*rb + 4*kb + i, local column 8*(16h + col16) + j.  With one
  // row only element 0 is formed, and it goes to a region of its own after
  // the copy regions ([wave][j][word column], WAVES KiB); more rows go to
  // the wave's own copy region when the pass fits there, else to the copy
  // regions of all waves once every wave is past its last step.  In the
  // first two cases each wave stores as soon as its steps are done and one
  // barrier precedes the sum.  One thread per column of the tile then holds
  // its partial; with eight waves the upper half of the work-group is done.
  float* red = reinterpret_cast<float*>(smem);
  const bool col_thread = WAVES == 4 || tid < kDecodeCols;
  const int n = n_tile * kDecodeCols + tid;
  const bool nvalid = col_thread && n < N;
  float part[kDecodeBlockM * RB];
  if (one_row) {
    if (SINGLE_GROUP) {
#pragma unroll
      for (int h = 0; h < 2; ++h) fold(0, h, sv[0][h], OneRow{});
    }
    float* red1 = reinterpret_cast<float*>(smem + WAVES * kWaveBytes);
    if (kb == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) red1[(wave * 8 + j) * 32 + 16 * h + col16] = tot[0][h][j][0];
    }
    __syncthreads();
    if (col_thread) {
      // Column tid: word column tid / 8, nibble j = tid % 8; waves in order.
      const int at = (tid & 7) * 32 + ((tid & (kDecodeCols - 1)) >> 3);
      float v = red1[at];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red1[w * 256 + at];
      part[0] = v;
    }
  } else {
    if (SINGLE_GROUP) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) fold(rb, h, sv[0][h], FourRows{});
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int Mr = min(M - kDecodeBlockM * rb, kDecodeBlockM);   // rows of this pass
      const int Mq = (Mr + 3) >> 2;
      // A pass that fits a wave's own copy region goes there: the wave is
      // past its last step, so it stores without waiting for the others.
      const bool own = Mq * kDecodeCols * 16 <= kWaveBytes;
      const int stride = own ? kWaveBytes / 4 : Mq * kDecodeCols * 4;
      if (!own || rb > 0) __syncthreads();   // the copy regions, or the previous pass, are done with
      if (4 * kb < Mr) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            red_store(red, stride, wave, kb, 8 * (16 * h + col16) + j, tot[rb][h][j]);
      }
      __syncthreads();
      if (col_thread) red_sum<WAVES>(red, stride, Mr, tid, part + kDecodeBlockM * rb);
    }
  }
  if (splits == 1) {
    if (nvalid) store_rows(part, bias, y, M, N, n);
    return;
  }
  if (!nvalid) return;
  if (sk.atomic)
    splitk_atomic(part, sk, bias, y, M, N, n, split, splits);
  else
    store_partials(part, sk.partial, M, N, n, split);
}

// The two-launch exchange's sum: y = the split partials summed in split
// order from zero, + bias.  64 threads per work-group, thread i takes the
// four adjacent outputs 4i .. 4i+3 (N % 8 == 0: never across a row) with
// 16-byte loads of each split's partials (the partial planes are 16-byte
// aligned), SB splits' loads in flight at a time (8, or 16 above eight
// splits, so that up to 16 splits take one round trip); loads past the last
// split re-read it and are dropped.
template <int SB>
__global__ __launch_bounds__(64) void decode_sum_kernel(const float* __restrict__ partial,
                                                        const _Float16* __restrict__ bias,
                                                        _Float16* __restrict__ y, int M, int N,
                                                        int splits) {
  const size_t plane = static_cast<size_t>(M) * N;
  const size_t e = (static_cast<size_t>(blockIdx.x) * 64 + threadIdx.x) * 4;
  if (e >= plane) return;
  floatx4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; sp += SB) {
    floatx4 v[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u)
      v[u] = *reinterpret_cast<const floatx4*>(partial + min(sp + u, splits - 1) * plane + e);
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      sum += (sp + u < splits) ? v[u] : zero;
    }
  }
  if (bias) {
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] += static_cast<float>(bias[e % N + q]);
  }
  half4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = static_cast<_Float16>(sum[q]);
  if ((reinterpret_cast<uintptr_t>(y) & 7) == 0) {
    *reinterpret_cast<half4_t*>(y + e) = o;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) y[e + q] = o[q];
  }
}

// Launches the sum kernel after a split decode kernel whose exchange is the
// two-launch one.
hipError_t launch_sum(const SplitK& sk, const _Float16* bias, _Float16* y, int M, int N,
                      int splits, hipStream_t stream) {
  if (splits <= 1 || sk.atomic) return hipSuccess;
  const size_t quads = static_cast<size_t>(M) * N / 4;
  // Same box, M = 16 / 8, K = 14336, N = 4096 (14 splits): 14.32 -> 14.18 /
  // 13.28 -> 13.00 us with sixteen loads in flight; eight splits lose with
  // sixteen (K = 8192, N = 7168, M = 16: 13.47 -> 13.75 us).
  const dim3 grid(static_cast<unsigned>((quads + 63) / 64));
  if (splits > 8)
    hipLaunchKernelGGL(decode_sum_kernel<16>, grid, dim3(64), 0, stream, sk.partial, bias, y, M, N,
                       splits);
  else
    hipLaunchKernelGGL(decode_sum_kernel<8>, grid, dim3(64), 0, stream, sk.partial, bias, y, M, N,
                       splits);
  return hipGetLastError();
}

template <int STEPS, bool GATHER, int WAVES>
hipError_t launch_lds_waves(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                            const _Float16* scales, const _Float16* bias, _Float16* y,
                            int M, int K, int N, int g, int G, int splits, int n_tiles,
                            SplitK sk, const int32_t* perm, int Kx, hipStream_t stream) {
  // The LDS holds the weight copies, then one reduction pass (at most 16
  // rows) in the same bytes; one row has a reduction region of its own after
  // the copies.
  const size_t copy_bytes = WAVES * STEPS * 4 * kLdsBlockPitch;
  const int pass_rows = M < kDecodeBlockM ? ((M + 3) & ~3) : kDecodeBlockM;
  const size_t red_bytes = WAVES * static_cast<size_t>(pass_rows) * kDecodeCols * sizeof(float);
  const size_t shmem = M == 1 ? copy_bytes + WAVES * kDecodeCols * sizeof(float)
                              : (copy_bytes > red_bytes ? copy_bytes : red_bytes);
  const bool single = (G == 1) || (g % (kDecodeRowsPerStep * STEPS) == 0);
  const dim3 grid(n_tiles * splits), block(64 * WAVES);
  if (M > kDecodeBlockM) {
    // Two row blocks: the planner takes this variant only with one group per
    // wave and no gather.
    if constexpr (!GATHER) {
      if (!single) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decode_lds_kernel<STEPS, true, false, WAVES, 2>), grid, block, shmem,
                         stream, x, qweight, qzeros, scales, bias, y, sk, M, K, N, g, G, splits,
                         perm, Kx);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (single) {
    hipLaunchKernelGGL((decode_lds_kernel<STEPS, true, GATHER, WAVES, 1>), grid, block, shmem,
                       stream, x, qweight, qzeros, scales, bias, y, sk, M, K, N, g, G, splits,
                       perm, Kx);
  } else {
    hipLaunchKernelGGL((decode_lds_kernel<STEPS, false, GATHER, WAVES, 1>), grid, block, shmem,
                       stream, x, qweight, qzeros, scales, bias, y, sk, M, K, N, g, G, splits,
                       perm, Kx);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum(sk, bias, y, M, N, splits, stream);
}

template <int STEPS, bool GATHER>
hipError_t launch_lds_steps(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                            const _Float16* scales, const _Float16* bias, _Float16* y,
                            int M, int K, int N, int g, int G, int splits, int n_tiles,
                            int waves, SplitK sk, const int32_t* perm, int Kx,
                            hipStream_t stream) {
  if (waves == 8)
    return launch_lds_waves<STEPS, GATHER, 8>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                              G, splits, n_tiles, sk, perm, Kx, stream);
  return launch_lds_waves<STEPS, GATHER, 4>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G,
                                            splits, n_tiles, sk, perm, Kx, stream);
}

template <int STEPS>
hipError_t launch_steps(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                        const _Float16* scales, const _Float16* bias, _Float16* y,
                        int M, int K, int N, int g, int G, int splits, int n_tiles,
                        SplitK sk, hipStream_t stream) {
  const size_t shmem = 2 * static_cast<size_t>((M + 3) & ~3) * kDecodeCols * sizeof(float);
  // Work-group row ranges start at multiples of 64*STEPS, so every wave's
  // 32*STEPS rows share a group exactly when g is a multiple of 32*STEPS.
  const bool single = (G == 1) || (g % (kDecodeRowsPerStep * STEPS) == 0);
  if (single)
    hipLaunchKernelGGL((decode_kernel<STEPS, true>), dim3(n_tiles * splits), dim3(256), shmem,
                       stream, x, qweight, qzeros, scales, bias, y, sk, M, K, N,
                       g, G, splits);
  else
    hipLaunchKernelGGL((decode_kernel<STEPS, false>), dim3(n_tiles * splits), dim3(256), shmem,
                       stream, x, qweight, qzeros, scales, bias, y, sk, M, K, N,
                       g, G, splits);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum(sk, bias, y, M, N, splits, stream);
}

}  // namespace

hipError_t launch_decode(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                         const _Float16* scales, const _Float16* bias, _Float16* y,
                         int M, int K, int N, int g, int G, int steps, int splits,
                         int n_tiles, bool lds_variant, int waves, bool atomic,
                         void* workspace, const int32_t* perm, int Kx, hipStream_t stream) {
  if (waves != 4 && !(lds_variant && waves == 8)) return hipErrorInvalidValue;
  if (M > kDecodeBlockM && (!lds_variant || perm)) return hipErrorInvalidValue;
  if (atomic && !decode_atomic_capable(M, N)) return hipErrorInvalidValue;
  // Workspace: accumulator region ([M][N] accumulators, then [M][N] masks),
  // then [splits][M][N] partials.
  char* ws = static_cast<char*>(workspace);
  const size_t mn = static_cast<size_t>(M) * N;
  const SplitK sk{ws ? reinterpret_cast<unsigned long long*>(ws) : nullptr,
                  ws ? reinterpret_cast<unsigned long long*>(ws + mn * 8) : nullptr,
                  ws ? reinterpret_cast<float*>(ws + kAtomicRegionBytes) : nullptr,
                  atomic ? 1 : 0};
  if (lds_variant && perm) {
    switch (steps) {
      case 1: return launch_lds_steps<1, true>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                               G, splits, n_tiles, waves, sk, perm, Kx, stream);
      case 2: return launch_lds_steps<2, true>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                               G, splits, n_tiles, waves, sk, perm, Kx, stream);
      case 4: return launch_lds_steps<4, true>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                               G, splits, n_tiles, waves, sk, perm, Kx, stream);
      default: return hipErrorInvalidValue;   // decode_gathers() is false for 8 steps
    }
  }
  if (perm) return hipErrorInvalidValue;
  if (lds_variant) {
    switch (steps) {
      case 1: return launch_lds_steps<1, false>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                                G, splits, n_tiles, waves, sk, nullptr, K, stream);
      case 2: return launch_lds_steps<2, false>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                                G, splits, n_tiles, waves, sk, nullptr, K, stream);
      case 4: return launch_lds_steps<4, false>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                                G, splits, n_tiles, waves, sk, nullptr, K, stream);
      case 8: return launch_lds_steps<8, false>(x, qweight, qzeros, scales, bias, y, M, K, N, g,
                                                G, splits, n_tiles, waves, sk, nullptr, K, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (steps) {
    case 1: return launch_steps<1>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, sk, stream);
    case 2: return launch_steps<2>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, sk, stream);
    case 4: return launch_steps<4>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, sk, stream);
    case 8: return launch_steps<8>(x, qweight, qzeros, scales, bias, y, M, K, N, g, G, splits,
                                   n_tiles, sk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
