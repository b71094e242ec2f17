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
// * x tiles (256 rows x 64 k) move HBM -> LDS directly (16-byte buffer loads
//   with an LDS destination; no registers) into a 3-stage ring, two K steps
//   ahead of the matrix cores.  Within each 128-byte row the eight 16-byte
//   chunks are XOR-swizzled by (row / 2) % 8, so the 16-byte operand reads of
//   16 consecutive rows hit 16 distinct bank groups.
// * Packed weights (one word, four rows per thread), zeros and scales are
//   loaded into registers two K steps ahead and dequantised one step ahead:
//   float16_RNE((q - z) * s), exactly the value awq_dequant writes, for two
//   adjacent columns per packed float16 operation (byte shuffles place
//   nibbles 2b and 2b+1 in the two halves, OR-ing into float16 1024.0 gives
//   1024 + q exactly, then one packed subtract and one packed multiply).
//   The weight tile is stored k-major ([k][n], 16-byte writes of 8 adjacent
//   columns: conflict-free) and read back with ds_read_b64_tr_b16, whose
//   16-lane transpose turns four k-rows of four adjacent columns into the
//   k-contiguous operand the matrix cores need.
// * Tile order: work-group ids are remapped so that each of the 8 XCDs (which
//   receive ids round-robin) works on a contiguous range of tiles that share
//   rows of x, keeping that slab resident in the XCD's L2.
#include "awq_device.h"
#include "awq_plan.h"

namespace awq {
namespace {

constexpr int BM = kPrefillBM;   // 256
constexpr int BN = kPrefillBN;   // 128
constexpr int BK = kPrefillBK;   // 64
constexpr int kAStages = 3;
constexpr int kATileBytes = BM * BK * 2;        // 32 KiB, 128-byte rows
constexpr int kBPitch = BN * 2 + 64;            // bytes per k-row of the weight tile
constexpr int kBTileBytes = BK * kBPitch;       // 20 KiB
constexpr int kLdsBytes = kAStages * kATileBytes + 2 * kBTileBytes;
constexpr int kLoadsPerStep = 6 + 8;            // weight words/zeros/scales, x copies

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS byte address of a pointer into the kernel's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// ds_read_b64_tr_b16 issued as inline assembly: the compiler treats the
// intrinsic as touching unknown LDS and drains every outstanding
// LDS-destination copy before it, which would serialise the x prefetch.
// The caller must wait on lgkmcnt (lds_wait below) before using the result.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// Wait until every LDS operation has completed.  The raw results of the
// transposed reads are tied through the wait, so any register copy the
// compiler makes of them (to assemble an operand) happens after it.
__device__ __forceinline__ void lds_wait_all(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

__global__ __launch_bounds__(256) void prefill_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    int M, int K, int N, int gsh, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_ring = smem;
  char* const b_buf = smem + kAStages * kATileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int G = gsh >= 31 ? 1 : (K >> gsh);
  const int nkt = (K + BK - 1) / BK;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(M) * K * 2u);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);

  // Every load address is a thread-constant part (computed once here) plus a
  // uniform per-step part.  Loads of k >= K get an out-of-range offset and
  // read zeros on both operands.  Rows of x past M and columns past N only
  // reach outputs that are never stored, so they are clamped / left to read
  // whatever in-range data lies there, not masked.
  //
  // x copy: instruction i of this wave covers tile rows 64*wave + 8*i .. +7;
  // lane -> (row, physical chunk lane % 8), logical chunk = physical ^ swz(row)
  // with swz(row) = (row / 2) % 8 = (4*i + lane/16) % 8: two chunk values.
  const int a_lrow = lane >> 3;
  const int a_chunk0 = (lane & 7) ^ ((lane >> 4) & 7);   // even i
  const int a_chunk1 = a_chunk0 ^ 4;                     // odd i
  uint32_t a_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = min(m0 + 64 * wave + 8 * i + a_lrow, M - 1);
    a_off[i] = static_cast<uint32_t>(m * K + 8 * ((i & 1) ? a_chunk1 : a_chunk0)) * 2u;
  }

  // Weight loader: word column bwc of the tile, rows 4*brb .. 4*brb+3; the
  // group of row k is k >> gsh (gsh = 31 for a single group).
  const int bwc = tid & 15;
  const int brb = tid >> 4;
  const int bc = min((n0 >> 3) + bwc, NW - 1);
  const uint32_t q_off = static_cast<uint32_t>(4 * brb * NW + bc) * 4u;
  const uint32_t z_off = static_cast<uint32_t>(((4 * brb) >> gsh) * NW + bc) * 4u;
  const uint32_t s_off = static_cast<uint32_t>(((4 * brb) >> gsh) * N + 8 * bc) * 2u;
  const uint32_t q_row = static_cast<uint32_t>(NW) * 4u;

  auto issue_b = [&](int kt, uint32_t (&w)[4], uint32_t& zw, u32x4& sv) {
    const int kb = kt * BK;
    const uint32_t oob = (4 * brb < K - kb) ? 0u : kOutOfRange;
    const uint32_t qb = static_cast<uint32_t>(kb) * q_row + q_off;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = buf_load_u32(rq, (qb + r * q_row) | oob);
    const uint32_t gb = static_cast<uint32_t>(kb >> gsh);
    zw = buf_load_u32(rz, (gb * q_row + z_off) | oob);
    sv = buf_load_u32x4(rs, (gb * static_cast<uint32_t>(N) * 2u + s_off) | oob);
  };
  auto issue_a = [&](int kt) {
    char* slot = a_ring + (kt % kAStages) * kATileBytes;
    const int kb = kt * BK;
    const uint32_t oob0 = (8 * a_chunk0 < K - kb) ? 0u : kOutOfRange;
    const uint32_t oob1 = (8 * a_chunk1 < K - kb) ? 0u : kOutOfRange;
    const uint32_t kb2 = static_cast<uint32_t>(kb) * 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(slot + (64 * wave + 8 * i) * 128), 16,
          (a_off[i] + kb2) | ((i & 1) ? oob1 : oob0), 0, 0, 0);
    }
  };
  // Dequantise one K step of packed words into weight buffer `buf` (k-major).
  auto dequant_b = [&](int buf, const uint32_t (&w)[4], uint32_t zw, u32x4 sv) {
    char* dst = b_buf + buf * kBTileBytes + (4 * brb) * kBPitch + 16 * bwc;
    const uint32_t zs = zw >> 4;
    half2_t zp[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
      zp[b] = as_h2(magic_pair(__builtin_amdgcn_perm(zs, zw, sel), 0));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t ws = w[r] >> 4;
      u32x4 out;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
        const half2_t q2 = as_h2(magic_pair(__builtin_amdgcn_perm(ws, w[r], sel), 0));
        out[b] = as_u32((q2 - zp[b]) * as_h2(sv[b]));
      }
      *reinterpret_cast<u32x4*>(dst + r * kBPitch) = out;
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // Operand addressing.  A: lane -> row (lane % 32) of a 32-row block,
  // logical 16-byte chunk 2*ks + lane/32.  B (transposed read): 16-lane group
  // gr = lane / 16 -> columns 16*(gr % 2) .. +15, k-block gr / 2; source lane
  // s = lane % 16 reads k-row s/4 (+4 for the second half), columns 4*(s%4)..
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int gr = lane >> 4;
  const int sl = lane & 15;
  const int b_col = 64 * wn + 16 * (gr & 1) + 4 * (sl & 3);
  const int b_krow = 8 * (gr >> 1) + (sl >> 2);

  auto compute = [&](int kt) {
    const char* a_slot = a_ring + (kt % kAStages) * kATileBytes;
    const uint32_t b_base = lds_addr(b_buf + (kt & 1) * kBTileBytes) +
                            static_cast<uint32_t>(b_krow * kBPitch + 2 * b_col);
    // Weight operands of one 16-deep k slice: two transposed 8-byte reads
    // (k-rows +0..3 and +4..7) per 32-column block.
    auto read_b = [&](int ks, u32x2 (&raw)[4]) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint32_t addr = b_base + static_cast<uint32_t>(16 * ks * kBPitch + 64 * ni);
        raw[2 * ni] = ds_read_tr16<0>(addr);
        raw[2 * ni + 1] = ds_read_tr16<4 * kBPitch>(addr);
      }
    };
    u32x2 raw[4];
    read_b(0, raw);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      lds_wait_all(raw[0], raw[1], raw[2], raw[3]);
      half8_t bcur[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bcur[ni] = __builtin_bit_cast(
            half8_t, u32x4{raw[2 * ni][0], raw[2 * ni][1], raw[2 * ni + 1][0], raw[2 * ni + 1][1]});
      if (ks + 1 < BK / 16) read_b(ks + 1, raw);
      half8_t af[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = 128 * wm + 32 * mi + frow;
        const int chunk = (2 * ks + fhalf) ^ ((row >> 1) & 7);
        af[mi] = *reinterpret_cast<const half8_t*>(a_slot + row * 128 + 16 * chunk);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bcur[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  // Pipeline.  Per K step the issue order is: weight words/zeros/scales for
  // step kt+2 (6 loads), then x copies for step kt+2 (8 loads), so when step
  // kt starts, the x copies of kt are complete once at most 14 loads (those
  // of step kt+1) are outstanding.  Loads past the end of K read zeros, so
  // every step issues the same 14 loads and the counts stay exact.  The two
  // register sets for packed weights alternate between "in flight" and
  // "being dequantised"; the loop is unrolled by two to keep that static.
  uint32_t wa[4], wb[4];
  uint32_t za, zb;
  u32x4 sa, sb;
  auto kstep = [&](int kt, uint32_t (&wi)[4], uint32_t& zi, u32x4& si,
                   const uint32_t (&wd)[4], uint32_t zd, u32x4 sd) {
    wait_vmcnt<kLoadsPerStep>();    // this wave's x copies of step kt landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // weight tile kt written
    __builtin_amdgcn_s_barrier();   // ... by every wave
    __builtin_amdgcn_sched_barrier(0);
    issue_b(kt + 2, wi, zi, si);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(kt);
    dequant_b((kt + 1) & 1, wd, zd, sd);
  };
  issue_b(0, wa, za, sa);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(0);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(1, wb, zb, sb);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(1);
  __builtin_amdgcn_sched_barrier(0);
  dequant_b(0, wa, za, sa);          // waits (compiler) for step 0's words
  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    kstep(kt, wa, za, sa, wb, zb, sb);
    kstep(kt + 1, wb, zb, sb, wa, za, sa);
  }
  if (kt < nkt) kstep(kt, wa, za, sa, wb, zb, sb);
  wait_vmcnt<0>();                   // drain the trailing (out-of-range) copies

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
                          int M, int K, int N, int group_shift, int m_tiles, int n_tiles,
                          hipStream_t stream) {
  hipLaunchKernelGGL(prefill_kernel, dim3(m_tiles * n_tiles), dim3(256), kLdsBytes, stream,
                     x, qweight, qzeros, scales, bias, y, M, K, N, group_shift, n_tiles);
  return hipGetLastError();
}

}  // namespace awq
