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

typedef int v4i __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

// Buffer resource words for a raw (unswizzled) byte buffer: out-of-range
// offsets read zero.
__device__ __forceinline__ v4i raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>((a >> 32) & 0xffffu),
             static_cast<int>(bytes), 0x00020000};
}

// 16-byte HBM -> LDS copy per lane (lane i writes lds + 16 * i), issued as
// inline assembly so that the compiler does not track it: it would otherwise
// make every transposing LDS read wait for all outstanding copies, which
// serialises the prefetch.  Completion is awaited with explicit vmcnt waits.
__device__ __forceinline__ void copy_to_lds(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// Register loads issued as inline assembly as well, so that the compiler's
// own wait counting (which cannot see the copies above) inserts no waits
// for them; wait_regs below waits explicitly and ties the loaded registers
// through the wait, so nothing reads them before it.
__device__ __forceinline__ uint32_t load_u32(v4i rsrc, uint32_t voff) {
  uint32_t v;
  asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}
__device__ __forceinline__ u32x4 load_u32x4(v4i rsrc, uint32_t voff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}
template <int N>
__device__ __forceinline__ void wait_regs(uint32_t (&w)[4], uint32_t& z, u32x4& s) {
  asm volatile("s_waitcnt vmcnt(%6)"
               : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(z), "+v"(s)
               : "n"(N));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

__device__ __forceinline__ short4_t read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

// Operands of one 16-deep k slice for a wave's 128 x 64 sub-tile.
struct Frag {
  half8_t a[4];
  half8_t b[2];
};

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

  const v4i rx = raw_rsrc(x, static_cast<uint32_t>(M) * K * 2u);
  const v4i rq = raw_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const v4i rz = raw_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const v4i rs = raw_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);

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
    for (int r = 0; r < 4; ++r) w[r] = load_u32(rq, (qb + r * q_row) | oob);
    const uint32_t gb = static_cast<uint32_t>(kb >> gsh);
    zw = load_u32(rz, (gb * q_row + z_off) | oob);
    sv = load_u32x4(rs, (gb * static_cast<uint32_t>(N) * 2u + s_off) | oob);
  };
  auto issue_a = [&](int kt) {
    const uint32_t slot = lds_addr(a_ring + (kt % kAStages) * kATileBytes) + 64 * wave * 128;
    const int kb = kt * BK;
    const uint32_t oob0 = (8 * a_chunk0 < K - kb) ? 0u : kOutOfRange;
    const uint32_t oob1 = (8 * a_chunk1 < K - kb) ? 0u : kOutOfRange;
    const uint32_t kb2 = static_cast<uint32_t>(kb) * 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy_to_lds(rx, (a_off[i] + kb2) | ((i & 1) ? oob1 : oob0),
                  __builtin_amdgcn_readfirstlane(slot + 8 * i * 128));
  };
  // Dequantisation of one packed word (k-row 4*brb + r of a K step) into
  // weight buffer `buf` (k-major): bytes b of the word and of the word >> 4
  // give nibbles 2b and 2b+1 in the two float16 halves, OR-ed into 1024.0.
  auto zero_pairs = [&](uint32_t zw, half2_t (&zp)[4]) {
    const uint32_t zs = zw >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
      zp[b] = as_h2(magic_pair(__builtin_amdgcn_perm(zs, zw, sel), 0));
    }
  };
  auto dequant_word = [&](int buf, int r, uint32_t w, const half2_t (&zp)[4], u32x4 sv) {
    char* dst = b_buf + buf * kBTileBytes + (4 * brb + r) * kBPitch + 16 * bwc;
    const uint32_t ws = w >> 4;
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
      const half2_t q2 = as_h2(magic_pair(__builtin_amdgcn_perm(ws, w, sel), 0));
      out[b] = as_u32((q2 - zp[b]) * as_h2(sv[b]));
    }
    *reinterpret_cast<u32x4*>(dst) = out;
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

  auto read_frag = [&](int kt, int ks, Frag& f) {
    const char* a_slot = a_ring + (kt % kAStages) * kATileBytes;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = 128 * wm + 32 * mi + frow;
      const int chunk = (2 * ks + fhalf) ^ ((row >> 1) & 7);
      f.a[mi] = *reinterpret_cast<const half8_t*>(a_slot + row * 128 + 16 * chunk);
    }
    // Weight operand: two transposed 8-byte reads (k-rows +0..3, +4..7).
    const char* bp = b_buf + (kt & 1) * kBTileBytes + (16 * ks + b_krow) * kBPitch + 2 * b_col;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const short4_t lo = read_tr16(bp + 64 * ni);
      const short4_t hi = read_tr16(bp + 64 * ni + 4 * kBPitch);
      f.b[ni] = __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
  };

  // Pipeline.  Step s issues one group of 14 global loads in a fixed order:
  // packed weights/zeros/scales of step s+3 (6 loads), then the x copies of
  // step s+2 (8 loads).  Loads past the end of K read zeros, so every group
  // has 14 loads and one wait count serves: at the start of step kt, group
  // kt-2 = {weights of kt+1, x of kt} is complete once at most 14 loads (group
  // kt-1) are outstanding.  Both operands are thus fetched two steps ahead.
  // LDS operands are read one k slice ahead of the matrix cores; the last
  // slice of a step is multiplied after the next step's barrier, overlapping
  // that step's first reads.  Step kt+1's weights are dequantised during step
  // kt, one packed word per k slice, interleaved with the matrix-core work.
  // Three register sets for packed weights rotate (in flight twice, being
  // dequantised once); the loop is unrolled by three to keep that static,
  // which also makes the x ring slot static.
  uint32_t w3[3][4];
  uint32_t z3[3];
  u32x4 s3[3];
  Frag cur, nxt;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) cur.a[mi] = half8_t{};
  cur.b[0] = half8_t{};
  cur.b[1] = half8_t{};
  // j = kt % 3: set j receives step kt+3, set (j+1) % 3 holds step kt+1.
  // A step runs as 16 sub-blocks (4 k slices x 4 row blocks); each issues two
  // LDS operand reads of slice ks, two MFMAs on the previous slice (for
  // ks = 0 the last slice of step kt-1), one float16 pair of the
  // dequantisation and at most one global load, so that loads, LDS traffic
  // and vector work are spread between the matrix-core operations instead of
  // queueing behind each other.
  auto kstep = [&](int kt, int j) {
    const int jd = (j + 1) % 3;
    wait_regs<kLoadsPerStep>(w3[jd], z3[jd], s3[jd]);  // x of kt, weights of kt+1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // weight tile kt written,
    __builtin_amdgcn_s_barrier();   // ... and every read of step kt-1 done, by all waves
    __builtin_amdgcn_sched_barrier(0);
    // Global loads of this step: weights of kt+3 into set j, x of kt+2.
    const int kbB = (kt + 3) * BK;
    const uint32_t oobB = (4 * brb < K - kbB) ? 0u : kOutOfRange;
    const uint32_t qb = static_cast<uint32_t>(kbB) * q_row + q_off;
    const uint32_t gb = static_cast<uint32_t>(kbB >> gsh);
    const int kbA = (kt + 2) * BK;
    const uint32_t oobA0 = (8 * a_chunk0 < K - kbA) ? 0u : kOutOfRange;
    const uint32_t oobA1 = (8 * a_chunk1 < K - kbA) ? 0u : kOutOfRange;
    const uint32_t kbA2 = static_cast<uint32_t>(kbA) * 2u;
    const uint32_t slotA =
        lds_addr(a_ring + ((kt + 2) % kAStages) * kATileBytes) + 64 * wave * 128;
    auto dma = [&](int i) {
      copy_to_lds(rx, (a_off[i] + kbA2) | ((i & 1) ? oobA1 : oobA0),
                  __builtin_amdgcn_readfirstlane(slotA + 8 * i * 128));
    };
    auto issue_one = [&](int q) {
      switch (q) {
        case 0: w3[j][0] = load_u32(rq, qb | oobB); break;
        case 2: w3[j][1] = load_u32(rq, (qb + q_row) | oobB); break;
        case 4: w3[j][2] = load_u32(rq, (qb + 2 * q_row) | oobB); break;
        case 6: w3[j][3] = load_u32(rq, (qb + 3 * q_row) | oobB); break;
        case 8: z3[j] = load_u32(rz, (gb * q_row + z_off) | oobB); break;
        case 11: s3[j] = load_u32x4(rs, (gb * static_cast<uint32_t>(N) * 2u + s_off) | oobB); break;
        case 1: dma(0); break;
        case 3: dma(1); break;
        case 5: dma(2); break;
        case 7: dma(3); break;
        case 9: dma(4); break;
        case 10: dma(5); break;
        case 12: dma(6); break;
        case 13: dma(7); break;
        default: break;
      }
    };
    half2_t zp[4];
    zero_pairs(z3[jd], zp);
    const char* a_slot = a_ring + (kt % kAStages) * kATileBytes;
    const char* b_rd = b_buf + (kt & 1) * kBTileBytes + b_krow * kBPitch + 2 * b_col;
    char* b_wr = b_buf + ((kt + 1) & 1) * kBTileBytes + (4 * brb) * kBPitch + 16 * bwc;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const uint32_t w = w3[jd][ks];
      const uint32_t ws = w >> 4;
      u32x4 out;
      short4_t raw[4];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        {
          const int row = 128 * wm + 32 * sub + frow;
          const int chunk = (2 * ks + fhalf) ^ ((row >> 1) & 7);
          nxt.a[sub] = *reinterpret_cast<const half8_t*>(a_slot + row * 128 + 16 * chunk);
          raw[sub] = read_tr16(b_rd + 16 * ks * kBPitch + 64 * (sub >> 1) + (sub & 1) * 4 * kBPitch);
        }
        acc[sub][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[sub], cur.b[0], acc[sub][0], 0, 0, 0);
        acc[sub][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[sub], cur.b[1], acc[sub][1], 0, 0, 0);
        {
          const uint32_t sel = 0x0C000C00u | ((4u + sub) << 16) | sub;
          const half2_t q2 = as_h2(magic_pair(__builtin_amdgcn_perm(ws, w, sel), 0));
          out[sub] = as_u32((q2 - zp[sub]) * as_h2(s3[jd][sub]));
        }
        issue_one(4 * ks + sub);
        __builtin_amdgcn_sched_barrier(0);
      }
      *reinterpret_cast<u32x4*>(b_wr + ks * kBPitch) = out;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        nxt.b[ni] = __builtin_bit_cast(
            half8_t, __builtin_shufflevector(raw[2 * ni], raw[2 * ni + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      cur = nxt;
    }
  };
  // Prologue: weights of step 0 alone, then groups "-2" and "-1".
  issue_b(0, w3[0], z3[0], s3[0]);
  issue_b(1, w3[1], z3[1], s3[1]);
  issue_a(0);
  issue_b(2, w3[2], z3[2], s3[2]);
  issue_a(1);
  wait_regs<2 * kLoadsPerStep>(w3[0], z3[0], s3[0]);
  {
    half2_t zp[4];
    zero_pairs(z3[0], zp);
#pragma unroll
    for (int r = 0; r < 4; ++r) dequant_word(0, r, w3[0][r], zp, s3[0]);
  }
  int kt = 0;
  for (; kt + 2 < nkt; kt += 3) {
    kstep(kt, 0);
    kstep(kt + 1, 1);
    kstep(kt + 2, 2);
  }
  if (kt < nkt) kstep(kt, 0);
  if (kt + 1 < nkt) kstep(kt + 1, 1);
  mma(cur);
  // Drain the trailing (out-of-range) loads.  Their destination registers
  // are tied through the wait so that none is reused while a load is still
  // in flight.
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(w3[0][0]), "+v"(w3[0][1]), "+v"(w3[0][2]), "+v"(w3[0][3]), "+v"(z3[0]),
                 "+v"(s3[0]), "+v"(w3[1][0]), "+v"(w3[1][1]), "+v"(w3[1][2]), "+v"(w3[1][3]),
                 "+v"(z3[1]), "+v"(s3[1]), "+v"(w3[2][0]), "+v"(w3[2][1]), "+v"(w3[2][2]),
                 "+v"(w3[2][3]), "+v"(z3[2]), "+v"(s3[2])
               :
               : "memory");

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
