// Prefill W4A16 GEMM (large M): LDS-tiled matrix-core GEMM whose weight tile
// is dequantised into LDS, with the bias epilogue fused in.
//
// The product of the page "Predibase Lorax AWQ WQLinear" (Description, forward
// step 2) is compute-bound at prefill sizes, so the dequantisation must be
// amortised over many rows of x: each BM x BN output tile (up to 256 x 192)
// dequantises its 64 x BN weight slab once per K step into LDS and feeds it
// to all BM rows.
//
// * Work-group: 512 threads = 8 waves, 4 consumers in a 2 x 2 grid of
//   (BM/2) x (BN/2) sub-tiles (fp32 accumulators in registers) and 4
//   producers.  One work-group per CU (LDS-limited); each SIMD runs one
//   consumer and one producer wave.
// * Matrix instruction: 256-row tiles use v_mfma_f32_16x16x32_f16, the 64-
//   and 128-row tiles v_mfma_f32_32x32x16_f16.  With random operands the
//   chip runs this kernel at its power limit (about 1.46 GHz against 2.2 GHz
//   for constant data), and the 16x16x32 form finishes the same flops with
//   less energy: it reads and writes a quarter of the accumulator registers
//   per product.
// * x tiles (BM rows x 64 k) move HBM -> LDS directly (16-byte buffer loads
//   with an LDS destination; no registers) into a 3-stage ring, two K steps
//   ahead of the matrix cores.  Within each 128-byte row the eight 16-byte
//   chunks are XOR-swizzled by (row / 2) % 8, so the 16-byte operand reads of
//   16 consecutive rows hit 16 distinct bank groups.
// * Packed weights, zeros and scales are loaded by the producers into
//   registers three K steps ahead and dequantised one step ahead:
//   float16_RNE((q - z) * s), exactly the value awq_dequant writes, for two
//   adjacent columns per packed float16 operation (byte shuffles place
//   nibbles 2b and 2b+1 in the two halves, OR-ing into float16 1024.0 gives
//   1024 + q exactly, then one packed subtract and one packed multiply).
//   The weight tile is stored k-major ([k][n], 16-byte writes of 8 adjacent
//   columns: conflict-free) and read back with ds_read_b64_tr_b16, whose
//   16-lane transpose turns four k-rows of four adjacent columns into the
//   k-contiguous operand the matrix cores need.
// * Consumers read each operand well before its MFMA and replace it in place
//   after its last use; the last operands of a K step are multiplied after
//   the next step's barrier, overlapping that step's first reads.  One
//   barrier per K step.
// * Every global load takes a thread-constant lane offset plus a uniform
//   per-step offset in an SGPR; prefetches past the last K step re-read the
//   last step (in bounds, never used).  Only when K % 64 != 0 does the last
//   step need per-lane masks (the KTAIL instantiation).
// * The consumer waves run at a raised wave priority, so that an MFMA is
//   never held back by producer work that could wait.
// * Tile order: work-group ids are remapped so that each of the 8 XCDs (which
//   receive ids round-robin) works on a block of the tile grid (tile_of), so
//   the tiles resident on one XCD share rows of x and columns of the weight
//   through its L2.
#include "awq_device.h"
#include "awq_plan.h"

namespace awq {
namespace {

constexpr int BK = kPrefillBK;   // 64
constexpr int kAStages = 3;

// Tile shapes BM x BN: BM = 64, 128 or 256 rows (the smallest covering the
// batch, up to 256), BN = 128 or 192 columns (192 with 256 rows only).
//   MI: 32-row MFMA blocks per consumer wave (its sub-tile is BM/2 x BN/2)
//   NB: 32-column MFMA blocks per consumer wave
//   BST: weight-tile buffers (x always has a 3-slot ring)
//   NDMA: x copies per producer thread per step (8 rows of 128 bytes each)
template <int BM, int BN>
struct Cfg {
  static_assert((BM == 64 || BM == 128 || BM == 256) && (BN == 128 || (BN == 192 && BM == 256)),
                "tile shape");
  static constexpr int MI = BM / 64, NB = BN / 64, BST = BN == 192 ? 2 : 3, NDMA = BM / 32;
  // 256-row tiles multiply with v_mfma_f32_16x16x32_f16 (MR x NC blocks of
  // 16 x 16 per consumer wave), the smaller ones with 32x32x16 (MI x NB
  // blocks of 32 x 32).
  static constexpr bool MF16 = BM == 256;
  static constexpr int MR = BM / 32, NC = BN / 32;
  static constexpr int kATileBytes = BM * BK * 2;
  static constexpr int kLoadsPerStep = 6 + NDMA;   // weight words/zeros/scales, x copies
};
template <int BN> constexpr int b_pitch() { return BN * 2 + 64; }   // bytes per k-row
template <int BN> constexpr int b_tile_bytes() { return BK * b_pitch<BN>(); }
// Byte shift of weight-tile row k for the 16x16x32 operand reads: rows 8
// apart are read by one transposing-read pass and would hit the same banks
// at this pitch, so every other 8-row block sits 32 bytes further along its
// row (inside the row's 64 padding bytes).
template <int BM, int BN> __host__ __device__ constexpr int w_shift(int k) {
  return Cfg<BM, BN>::MF16 ? ((k >> 3) & 1) * 32 : 0;
}template <int BM, int BN> constexpr int lds_bytes() {
  return kAStages * Cfg<BM, BN>::kATileBytes + Cfg<BM, BN>::BST * b_tile_bytes<BN>();
}
static_assert(lds_bytes<256, 128>() == 156 * 1024 && lds_bytes<256, 192>() == 152 * 1024,
              "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// Buffer resource words for a raw (unswizzled) byte buffer: out-of-range
// offsets read zero.
__device__ __forceinline__ v4i raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>((a >> 32) & 0xffffu),
             static_cast<int>(bytes), 0x00020000};
}

// Global loads are issued as inline assembly so that the compiler does not
// track them: it would make every transposing LDS read wait for all
// outstanding LDS-destination copies (serialising the prefetch), and its
// counts for the register loads could not include the copies.  Completion is
// awaited with explicit vmcnt waits that tie the loaded registers, so nothing
// reads them earlier.
//
// 16-byte HBM -> LDS copy per lane (lane i writes lds + 16 * i).
__device__ __forceinline__ void copy_to_lds(v4i rsrc, uint32_t voff, uint32_t soff,
                                            uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ uint32_t load_u32(v4i rsrc, uint32_t voff, uint32_t soff) {
  uint32_t v;
  asm volatile("buffer_load_dword %0, %1, %2, %3 offen" : "=v"(v) : "v"(voff), "s"(rsrc), "s"(soff));
  return v;
}
__device__ __forceinline__ u32x4 load_u32x4(v4i rsrc, uint32_t voff, uint32_t soff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen"
               : "=v"(v)
               : "v"(voff), "s"(rsrc), "s"(soff));
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

// Zero points of one packed word as float16 pairs 1024 + z for columns
// (2b, 2b+1): bytes b of the word and of the word >> 4 give nibbles 2b and
// 2b+1 in the low bits of the two halves.
__device__ __forceinline__ void zero_pairs(uint32_t zw, half2_t (&zp)[4]) {
  const uint32_t zs = zw >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
    zp[b] = as_h2(magic_pair(__builtin_amdgcn_perm(zs, zw, sel), 0));
  }
}
// float16_RNE((q - z) * s) for columns (2b, 2b+1) of packed word w (ws = w >> 4).
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, uint32_t ws, int b,
                                                 const half2_t (&zp)[4], u32x4 sv) {
  const uint32_t sel = 0x0C000C00u | ((4u + b) << 16) | b;
  const half2_t q2 = as_h2(magic_pair(__builtin_amdgcn_perm(ws, w, sel), 0));
  return as_u32((q2 - zp[b]) * as_h2(sv[b]));
}

template <int MI, int NB>
struct Frag {
  half8_t a[MI];
  half8_t b[NB];
};

// Tile coordinates and K range of this work-group.  The 8 XCDs receive
// work-group ids round-robin.  Without a split, each XCD takes one block of
// the tile grid, 2 or 4 row tiles by the matching share of column tiles, so
// that every column tile's weights reach 2 or 4 XCDs' L2 instead of all
// eight (M = 2048, K = 4096, N = 12288: 252 -> 181 MB fetched per call, same
// time); within the block row tiles run fastest.  Otherwise each XCD takes a
// contiguous range of ids, which run over the tiles of split 0, then of
// split 1, ..., so an XCD's tiles share rows of x and the same K range.
struct Tile {
  int m0, n0;    // first row and column
  int tile;      // tile index (row-tile major)
  int sp;        // split index
  int kt0, nks;  // first K step and number of K steps of the split
};
template <int BM, int BN>
__device__ __forceinline__ Tile tile_of(int n_tiles, int splits, int kps, int nkt) {
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  const int tiles = nb / splits;
  Tile t;
  // XCD blocks: XM x (8 / XM) XCDs over the (m_tiles, n_tiles) grid.
  const int m_tiles = tiles / n_tiles;
  int xm = 0;
  if (splits == 1 && (nb & 7) == 0) {
    if (m_tiles % 4 == 0 && n_tiles % 2 == 0) xm = 4;
    else if (m_tiles % 2 == 0 && n_tiles % 4 == 0) xm = 2;
  }
  if (xm != 0) {
    const int xn = 8 / xm;
    const int xcd = bid & 7, r = bid >> 3;
    const int mt_per = m_tiles / xm, nt_per = n_tiles / xn;
    const int mt = (xcd / xn) * mt_per + r % mt_per;
    const int nt = (xcd % xn) * nt_per + r / mt_per;
    t.sp = 0;
    t.tile = mt * n_tiles + nt;
    t.m0 = mt * BM;
    t.n0 = nt * BN;
    t.kt0 = 0;
    t.nks = min(kps, nkt);
    return t;
  }
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  t.sp = bid / tiles;
  t.tile = bid - t.sp * tiles;
  const int mt = t.tile / n_tiles;
  t.m0 = mt * BM;
  t.n0 = (t.tile - mt * n_tiles) * BN;
  t.kt0 = t.sp * kps;
  t.nks = min(kps, nkt - t.kt0);
  return t;
}

// Output staging (one split, y 16-byte aligned): once the K loop is done the
// LDS is free; the consumers write float16(acc + bias) into it as a
// row-major 256 x BN tile (row pitch out_pitch: the two row groups of one
// store fall in different banks), then all 512 threads copy it to y with
// 16-byte loads and stores.
template <int BN> constexpr int out_pitch() { return BN * 2 + 16; }
static_assert(256 * out_pitch<128>() <= lds_bytes<256, 128>() &&
                  256 * out_pitch<192>() <= lds_bytes<256, 192>() &&
                  128 * out_pitch<128>() <= lds_bytes<128, 128>() &&
                  64 * out_pitch<128>() <= lds_bytes<64, 128>(),
              "output tile fits the LDS");

template <int BM, int BN, int MI, int NB>
__device__ __forceinline__ void stage_tile(const floatx16 (&acc)[MI][NB],
                                           const _Float16* __restrict__ bias, char* stage, int N,
                                           Tile t, int wave, int lane) {
  const int wm = wave >> 1;
  const int wn = wave & 1;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int lcol = (BN / 2) * wn + 32 * ni + (lane & 31);
    const int col = t.n0 + lcol;
    const float b = (bias && col < N) ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = (BM / 2) * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        *reinterpret_cast<_Float16*>(stage + lrow * out_pitch<BN>() + 2 * lcol) =
            static_cast<_Float16>(acc[mi][ni][r] + b);
      }
    }
  }
}
// tid = 0..511: chunk c = 512*i + tid is 8 columns (16 bytes) of tile row
// c / (BN/8).
template <int BM, int BN>
__device__ __forceinline__ void store_tile(const char* stage, _Float16* __restrict__ y, int M,
                                           int N, Tile t, int tid) {
  constexpr int kChunksPerRow = BN / 8;
  static_assert(BM * BN / 8 % 512 == 0, "whole chunks per thread");
#pragma unroll
  for (int i = 0; i < BM * BN / 8 / 512; ++i) {
    const int c = 512 * i + tid;
    const int lrow = c / kChunksPerRow;
    const int lcol = 8 * (c - lrow * kChunksPerRow);
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * out_pitch<BN>() + 2 * lcol);
    const int row = t.m0 + lrow;
    const int col = t.n0 + lcol;
    if (row < M && col < N)
      *reinterpret_cast<u32x4*>(y + static_cast<size_t>(row) * N + col) = v;
  }
}

// Split K: the fp32 partial of a split goes out the same way, staged as a
// row-major BM x BN fp32 tile (row pitch part_pitch) and copied with 16-byte
// loads and stores (64 per row of 128 columns), instead of 4-byte stores
// scattered over 2 rows per instruction.  Used when the tile fits the LDS.
template <int BN> constexpr int part_pitch() { return BN * 4 + 16; }
template <int BM, int BN> constexpr bool partial_stages() {
  return BM * part_pitch<BN>() <= lds_bytes<BM, BN>();
}
static_assert(partial_stages<256, 128>() && partial_stages<128, 128>() &&
                  partial_stages<64, 128>(),
              "split partials of the narrow tiles are staged");
template <int BM, int BN, int MI, int NB>
__device__ __forceinline__ void stage_partial(const floatx16 (&acc)[MI][NB], char* stage,
                                              int wave, int lane) {
  const int wm = wave >> 1;
  const int wn = wave & 1;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int lcol = (BN / 2) * wn + 32 * ni + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = (BM / 2) * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        *reinterpret_cast<float*>(stage + lrow * part_pitch<BN>() + 4 * lcol) = acc[mi][ni][r];
      }
    }
  }
}
// tid = 0..511: chunk c = 512*i + tid is 4 columns (16 bytes) of tile row
// c / (BN/4); pp is this split's [M][N] partial plane.
template <int BM, int BN>
__device__ __forceinline__ void store_partial(const char* stage, float* __restrict__ pp, int M,
                                              int N, Tile t, int tid) {
  constexpr int kChunksPerRow = BN / 4;
  static_assert(BM * BN / 4 % 512 == 0, "whole chunks per thread");
#pragma unroll
  for (int i = 0; i < BM * BN / 4 / 512; ++i) {
    const int c = 512 * i + tid;
    const int lrow = c / kChunksPerRow;
    const int lcol = 4 * (c - lrow * kChunksPerRow);
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * part_pitch<BN>() + 4 * lcol);
    const int row = t.m0 + lrow;
    const int col = t.n0 + lcol;
    if (row < M && col < N)
      *reinterpret_cast<u32x4*>(pp + static_cast<size_t>(row) * N + col) = v;
  }
}

// Output modes of a work-group: direct per-lane stores, the staged float16
// y tile (one split), or the staged fp32 partial (split K).
enum : int { kOutDirect = 0, kOutStagedY = 1, kOutStagedPartial = 2 };

// Producer waves (4 of the 8): every global load of the tile and the
// dequantisation of the weight slab into LDS.  pw = producer wave 0..3,
// pt = producer thread 0..255.
//
// Step s issues one group of 6 + NDMA loads per thread: packed weights/
// zeros/scales of step s+3 (6 loads) and the x copies of step s+2 (NDMA =
// BM/32: each producer wave copies BM/4 rows).  Every group has the same
// count, so one wait count serves: before the barrier of step kt, group
// kt-2 = {weights of kt+1, x of kt} is complete once at most one group
// (kt-1) is outstanding.  Both operands are thus fetched two
// steps ahead.  Step kt+1's weights are dequantised during step kt into
// weight buffer (kt+1) % BST.  Three register sets for packed weights rotate
// (in flight twice, being dequantised once); the loop is unrolled so that
// sets, ring slots, buffers and LDS addresses are static.
//
// Weight loader, by tile width.  BN = 128: word column pt % 16 of the tile,
// rows 4*(pt/16) .. +3 of a step (four 4-byte loads, one zero word, one
// 16-byte scale load).  BN = 192: word columns 3*(pt%8) .. +2, rows
// 2*(pt/8) and +1 (two 16-byte loads of which three words are used, one
// 16-byte zero load, three 16-byte scale loads).  Either way 6 loads.  The
// group of row k is k >> gsh (gsh = 31 for a single group); a thread's rows
// of a step share one group (groups are at least 4 rows, aligned).  For
// BN = 192, words and scales past the last column are read from wherever
// they fall (the next row, or zero past the end of the buffer): they only
// reach outputs that are never stored.
template <int BN>
struct WSet;
template <>
struct WSet<128> {
  uint32_t w[4];
  uint32_t z;
  u32x4 s;
};
template <>
struct WSet<192> {
  u32x4 w[2];
  u32x4 z;
  u32x4 s[3];
};
template <int N>
__device__ __forceinline__ void wait_set(WSet<128>& r) {
  asm volatile("s_waitcnt vmcnt(%6)"
               : "+v"(r.w[0]), "+v"(r.w[1]), "+v"(r.w[2]), "+v"(r.w[3]), "+v"(r.z), "+v"(r.s)
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void wait_set(WSet<192>& r) {
  asm volatile("s_waitcnt vmcnt(%6)"
               : "+v"(r.w[0]), "+v"(r.w[1]), "+v"(r.z), "+v"(r.s[0]), "+v"(r.s[1]), "+v"(r.s[2])
               : "n"(N));
}
// Wait for everything; every register set is tied so that none is reused
// while a load into it is still in flight.
__device__ __forceinline__ void drain_sets(WSet<128> (&r)[3]) {
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(r[0].w[0]), "+v"(r[0].w[1]), "+v"(r[0].w[2]), "+v"(r[0].w[3]), "+v"(r[0].z),
                 "+v"(r[0].s), "+v"(r[1].w[0]), "+v"(r[1].w[1]), "+v"(r[1].w[2]), "+v"(r[1].w[3]),
                 "+v"(r[1].z), "+v"(r[1].s), "+v"(r[2].w[0]), "+v"(r[2].w[1]), "+v"(r[2].w[2]),
                 "+v"(r[2].w[3]), "+v"(r[2].z), "+v"(r[2].s)
               :
               : "memory");
}
__device__ __forceinline__ void drain_sets(WSet<192> (&r)[3]) {
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(r[0].w[0]), "+v"(r[0].w[1]), "+v"(r[0].z), "+v"(r[0].s[0]), "+v"(r[0].s[1]),
                 "+v"(r[0].s[2]), "+v"(r[1].w[0]), "+v"(r[1].w[1]), "+v"(r[1].z), "+v"(r[1].s[0]),
                 "+v"(r[1].s[1]), "+v"(r[1].s[2]), "+v"(r[2].w[0]), "+v"(r[2].w[1]), "+v"(r[2].z),
                 "+v"(r[2].s[0]), "+v"(r[2].s[1]), "+v"(r[2].s[2])
               :
               : "memory");
}

// The dequantised halves of one packed word (8 columns of one k-row).
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, const half2_t (&zp)[4], u32x4 sv) {
  const uint32_t ws = w >> 4;
  u32x4 out;
#pragma unroll
  for (int b = 0; b < 4; ++b) out[b] = dequant_pair(w, ws, b, zp, sv);
  return out;
}

template <int BM, int BN, bool KTAIL>
__device__ __forceinline__ void producer(const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
                                         const uint32_t* __restrict__ qz,
                                         const _Float16* __restrict__ sc, _Float16* __restrict__ y,
                                         int M, int K, int N, int gsh, Tile t, char* a_ring,
                                         char* b_ring, int pw, int pt, int out_mode,
                                         float* __restrict__ partial) {
  using C = Cfg<BM, BN>;
  constexpr int kBPitch = b_pitch<BN>();
  constexpr int kBTileBytes = b_tile_bytes<BN>();
  constexpr int kATileBytes = C::kATileBytes;
  constexpr int kLoadsPerStep = C::kLoadsPerStep;
  constexpr int NDMA = C::NDMA;
  const int lane = pt & 63;
  const int NW = N >> 3;
  const int G = gsh >= 31 ? 1 : (K >> gsh);
  const int nks = t.nks;   // K steps of this split, from step t.kt0
  const v4i rx = raw_rsrc(x, static_cast<uint32_t>(M) * K * 2u);
  const v4i rq = raw_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const v4i rz = raw_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const v4i rs = raw_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);

  // Lane offsets.  Rows of x past M and columns past N only reach outputs
  // that are never stored, so they are clamped to in-range data, not masked.
  //
  // x copy: instruction i of producer wave pw covers tile rows
  // (BM/4)*pw + 8*i .. +7; lane -> (row, physical chunk lane % 8), logical
  // chunk = physical ^ swz(row) with swz(row) = (row / 2) % 8 =
  // (4*i + lane/16) % 8 (BM/8 is a multiple of 8): two values.
  const int a_lrow = lane >> 3;
  const int a_chunk0 = (lane & 7) ^ ((lane >> 4) & 7);   // even i
  const int a_chunk1 = a_chunk0 ^ 4;                     // odd i
  uint32_t a_off[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int m = min(t.m0 + (BM / 4) * pw + 8 * i + a_lrow, M - 1);
    a_off[i] = static_cast<uint32_t>(m * K + 8 * ((i & 1) ? a_chunk1 : a_chunk0)) * 2u;
  }
  // Weight loader lane offsets (see above).
  constexpr int WR = BN == 128 ? 4 : 2;   // k-rows per thread
  const int wrow = BN == 128 ? 4 * (pt >> 4) : 2 * (pt >> 3);
  const int wcol = BN == 128 ? min((t.n0 >> 3) + (pt & 15), NW - 1) : (t.n0 >> 3) + 3 * (pt & 7);
  const uint32_t q_row = static_cast<uint32_t>(NW) * 4u;
  uint32_t q_off[WR];
#pragma unroll
  for (int r = 0; r < WR; ++r) q_off[r] = static_cast<uint32_t>((wrow + r) * NW + wcol) * 4u;
  const uint32_t z_off = static_cast<uint32_t>((wrow >> gsh) * NW + wcol) * 4u;
  const uint32_t s_off = static_cast<uint32_t>((wrow >> gsh) * N + 8 * wcol) * 2u;
  // A thread's k-rows lie in one 8-row block, so they share one row shift.
  char* const b_wr0 = b_ring + wrow * kBPitch + w_shift<BM, BN>(wrow) +
                      (BN == 128 ? 16 * (pt & 15) : 48 * (pt & 7));

  // Per-step load parameters: uniform offsets of step k (clamped to the last
  // step; prefetches past the end re-read it and are never used) and, for a
  // partial last step only, per-lane out-of-range masks.
  struct StepA {
    uint32_t soff, oob0, oob1;
  };
  struct StepB {
    uint32_t sq, sz, ss, oob;
  };
  auto step_a = [&](int k) {
    const int kb = (t.kt0 + min(k, nks - 1)) * BK;
    StepA p;
    p.soff = static_cast<uint32_t>(kb) * 2u;
    p.oob0 = (KTAIL && 8 * a_chunk0 >= K - kb) ? kOutOfRange : 0u;
    p.oob1 = (KTAIL && 8 * a_chunk1 >= K - kb) ? kOutOfRange : 0u;
    return p;
  };
  auto step_b = [&](int k) {
    const int kb = (t.kt0 + min(k, nks - 1)) * BK;
    const uint32_t gb = static_cast<uint32_t>(kb >> gsh);
    StepB p;
    p.sq = static_cast<uint32_t>(kb) * q_row;
    p.sz = gb * q_row;
    p.ss = gb * static_cast<uint32_t>(N) * 2u;
    p.oob = (KTAIL && wrow >= K - kb) ? kOutOfRange : 0u;
    return p;
  };
  WSet<BN> ws[3];
  // Load number u (0..5) of one step's weight group into set `set`.
  auto load_b = [&](const StepB& p, int set, int u) {
    if constexpr (BN == 128) {
      if (u < 4) ws[set].w[u] = load_u32(rq, q_off[u] | p.oob, p.sq);
      if (u == 4) ws[set].z = load_u32(rz, z_off | p.oob, p.sz);
      if (u == 5) ws[set].s = load_u32x4(rs, s_off | p.oob, p.ss);
    } else {
      if (u < 2) ws[set].w[u] = load_u32x4(rq, q_off[u] | p.oob, p.sq);
      if (u == 2) ws[set].z = load_u32x4(rz, z_off | p.oob, p.sz);
      if (u >= 3) ws[set].s[u - 3] = load_u32x4(rs, (s_off + 16u * (u - 3)) | p.oob, p.ss);
    }
  };
  auto issue_b = [&](const StepB& p, int set) {
#pragma unroll
    for (int u = 0; u < 6; ++u) load_b(p, set, u);
  };
  auto issue_a = [&](const StepA& p, int slot) {
    const uint32_t base = lds_addr(a_ring + slot * kATileBytes) + (BM / 4) * pw * 128;
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      copy_to_lds(rx, a_off[i] | ((i & 1) ? p.oob1 : p.oob0), p.soff,
                  __builtin_amdgcn_readfirstlane(base + 8 * i * 128));
  };
  // Dequantisation unit u of a set: BN = 128: row u (0..3); BN = 192:
  // word column u / 2, row u % 2 (0..5).  New zero pairs at each new column.
  constexpr int kUnits = BN == 128 ? 4 : 6;
  auto new_zero = [](int u) { return u == 0 || (BN == 192 && (u & 1) == 0); };
  auto zero_of = [&](int set, int u) -> uint32_t {
    if constexpr (BN == 128) return ws[set].z;
    else return ws[set].z[u >> 1];
  };
  auto dequant_unit = [&](int buf, int set, int u, const half2_t (&zp)[4]) {
    char* const dst = b_wr0 + static_cast<uint32_t>(buf) * kBTileBytes;
    if constexpr (BN == 128) {
      *reinterpret_cast<u32x4*>(dst + u * kBPitch) = dequant_word(ws[set].w[u], zp, ws[set].s);
    } else {
      const int c = u >> 1, r = u & 1;
      *reinterpret_cast<u32x4*>(dst + r * kBPitch + 16 * c) =
          dequant_word(ws[set].w[r][c], zp, ws[set].s[c]);
    }
  };
  auto dequant_to = [&](int buf, int set) {
    half2_t zp[4];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      if (new_zero(u)) zero_pairs(zero_of(set, u), zp);
      dequant_unit(buf, set, u, zp);
    }
  };

  // Prologue: weights of step 0 alone, then groups "-2" and "-1".
  issue_b(step_b(0), 0);
  issue_b(step_b(1), 1);
  issue_a(step_a(0), 0);
  issue_b(step_b(2), 2);
  issue_a(step_a(1), 1);
  wait_set<2 * kLoadsPerStep>(ws[0]);
  dequant_to(0, 0);

  // Step kt: j = kt % 3.  Set j receives step kt+3; set (j+1) % 3 holds
  // step kt+1, dequantised into buffer (kt+1) % BST (static for BST = 3,
  // computed per step otherwise).
  auto pstep = [&](int kt, int j) {
    const int jd = (j + 1) % 3;
    const int bd = C::BST == 3 ? jd : (kt + 1) % C::BST;
    wait_set<kLoadsPerStep>(ws[jd]);                    // x of kt, weights of kt+1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // weight tile kt written
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // Loads are spread between the dequantised words, so that the wave never
    // stalls behind a full load queue with vector work pending.
    const StepB pb = step_b(kt + 3);
    const StepA pa = step_a(kt + 2);
    const uint32_t abase =
        lds_addr(a_ring + ((j + 2) % 3) * kATileBytes) + (BM / 4) * pw * 128;
    auto dma = [&](int i) {
      copy_to_lds(rx, a_off[i] | ((i & 1) ? pa.oob1 : pa.oob0), pa.soff,
                  __builtin_amdgcn_readfirstlane(abase + 8 * i * 128));
    };
    half2_t zp[4];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      if constexpr (BN == 128) {
        // x copies [u*NDMA/4, (u+1)*NDMA/4) with this unit.
        constexpr int kPer = NDMA / 4;
        load_b(pb, j, u);
        if constexpr (kPer >= 1) dma(kPer * u);
        if (u == 1) load_b(pb, j, 4);
        if (u == 2) load_b(pb, j, 5);
        if constexpr (kPer >= 2) dma(kPer * u + 1);
        if constexpr (kPer == 0) {
          if (u & 1) dma(u >> 1);
        }
      } else {
        load_b(pb, j, u);
        if (u < 2) {
          dma(2 * u);
          dma(2 * u + 1);
        } else {
          dma(u + 2);
        }
      }
      if (new_zero(u)) zero_pairs(zero_of(jd, u), zp);
      dequant_unit(bd, jd, u, zp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  for (; kt + 2 < nks; kt += 3) {
    pstep(kt, 0);
    pstep(kt + 1, 1);
    pstep(kt + 2, 2);
  }
  if (kt < nks) pstep(kt, 0);
  if (kt + 1 < nks) pstep(kt + 1, 1);
  drain_sets(ws);
  if (out_mode == kOutDirect) return;
  __syncthreads();   // every wave is done with the LDS
  __syncthreads();   // the consumers have staged the output tile
  if (out_mode == kOutStagedY)
    store_tile<BM, BN>(a_ring, y, M, N, t, 256 + pt);
  else if constexpr (partial_stages<BM, BN>())
    store_partial<BM, BN>(a_ring, partial + static_cast<size_t>(t.sp) * M * N, M, N, t, 256 + pt);
}

// Consumer waves of the 64- and 128-row tiles (4 of the 8, a 2 x 2 grid):
// LDS operand reads and the matrix-core work for a (BM/2) x 64 sub-tile each
// (MI x 2 blocks of 32 x 32), then the epilogue.  Two operand sets: LDS
// operands are read one k slice ahead of the MFMAs; the last slice of a step
// is multiplied after the next step's barrier, overlapping that step's
// first reads.  Each slice runs as MI sub-blocks of LDS reads (one x block,
// and the four weight reads spread over them) and two MFMAs.
template <int BM, int BN>
__device__ __forceinline__ void consumer(const _Float16* __restrict__ bias, _Float16* __restrict__ y,
                                         float* __restrict__ partial, int M, int N, int splits,
                                         Tile t, char* a_ring, const char* b_ring, int wave,
                                         int lane, int out_mode) {
  using C = Cfg<BM, BN>;
  static_assert(!C::MF16 && BN == 128 && C::BST == 3, "64- and 128-row tiles");
  constexpr int MI = C::MI;
  constexpr int NB = C::NB;
  constexpr int kBPitch = b_pitch<BN>();
  constexpr int kBTileBytes = b_tile_bytes<BN>();
  constexpr int kATileBytes = C::kATileBytes;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int nkt = t.nks;
  // Operand addressing.  A: lane -> row (lane % 32) of a 32-row block,
  // logical 16-byte chunk 2*ks + lane/32.  B (transposed read): 16-lane group
  // gr = lane / 16 -> columns 16*(gr % 2) .. +15 of a 32-column block, k-block
  // gr / 2; source lane s = lane % 16 reads k-row s/4 (+4 for the second
  // half), columns 4*(s%4) ..
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int gr = lane >> 4;
  const int sl = lane & 15;
  const int b_col = (BN / 2) * wn + 16 * (gr & 1) + 4 * (sl & 3);
  const int b_krow = 8 * (gr >> 1) + (sl >> 2);
  const char* const b_rd0 = b_ring + b_krow * kBPitch + 2 * b_col;

  floatx16 acc[MI][NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  Frag<MI, NB> cur, nxt;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) cur.a[mi] = half8_t{};
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) cur.b[ni] = half8_t{};

  // Weight read number q (0 .. 3) of a slice: block q / 2, k-rows +4*(q%2).
  // Step with x slot j and weight buffer jb.
  auto cstep = [&](int j, int jb) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of step kt-1 done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const char* a_slot = a_ring + static_cast<uint32_t>(j) * kATileBytes;
    const char* b_rd = b_rd0 + static_cast<uint32_t>(jb) * kBTileBytes;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      auto a_src = [&](int sub) {
        const int row = (BM / 2) * wm + 32 * sub + frow;
        const int chunk = (2 * ks + fhalf) ^ ((row >> 1) & 7);
        return reinterpret_cast<const half8_t*>(a_slot + row * 128 + 16 * chunk);
      };
      auto b_src = [&](int q) {
        return b_rd + 16 * ks * kBPitch + 64 * (q >> 1) + (q & 1) * 4 * kBPitch;
      };
      // The four weight reads of a slice spread over the MI sub-blocks.
      short4_t raw[4];
#pragma unroll
      for (int sub = 0; sub < MI; ++sub) {
        nxt.a[sub] = *a_src(sub);
#pragma unroll
        for (int q = sub * 4 / MI; q < (sub + 1) * 4 / MI; ++q) raw[q] = read_tr16(b_src(q));
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
          acc[sub][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[sub], cur.b[ni],
                                                                acc[sub][ni], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
        nxt.b[ni] = __builtin_bit_cast(
            half8_t, __builtin_shufflevector(raw[2 * ni], raw[2 * ni + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      cur = nxt;
    }
  };
  // x slot and weight buffer of step kt are both kt % 3 (static: the loop
  // is unrolled by three).
  int kt = 0;
  for (; kt + 2 < nkt; kt += 3) {
    cstep(0, 0);
    cstep(1, 1);
    cstep(2, 2);
  }
  if (kt < nkt) cstep(0, 0);
  if (kt + 1 < nkt) cstep(1, 1);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[mi], cur.b[ni], acc[mi][ni], 0, 0, 0);

  // Epilogue: 32x32 block output, lane holds column (lane % 32) and rows
  // 8*(r/4) + 4*(lane/32) + r%4 of register r.
  if (out_mode == kOutStagedY) {
    __syncthreads();   // every wave is done with the LDS
    stage_tile<BM, BN, MI, NB>(acc, bias, a_ring, N, t, wave, lane);
    __syncthreads();
    store_tile<BM, BN>(a_ring, y, M, N, t, 64 * wave + lane);
    return;
  }
  if constexpr (partial_stages<BM, BN>()) {
    if (out_mode == kOutStagedPartial) {
      __syncthreads();   // every wave is done with the LDS
      stage_partial<BM, BN, MI, NB>(acc, a_ring, wave, lane);
      __syncthreads();
      store_partial<BM, BN>(a_ring, partial + static_cast<size_t>(t.sp) * M * N, M, N, t,
                            64 * wave + lane);
      return;
    }
  }
  // Otherwise one split: y = acc + bias, 2-byte stores; several: the fp32
  // partial of this split (summed by prefill_reduce_kernel).
  float* const pp = partial + static_cast<size_t>(t.sp) * M * N;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int col = t.n0 + (BN / 2) * wn + 32 * ni + frow;
    if (col >= N) continue;
    const float b = (bias && splits == 1) ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = t.m0 + (BM / 2) * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        if (splits == 1)
          y[row * N + col] = static_cast<_Float16>(acc[mi][ni][r] + b);
        else
          pp[static_cast<size_t>(row) * N + col] = acc[mi][ni][r];
      }
    }
  }
}

// The 256-row tiles' consumers: the same 2 x 2 grid of (BM/2) x (BN/2)
// sub-tiles, as MR x NC blocks of v_mfma_f32_16x16x32_f16 over 32-k slices.
// Under the chip's power limit (random operands) this instruction finishes
// the same flops sooner than 32x32x16: it moves a quarter of the accumulator
// registers per product.
//
// Operands (lane = 16 * grp + i): x block rb: row 16*rb + i, k 8*grp .. +7 of
// the slice (one 16-byte read); weight block cb: column 16*cb + i, the same
// k (two transposing reads of four k-rows each; source lane i of a 16-lane
// group reads k-row i/4 (+4), columns 4*(i%4) .. +3).  Accumulator register r
// of block (rb, cb): row 16*rb + 4*grp + r, column 16*cb + i.
//
// Order: x-block major.  The NC weight blocks of a slice stay in registers
// while the x blocks stream through two registers (block rb+1 is read during
// the NC MFMAs of block rb); during the slice's last x block each weight
// block is replaced by the next slice's right after its MFMA.  At the end of
// a K step that last x block is multiplied after the next step's barrier,
// overlapping that step's first reads.  Registers: 4*MR*NC accumulators
// (192 for 256 x 192) + 4*NC + 8 operands.
template <int BM, int BN>
__device__ __forceinline__ void stage_tile16(const floatx4 (&acc)[BM / 32][BN / 32],
                                             const _Float16* __restrict__ bias, char* stage,
                                             int N, Tile t, int wave, int lane) {
  constexpr int MR = BM / 32, NC = BN / 32;
  const int wm = wave >> 1;
  const int wn = wave & 1;
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    const int lcol = (BN / 2) * wn + 16 * cb + (lane & 15);
    const int col = t.n0 + lcol;
    const float b = (bias && col < N) ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = (BM / 2) * wm + 16 * rb + 4 * (lane >> 4) + r;
        *reinterpret_cast<_Float16*>(stage + lrow * out_pitch<BN>() + 2 * lcol) =
            static_cast<_Float16>(acc[rb][cb][r] + b);
      }
    }
  }
}
template <int BM, int BN>
__device__ __forceinline__ void stage_partial16(const floatx4 (&acc)[BM / 32][BN / 32],
                                                char* stage, int wave, int lane) {
  constexpr int MR = BM / 32, NC = BN / 32;
  const int wm = wave >> 1;
  const int wn = wave & 1;
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    const int lcol = (BN / 2) * wn + 16 * cb + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = (BM / 2) * wm + 16 * rb + 4 * (lane >> 4) + r;
        *reinterpret_cast<float*>(stage + lrow * part_pitch<BN>() + 4 * lcol) = acc[rb][cb][r];
      }
    }
  }
}

template <int BM, int BN>
__device__ __forceinline__ void consumer16(const _Float16* __restrict__ bias,
                                           _Float16* __restrict__ y, float* __restrict__ partial,
                                           int M, int N, int splits, Tile t, char* a_ring,
                                           const char* b_ring, int wave, int lane, int out_mode) {
  using C = Cfg<BM, BN>;
  constexpr int MR = C::MR;
  constexpr int NC = C::NC;
  constexpr int kBPitch = b_pitch<BN>();
  constexpr int kBTileBytes = b_tile_bytes<BN>();
  constexpr int kATileBytes = C::kATileBytes;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int nkt = t.nks;
  const int li = lane & 15;
  const int grp = lane >> 4;

  floatx4 acc[MR][NC];
#pragma unroll
  for (int rb = 0; rb < MR; ++rb)
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  half8_t b[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) b[cb] = half8_t{};

  half8_t a_cur = half8_t{}, a_nxt = half8_t{};
  // Operand addresses: a per-lane byte offset plus compile-time constants.
  // x: row (BM/2)*wm + 16*rb + li, 16-byte chunk (4*ks + grp) ^ ((row/2) % 8),
  // where (row/2) % 8 = (li/2) % 8 for every rb.  Weights: k-row 32*ks +
  // 8*grp + li/4 (+4), shifted as its 8-row block, column (BN/2)*wn + 16*cb +
  // 4*(li%4).
  const int a_row = (BM / 2) * wm + li;
  const uint32_t a_off0 = a_row * 128 + 16 * (grp ^ ((li >> 1) & 7));
  const uint32_t a_off1 = a_row * 128 + 16 * ((4 + grp) ^ ((li >> 1) & 7));
  const int b_krow = 8 * grp + (li >> 2);
  const uint32_t b_off =
      b_krow * kBPitch + w_shift<BM, BN>(b_krow) + 2 * ((BN / 2) * wn + 4 * (li & 3));
  auto a_src = [&](const char* a_slot, int ks, int rb) {
    return reinterpret_cast<const half8_t*>(a_slot + (ks ? a_off1 : a_off0) + 2048 * rb);
  };
  auto b_read = [&](const char* b_buf, int ks, int cb) {
    const char* p = b_buf + b_off + 32 * ks * kBPitch + 32 * cb;
    const short4_t lo = read_tr16(p);
    const short4_t hi = read_tr16(p + 4 * kBPitch);
    return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Rows 0 .. MR-2 of the slice held in b / a_cur: each row's x block for
  // the next row is read while the row's NC MFMAs run.
  auto body_rows = [&](const char* a_slot, int ks) {
#pragma unroll
    for (int rb = 0; rb + 1 < MR; ++rb) {
      a_nxt = *a_src(a_slot, ks, rb + 1);
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur, b[cb], acc[rb][cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      a_cur = a_nxt;
    }
  };
  // Last row of the slice held in b / a_cur, each weight block replaced by
  // slice ks of (a_slot, b_buf) right after its MFMA, and the first x block of
  // that slice read at the start.  In the first step the operands are still
  // zero and the MFMAs add nothing.
  auto last_row = [&](const char* a_slot, const char* b_buf, int ks) {
    a_nxt = *a_src(a_slot, ks, 0);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      acc[MR - 1][cb] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur, b[cb], acc[MR - 1][cb], 0, 0, 0);
      b[cb] = b_read(b_buf, ks, cb);
      __builtin_amdgcn_sched_barrier(0);
    }
    a_cur = a_nxt;
  };
  // Step with x slot j and weight buffer jb: the previous step's last row
  // (after the barrier: its operands are in registers), then slice 0, the
  // transition to slice 1, and slice 1 up to its last row.
  auto cstep = [&](int j, int jb) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of step kt-1 done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const char* a_slot = a_ring + static_cast<uint32_t>(j) * kATileBytes;
    const char* b_buf = b_ring + static_cast<uint32_t>(jb) * kBTileBytes;
    last_row(a_slot, b_buf, 0);
    body_rows(a_slot, 0);
    last_row(a_slot, b_buf, 1);
    body_rows(a_slot, 1);
  };
  {
    int j = 0;
#pragma unroll 1
    for (int kt = 0; kt < nkt; ++kt) {
      cstep(__builtin_amdgcn_readfirstlane(j), __builtin_amdgcn_readfirstlane(kt % C::BST));
      j = j == 2 ? 0 : j + 1;
    }
  }
#pragma unroll
  for (int cb = 0; cb < NC; ++cb)
    acc[MR - 1][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur, b[cb], acc[MR - 1][cb], 0, 0, 0);

  if (out_mode == kOutStagedY) {
    __syncthreads();   // every wave is done with the LDS
    stage_tile16<BM, BN>(acc, bias, a_ring, N, t, wave, lane);
    __syncthreads();
    store_tile<BM, BN>(a_ring, y, M, N, t, 64 * wave + lane);
    return;
  }
  if constexpr (partial_stages<BM, BN>()) {
    if (out_mode == kOutStagedPartial) {
      __syncthreads();   // every wave is done with the LDS
      stage_partial16<BM, BN>(acc, a_ring, wave, lane);
      __syncthreads();
      store_partial<BM, BN>(a_ring, partial + static_cast<size_t>(t.sp) * M * N, M, N, t,
                            64 * wave + lane);
      return;
    }
  }
  float* const pp = partial + static_cast<size_t>(t.sp) * M * N;
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    const int col = t.n0 + (BN / 2) * wn + 16 * cb + li;
    if (col >= N) continue;
    const float bv = (bias && splits == 1) ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t.m0 + (BM / 2) * wm + 16 * rb + 4 * grp + r;
        if (row >= M) continue;
        if (splits == 1)
          y[row * N + col] = static_cast<_Float16>(acc[rb][cb][r] + bv);
        else
          pp[static_cast<size_t>(row) * N + col] = acc[rb][cb][r];
      }
    }
  }
}

// 512 threads = 8 waves: waves 0-3 consume (MFMA), waves 4-7 produce (loads
// and dequantisation).  Waves are spread over the 4 SIMDs round-robin, so
// each SIMD runs one of each and the producer's vector work co-issues with
// the consumer's matrix-core work.  Both roles pass the same number of
// barriers (one per K step, two more when the output or partial is staged).
//
// Split K (few tiles): work-group (tile, split) covers kps K steps and
// stores its fp32 partial; prefill_reduce_kernel, next on the stream, sums
// them.
template <int BM, int BN, bool KTAIL>
__global__ __launch_bounds__(512) void prefill_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y,
    int M, int K, int N, int gsh, int n_tiles, int splits, int kps,
    float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const a_ring = smem;
  char* const b_ring = smem + kAStages * Cfg<BM, BN>::kATileBytes;
  pin_arg(x);
  pin_arg(qw);
  pin_arg(qz);
  pin_arg(sc);
  pin_arg(bias);
  pin_arg(y);
  pin_arg(partial);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Tile t = tile_of<BM, BN>(n_tiles, splits, kps, (K + BK - 1) / BK);
  // Each SIMD runs one consumer and one producer wave, whose matrix-core
  // and dequantisation instructions share the SIMD's vector issue port: the
  // consumer goes first when both are ready, so the matrix cores are fed
  // and the producer fills the cycles in between (3-11 % faster, most at
  // M = 128-1024).
  if (wave < 4) __builtin_amdgcn_s_setprio(1);
  // The partial plane is 16-byte aligned (workspace layout, N % 8 == 0).
  const int out_mode = splits == 1
                           ? ((reinterpret_cast<uintptr_t>(y) & 15) == 0 ? kOutStagedY : kOutDirect)
                           : (partial_stages<BM, BN>() ? kOutStagedPartial : kOutDirect);
  if (wave >= 4)
    producer<BM, BN, KTAIL>(x, qw, qz, sc, y, M, K, N, gsh, t, a_ring, b_ring, wave - 4,
                            tid - 256, out_mode, partial);
  else if constexpr (Cfg<BM, BN>::MF16)
    consumer16<BM, BN>(bias, y, partial, M, N, splits, t, a_ring, b_ring, wave, tid & 63, out_mode);
  else
    consumer<BM, BN>(bias, y, partial, M, N, splits, t, a_ring, b_ring, wave, tid & 63, out_mode);
}

// y = sum of the split partials, in split order (deterministic), + bias.
// Thread i takes four adjacent outputs (N % 8 == 0, so a quad never crosses
// a row): 16-byte loads of each split's partials (the workspace is 16-byte
// aligned), one 8-byte store when y allows it, else 2-byte ones.  SB bounds
// the split count: loads past the last split are clamped (unconditional, so
// all are in flight together) and their values dropped.
template <int SB>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float* __restrict__ partial,
                                                             const _Float16* __restrict__ bias,
                                                             _Float16* __restrict__ y, int M, int N,
                                                             int splits) {
  const size_t plane = static_cast<size_t>(M) * N;
  const size_t e = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= plane) return;
  floatx4 v[SB];
#pragma unroll
  for (int u = 0; u < SB; ++u)
    v[u] = *reinterpret_cast<const floatx4*>(partial + min(u, splits - 1) * plane + e);
  floatx4 sum = v[0];
#pragma unroll
  for (int u = 1; u < SB; ++u) {
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    sum += (u < splits) ? v[u] : zero;
  }
  if (bias) {
    const _Float16* bq = bias + e % N;
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] += static_cast<float>(bq[q]);
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


// ---------------------------------------------------------------------------
// Packed-weight prefill tile: 256 rows x BN columns (BN = 256 or 192), four
// waves, no producer waves.  The dequantised weight tile dominates the LDS
// traffic of the tile above (written once, read by two waves), so here the
// packed words themselves are staged -- a quarter of the bytes -- and each
// wave dequantises the operands it multiplies.
//
// * Wave arrangements (WAVES waves, WM along M): four waves of 256 rows x
//   64 columns (WM = 1: each dequantised weight fragment feeds eight MFMAs,
//   the dequantisation work is about a quarter of the matrix-core time), four
//   of 128 x BN/2 (WM = 2, the 192-column tile), or eight of 128 x 64 (two
//   waves per SIMD, each weight dequantised by two waves).  Accumulators:
//   256 (four waves) or 128 (eight) fp32 per lane.
// * A 3-slot ring of K steps (64 k each), filled two steps ahead by 16-byte
//   direct-to-LDS copies, the same eleven per wave per step: the x tile
//   (256 rows of 128 bytes, chunks XOR-swizzled by (row / 2) % 8 as above),
//   the packed rows (BN / 2 bytes per k-row, eight k-rows per KiB; the
//   16-byte chunks of row r rotated by r / 2 (BN = 256) or r / 8 (BN = 192),
//   which keeps the transposing reads below at most two-way bank conflicts)
//   and the zero words and scales of the step's group (group size a
//   multiple of 64, or one group; two waves copy each, the same bytes).
// * The weight operand is read with the 4-bit transposing LDS read: the 16
//   lanes of a group point at 16 consecutive k-rows of one 16-column unit,
//   and lane i receives column i's 16 nibbles -- 16 consecutive k of its
//   column, the operand of two MFMAs.  Lane halves cover k-rows 0-15 and
//   16-31 of a 32-row pair, so MFMA e of pair p contracts k
//   32p + 16h + 8e + (0..7) (h = lane / 32), and x is read with the same
//   k order.
// * Dequantisation: a byte shuffle places nibbles 2b and 2b+1 of the word
//   (byte b of w and of w >> 4) in the two float16 halves, OR-ed into 1024.0
//   (1024 + q, exact); a packed add of -(1024 + z) gives q - z exactly and a
//   packed multiply by s rounds once: float16_RNE((q - z) * s), the value
//   awq_dequant writes.
// * One split only (the plan sends problems with fewer tiles than CUs to the
//   split tile above).  Epilogue staged through LDS: float16(acc + bias)
//   written as a row-major tile, copied out with 16-byte stores.
// * Measured against the tile above (same box, same process): level at
//   M = 4096, K = 14336, N = 4096 (444-448 us against 438-441 us for every
//   arrangement) and slower at M = 2048, K = 4096, N = 12288 (241-247 us
//   against 217-218 us), so the planner takes it only when asked
//   (AWQ_OPT_PREFILL_PACKED).
namespace pk {
constexpr int kBM = 256;
// WM waves along M (4 / WM along N): WM = 1 gives each wave all 256 rows
// and 64 columns (every dequantised fragment feeds 8 MFMAs); WM = 2 gives
// 128 rows and BN / 2 columns.
template <int BN, int WM, int WAVES = 4>
struct L {
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
  static_assert((BN == 256 && (WAVES == 4 || WM == 2)) || (BN == 192 && WM == 2 && WAVES == 4),
                "packed tile shape");
  static_assert(WM == 1 || WM == 2, "waves along M");
  static constexpr int WN = WAVES / WM;
  static constexpr int XPW = 32 / WAVES;        // x copies per wave per step
  static constexpr int WPW = 8 / WAVES;         // packed-row copies per wave per step
  static constexpr int kLoads = XPW + WPW + 1;  // loads per wave per step
  static constexpr int NB = BN / WN / 32;       // 32-column blocks per wave
  static constexpr int MI = 8 / WM;             // 32-row blocks per wave
  static constexpr int WRow = BN / 2;           // packed bytes per k-row
  static constexpr int WChunks = WRow / 16;     // 16-byte chunks per packed row: 8 or 6
  static constexpr int XTile = kBM * BK * 2;    // 32 KiB
  static constexpr int WTile = BK / 8 * 1024;   // 8 k-rows per KiB (BN = 192 leaves gaps)
  static constexpr int ZOff = XTile + WTile;    // zero words (1 KiB area)
  static constexpr int SOff = ZOff + 1024;      // scales (1 KiB area)
  static constexpr int Slot = SOff + 1024;
  static constexpr int S = 3;                   // copies run S - 1 steps ahead
  static constexpr int OutPitch = BN * 2 + 16;  // staged output row, bytes
  static constexpr int Ring = S * Slot;
  static constexpr int Lds = Ring > kBM * OutPitch ? Ring : kBM * OutPitch;
};
static_assert(L<256, 1>::Lds <= 160 * 1024 && L<192, 2>::Lds <= 160 * 1024 &&
                  L<256, 2, 8>::Lds <= 160 * 1024,
              "LDS budget");

// Physical 16-byte chunk of logical chunk c in packed k-row r (see above).
template <int BN>
__device__ __forceinline__ int w_chunk(int r, int c) {
  if constexpr (BN == 256) return (c + (r >> 1)) & 7;
  else return (c + (r >> 3)) % 6;
}
// Logical chunk held by physical chunk pc of k-row r (the inverse).
template <int BN>
__device__ __forceinline__ int w_logical(int r, int pc) {
  if constexpr (BN == 256) return (pc - (r >> 1)) & 7;
  else return (pc + 6 - (r >> 3) % 6) % 6;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef int v2i __attribute__((ext_vector_type(2)));

// Eight k of one column from a word of nibbles (k = 2b: low nibble of byte
// b, k = 2b + 1: its high nibble), dequantised with zero pair zn =
// -(1024 + z) and scale pair s2.
__device__ __forceinline__ half8_t dequant8(uint32_t d, half2_t zn, half2_t s2) {
  const uint32_t ds = d >> 4;
  half8_t out;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sel = 0x0C000C00u | (static_cast<uint32_t>(4 + b) << 16) | b;
    const half2_t h = as_h2(magic_pair(__builtin_amdgcn_perm(ds, d, sel), 0));
    const half2_t w = (h + zn) * s2;
    out[2 * b] = w[0];
    out[2 * b + 1] = w[1];
  }
  return out;
}
}  // namespace pk

template <int BN, int WM, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void prefill_packed_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint32_t* __restrict__ qz, const _Float16* __restrict__ sc,
    const _Float16* __restrict__ bias, _Float16* __restrict__ y, int M, int K, int N, int gsh,
    int n_tiles) {
  using C = pk::L<BN, WM, WAVES>;
  constexpr int MI = C::MI, NB = C::NB, S = C::S, WN = C::WN;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  pin_arg(x);
  pin_arg(qw);
  pin_arg(qz);
  pin_arg(sc);
  pin_arg(bias);
  pin_arg(y);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int nkt = K / BK;
  const Tile t = tile_of<pk::kBM, BN>(n_tiles, 1, nkt, nkt);
  const int NW = N >> 3;
  const int G = gsh >= 31 ? 1 : (K >> gsh);
  const v4i rx = raw_rsrc(x, static_cast<uint32_t>(M) * K * 2u);
  const v4i rq = raw_rsrc(qw, static_cast<uint32_t>(K) * NW * 4u);
  const v4i rz = raw_rsrc(qz, static_cast<uint32_t>(G) * NW * 4u);
  const v4i rs = raw_rsrc(sc, static_cast<uint32_t>(G) * N * 2u);

  // x copies: instruction i of this wave covers tile rows 8 * (XPW * wave + i)
  // .. +7; lane -> row lane / 8, physical chunk lane % 8.  Rows past M are
  // clamped (they only reach rows that are never stored).
  uint32_t x_off[C::XPW];
#pragma unroll
  for (int i = 0; i < C::XPW; ++i) {
    const int r = 8 * (C::XPW * wave + i) + (lane >> 3);
    const int logical = (lane & 7) ^ ((r >> 1) & 7);
    const int m = min(t.m0 + r, M - 1);
    x_off[i] = static_cast<uint32_t>(m) * K * 2u + 16u * logical;
  }
  // Packed-row copies: instruction i (< WPW) of this wave covers k-rows
  // 8 * (WPW * wave + i) .. +7 of the step, one KiB of LDS each; lane -> row
  // lane / WChunks, physical chunk lane % WChunks.  When BN = 192 the lanes
  // past 8 rows read out of range and write zeros into the gap after them.
  constexpr int kWLanes = 8 * C::WChunks;
  uint32_t w_off[C::WPW];
#pragma unroll
  for (int i = 0; i < C::WPW; ++i) {
    const int r = 8 * (C::WPW * wave + i) + lane / C::WChunks;
    const int logical = pk::w_logical<BN>(r, lane % C::WChunks);
    w_off[i] = offset_or_oob(lane < kWLanes,
                             (static_cast<uint32_t>(r) * NW + (t.n0 >> 3)) * 4u + 16u * logical);
  }
  // Even waves copy the zero words of the tile's columns, odd waves the
  // scales (both copies of each write the same bytes; the lanes past them
  // copy bytes that are never read, zeros past the end of a buffer).  The
  // choices are wave-uniform selects, so every wave runs the same code.
  const bool zs_scales = (wave & 1) != 0;
  const v4i rzs = zs_scales ? rs : rz;
  const uint32_t zs_off = zs_scales ? (static_cast<uint32_t>(t.n0) * 2u + 16u * lane)
                                    : (static_cast<uint32_t>(t.n0 >> 3) * 4u + 16u * lane);
  const uint32_t zs_row = zs_scales ? static_cast<uint32_t>(N) * 2u : static_cast<uint32_t>(NW) * 4u;
  const uint32_t zs_dst = zs_scales ? C::SOff : C::ZOff;
  auto copy_step = [&](int s) {   // the copies of K step s (clamped) into slot s % S
    const int kstep = t.kt0 + min(s, nkt - 1);
    const uint32_t slot = lds_addr(smem + (s % S) * C::Slot);
#pragma unroll
    for (int i = 0; i < C::XPW; ++i)
      copy_to_lds(rx, x_off[i] + static_cast<uint32_t>(kstep) * (BK * 2), 0u,
                  __builtin_amdgcn_readfirstlane(slot + 1024u * (C::XPW * wave + i)));
#pragma unroll
    for (int i = 0; i < C::WPW; ++i)
      copy_to_lds(rq, w_off[i] + static_cast<uint32_t>(kstep) * (BK * NW * 4), 0u,
                  __builtin_amdgcn_readfirstlane(slot + C::XTile +
                                                 (C::WPW * wave + i) * 1024u));
    const int grp = gsh >= 31 ? 0 : ((kstep * BK) >> gsh);
    copy_to_lds(rzs, zs_off + static_cast<uint32_t>(grp) * zs_row, 0u,
                __builtin_amdgcn_readfirstlane(slot + zs_dst));
  };
  // Loads per wave per step: XPW + WPW + 1 (kLoads).
#pragma unroll
  for (int s = 0; s < S - 1; ++s) copy_step(s);

  floatx16 acc[MI][NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int half_l = lane >> 5;
  int a_row[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_row[mi] = 32 * MI * wm + 32 * mi + (lane & 31);
  int b_unit[NB], zs_col[NB];
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    b_unit[ni] = 2 * (NB * wn + ni) + ((lane >> 4) & 1);
    zs_col[ni] = 32 * (NB * wn + ni) + (lane & 31);
  }

  // Per-lane LDS byte offsets within a slot, computed once: the x operand
  // of pair kp, MFMA e for row block 0 (row block mi adds 4096 * mi; the
  // chunk swizzle (row / 2) % 8 is the same for all of the lane's rows), the
  // weight operand of pair kp, column block ni, and the zero word and scale
  // of column block ni.
  const int sw = ((lane & 31) >> 1) & 7;
  uint32_t a_off[2][2], b_off[2][NB], z_off[NB], z_sh[NB], s_off[NB];
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      a_off[kp][e] = static_cast<uint32_t>((32 * MI * wm + (lane & 31)) * 128 +
                                           16 * ((4 * kp + 2 * half_l + e) ^ sw));
    const int brow = 32 * kp + 16 * half_l + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) {
      const int u = b_unit[ni];
      b_off[kp][ni] = static_cast<uint32_t>(C::XTile + (brow >> 3) * 1024 + (brow & 7) * C::WRow +
                                            16 * pk::w_chunk<BN>(brow, u >> 1) + 8 * (u & 1));
    }
  }
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int c = zs_col[ni];
    z_off[ni] = static_cast<uint32_t>(C::ZOff + 4 * (c >> 3));
    z_sh[ni] = static_cast<uint32_t>(4 * (c & 7));
    s_off[ni] = static_cast<uint32_t>(C::SOff + 2 * c);
  }

  // Operands of one 32-k pair: x fragments of both MFMAs and the packed
  // weight words of each column block.
  struct Ops {
    half8_t a[MI][2];
    pk::v2i w[NB];
  };
  auto read_ops = [&](int j, int kp, Ops& o) {
    const char* slot = smem + j * C::Slot;
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
      o.w[ni] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
          (__attribute__((address_space(3))) pk::v2i*)(slot + b_off[kp][ni]));
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        o.a[mi][e] = *reinterpret_cast<const half8_t*>(slot + a_off[kp][e] + 4096 * mi);
  };
  half2_t zn[S][NB], s2[S][NB];
  auto read_zs = [&](int j) {
    const char* slot = smem + j * C::Slot;
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) {
      const uint32_t z = (*reinterpret_cast<const uint32_t*>(slot + z_off[ni]) >> z_sh[ni]) & 0xFu;
      zn[j][ni] = as_h2(((0xE400u | z) << 16) | 0xE400u | z);
      const uint32_t sb = *reinterpret_cast<const uint16_t*>(slot + s_off[ni]);
      s2[j][ni] = as_h2((sb << 16) | sb);
    }
  };
  // Step boundary: step k is in LDS (this wave's copies of it have landed,
  // and the barrier covers the other waves'), every wave's reads of the
  // previous slot are done, so that slot takes step k + S - 1.
  auto step_sync = [&](int k) {
    pk::wait_vm<(S - 2) * C::kLoads>();
    __syncthreads();
    copy_step(k + S - 1);
  };

  // Step kt sits in slot j = kt % S (static: the loop is unrolled by S).
  // Its first pair's operands are in set 0 when it starts; the second
  // pair's are read into set 1 at once, and halfway through the second
  // pair's MFMAs the next step's boundary (wait, barrier, copies) is passed
  // and its zero/scale pairs and first operands read into set 0, so the
  // matrix cores keep queued work while the wave waits.  Units run x-block
  // major (MFMA e of the pair, then column block ni); each is dequantised
  // one unit ahead of its MFMAs.
  constexpr int kUnits = 2 * NB;
  Ops ops[2];
  step_sync(0);
  read_zs(0);
  read_ops(0, 0, ops[0]);
  // (The step boundary also runs after the last step: its copies re-read
  // the last step, its reads go unused; the loop body stays branch-free.)
  auto step = [&](int kt, int j) {
    const int jn = (j + 1) % S;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      Ops& cur = ops[kp];
      if (kp == 0) read_ops(j, 1, ops[1]);
      half8_t b = pk::dequant8(static_cast<uint32_t>(cur.w[0][0]), zn[j][0], s2[j][0]);
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int e = u / NB, ni = u % NB;
        if (kp == 1 && u == kUnits / 2 && kt + 1 < nkt) {
          step_sync(kt + 1);
          read_zs(jn);
          read_ops(jn, 0, ops[0]);
        }
        half8_t bn = b;
        if (u + 1 < kUnits) {
          const int e1 = (u + 1) / NB, ni1 = (u + 1) % NB;
          bn = pk::dequant8(static_cast<uint32_t>(cur.w[ni1][e1]), zn[j][ni1], s2[j][ni1]);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[mi][e], b, acc[mi][ni], 0, 0, 0);
        b = bn;
      }
    }
  };
  int kt = 0;
  for (; kt + S <= nkt; kt += S) {
    step(kt, 0);
    step(kt + 1, 1);
    step(kt + 2, 2);
  }
  if (kt < nkt) step(kt, 0);
  if (kt + 1 < nkt) step(kt + 1, 1);
  pk::wait_vm<0>();

  // Epilogue: every wave is past its last LDS read; stage float16(acc +
  // bias) as a row-major 256 x BN tile, then copy it out with 16-byte
  // stores (y 16-byte aligned) or 2-byte stores.
  __syncthreads();
  char* stage = smem;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int lcol = (BN / WN) * wn + 32 * ni + (lane & 31);
    const int col = t.n0 + lcol;
    const float bv = (bias && col < N) ? static_cast<float>(bias[col]) : 0.f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = 32 * MI * wm + 32 * mi + 8 * (r >> 2) + 4 * half_l + (r & 3);
        *reinterpret_cast<_Float16*>(stage + lrow * C::OutPitch + 2 * lcol) =
            static_cast<_Float16>(acc[mi][ni][r] + bv);
      }
  }
  __syncthreads();
  constexpr int kChunksPerRow = BN / 8;
  const bool y16 = (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll 4
  for (int c = tid; c < pk::kBM * kChunksPerRow; c += 64 * WAVES) {
    const int lrow = c / kChunksPerRow;
    const int lcol = 8 * (c - lrow * kChunksPerRow);
    const int row = t.m0 + lrow;
    const int col = t.n0 + lcol;
    if (row >= M || col >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * C::OutPitch + 2 * lcol);
    _Float16* dst = y + static_cast<size_t>(row) * N + col;
    if (y16) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      const half8_t hv = __builtin_bit_cast(half8_t, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = hv[q];
    }
  }
}

}  // namespace

hipError_t launch_prefill_packed(const _Float16* x, const uint32_t* qweight,
                                 const uint32_t* qzeros, const _Float16* scales,
                                 const _Float16* bias, _Float16* y, int M, int K, int N,
                                 int group_shift, int bn, int wm, int m_tiles, int n_tiles,
                                 hipStream_t stream) {
  if (K % BK != 0) return hipErrorInvalidValue;
  const dim3 grid(m_tiles * n_tiles);
  auto go = [&](auto kernel, int lds, int waves) {
    hipLaunchKernelGGL(kernel, grid, dim3(64 * waves), lds, stream, x, qweight, qzeros, scales,
                       bias, y, M, K, N, group_shift, n_tiles);
  };
  // wm: 1 or 2 waves along M of four; 3: eight waves, two along M.
  if (bn == 256 && wm == 1) go(prefill_packed_kernel<256, 1, 4>, pk::L<256, 1>::Lds, 4);
  else if (bn == 256 && wm == 2) go(prefill_packed_kernel<256, 2, 4>, pk::L<256, 2>::Lds, 4);
  else if (bn == 256 && wm == 3) go(prefill_packed_kernel<256, 2, 8>, pk::L<256, 2, 8>::Lds, 8);
  else if (bn == 192 && wm == 2) go(prefill_packed_kernel<192, 2, 4>, pk::L<192, 2>::Lds, 4);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, const _Float16* bias, _Float16* y,
                          int M, int K, int N, int group_shift, int bm, int bn,
                          int m_tiles, int n_tiles, int splits, int ksteps, void* workspace,
                          hipStream_t stream) {
  // Workspace (split K only), laid out like the decode exchange's so that
  // one buffer serves both: the accumulator region (left untouched, it must
  // stay zero), then [splits][M][N] partials.
  char* ws = static_cast<char*>(workspace);
  float* partial = ws ? reinterpret_cast<float*>(ws + kAtomicRegionBytes) : nullptr;
  const dim3 grid(m_tiles * n_tiles * splits);
  const bool tail = K % BK != 0;
  auto go = [&](auto kernel, int lds) {
    hipLaunchKernelGGL(kernel, grid, dim3(512), lds, stream, x, qweight, qzeros, scales, bias, y,
                       M, K, N, group_shift, n_tiles, splits, ksteps, partial);
  };
  if (bm == 256 && bn == 192)
    tail ? go(prefill_kernel<256, 192, true>, lds_bytes<256, 192>())
         : go(prefill_kernel<256, 192, false>, lds_bytes<256, 192>());
  else if (bm == 256)
    tail ? go(prefill_kernel<256, 128, true>, lds_bytes<256, 128>())
         : go(prefill_kernel<256, 128, false>, lds_bytes<256, 128>());
  else if (bm == 128)
    tail ? go(prefill_kernel<128, 128, true>, lds_bytes<128, 128>())
         : go(prefill_kernel<128, 128, false>, lds_bytes<128, 128>());
  else
    tail ? go(prefill_kernel<64, 128, true>, lds_bytes<64, 128>())
         : go(prefill_kernel<64, 128, false>, lds_bytes<64, 128>());
  if (splits > 1) {
    const size_t quads = static_cast<size_t>(M) * N / 4;
    const dim3 rgrid(static_cast<unsigned>((quads + 255) / 256));
    if (splits <= 2)
      hipLaunchKernelGGL(prefill_reduce_kernel<2>, rgrid, dim3(256), 0, stream, partial, bias, y,
                         M, N, splits);
    else if (splits <= 4)
      hipLaunchKernelGGL(prefill_reduce_kernel<4>, rgrid, dim3(256), 0, stream, partial, bias, y,
                         M, N, splits);
    else
      hipLaunchKernelGGL(prefill_reduce_kernel<kPrefillMaxSplits>, rgrid, dim3(256), 0, stream,
                         partial, bias, y, M, N, splits);
  }
  return hipGetLastError();
}

}  // namespace awq
