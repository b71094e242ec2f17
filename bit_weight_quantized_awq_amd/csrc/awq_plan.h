// Host-side validation and kernel planning for the W4A16 linear forward.
// HIP-free: this translation unit is compiled with a plain host compiler too,
// so every argument check can be exercised (and sanitised) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace awq {

// Decode kernel geometry: a work-group is 4 waves; waves 0/1 and 2/3 split
// the K range of the work-group, waves 0/2 and 1/3 split its 256 columns.
constexpr int kDecodeCols = 256;         // columns per work-group
constexpr int kDecodeRowsPerStep = 32;   // rows one wave consumes per step
constexpr int kDecodeBlockM = 16;        // rows of one 16x16 MFMA output block
// Rows of the decode kernels: one MFMA row block, or two for the LDS
// variant when each wave's rows lie in one quantisation group.
constexpr int kDecodeMaxM = 32;
// The planner takes the two-block decode by itself only for weights of at
// least this many elements (16 MiB packed) whose split partials are at most
// half the packed bytes; the prefill kernel runs the others faster
// (K = 4096, N = 4096, g = 64, M = 20: 10.9 against 12.1 us).
constexpr int64_t kDecodeTwoBlockMinWeights = int64_t{1} << 25;
// Split-K exchange workspace, in two parts:
//  * a fixed accumulator region for the atomic exchange (M <= 4, N <= 65536):
//    an 8-byte fixed-point accumulator per output element, then an 8-byte
//    mask (one bit per split) per output element;
//  * 4 bytes per split per output element for partials (every split's for
//    the two-launch exchange, only the float ones for the atomic exchange).
// The first part is zero between calls (the atomic exchange resets what it
// used) and no exchange writes partials into it, so calls of any shapes can
// share one workspace.  The atomic exchange counts at most 63 splits.
constexpr int kDecodeMaxSplits = 63;
constexpr int kDecodeAtomicMaxM = 4;
constexpr int kDecodeGatherMaxM = 4;
// Eight waves of four steps for the two-launch exchange when they give this
// many work-groups (one resident round of 139 KiB work-groups, one per CU).
constexpr int64_t kDecodeEightWaveMinWGs = 160;
constexpr int64_t kDecodeEightWaveMaxWGs = 256;
constexpr int kDecodeAtomicMaxN = 65536;
// The atomic exchange (one device-scope atomic per output element and
// split) is possible for at most kDecodeAtomicMaxM rows, and the planner takes
// it while a call issues fewer than kDecodeAtomicMaxOps atomics; otherwise
// plain partial stores summed by a second kernel.  Same box, two launches
// against atomics: K = 4096, N = 4096, M = 4 (524K atomics): 8.5 against
// 10.4 us; K = 8192, N = 7168, M = 4 (458K): 12.3 against 12.7 us; M = 3
// (344K): 12.2 against 11.9 us; M = 1 (115K): 11.7 against 10.0 us.
constexpr int64_t kDecodeAtomicMaxOps = 380000;
constexpr bool decode_atomic_capable(int64_t M, int64_t N) {
  return M <= kDecodeAtomicMaxM && N <= kDecodeAtomicMaxN;
}
constexpr size_t kAtomicRegionBytes = static_cast<size_t>(kDecodeAtomicMaxM) * kDecodeAtomicMaxN * 16;

// Prefill kernel tile: 64, 128 or 256 rows (the smallest that covers the
// batch, so small batches waste no matrix-core work on padding rows), 128
// or 192 columns (192 only with 256 rows: the wider tile moves fewer LDS
// bytes per flop; it is chosen when it also takes fewer rounds of
// work-groups over the CUs), 64 K rows per step.
constexpr int kPrefillBM = 256;
constexpr int kPrefillMinBM = 64;
constexpr int kPrefillBN = 128;
constexpr int kPrefillWideBN = 192;
constexpr int kPrefillBK = 64;
// Prefill split K: shapes with fewer output tiles than kPrefillTargetWGs
// (one work-group per CU) split the K steps over up to kPrefillMaxSplits
// work-groups per tile, each with at least kPrefillMinSplitSteps steps; a
// second kernel sums the fp32 partials.  The workspace has the decode
// exchange's layout (so one buffer serves both): the accumulator region
// (unused here, left zero), then [splits][M][N] partials.
constexpr int kPrefillTargetWGs = 256;
constexpr int kPrefillMaxSplits = 8;
constexpr int kPrefillMinSplitSteps = 8;
// At most this many K steps (K <= 4096) the planner prefers lower tiles
// without a split to the 256-row tile with one.
constexpr int64_t kPrefillShortKSteps = 64;
// Packed-weight prefill tile (256 rows x 256 or 192 columns, packed words
// staged in LDS, dequantised by the matrix-core waves): K % 64 == 0,
// N % 32 == 0, qweight 16-byte aligned, groups of a multiple of 64 rows (or
// one group), and at least kPrefillTargetWGs tiles (it does not split K).
constexpr int kPackedBM = 256;
constexpr int kPackedBN = 256;
constexpr int kPackedNarrowBN = 192;
constexpr bool kPackedAuto = false;   // chosen automatically (else only when forced)

struct Problem {
  int64_t M, K, N;
  int64_t g;   // resolved group size (K when -1 was passed)
  int64_t G;   // number of groups
};

struct Plan {
  int path;          // awq_path value
  int steps;         // decode: 32-row steps per wave; prefill: K steps per split
  int splits;        // work-groups along K per output tile (decode and prefill)
  int n_tiles;       // column tiles
  int m_tiles;       // prefill: row tiles
  size_t ws_bytes;   // workspace bytes
  bool decode_lds;    // decode: LDS-streaming variant (N % 32 == 0) or register variant
  int group_shift;    // prefill: log2(group size), or 31 for a single group
  int prefill_bn;     // prefill: tile width (kPrefillBN or kPrefillWideBN)
  int prefill_bm;     // prefill: tile height (64, 128 or kPrefillBM)
  int decode_waves;   // decode, LDS variant: waves along K per work-group (4 or 8)
  bool decode_atomic; // decode, split K: the atomic exchange (else two launches)
  bool prefill_packed;  // prefill: the packed-weight 256-row tile (one split)
  int packed_wm;        // packed tile: waves along M (1 or 2)
};

// Checks of the page's WQLinear construction (K % g == 0, N % 8 == 0, the -1
// rule) plus this library's argument rules.  Returns an awq_status value.
int validate_shape(int64_t M, int64_t K, int64_t N, int64_t group_size, Problem* out);

// Pointer checks: required pointers non-NULL, element alignment.
int validate_gemm_pointers(const void* x, const void* qweight, const void* qzeros,
                           const void* scales, const void* bias, const void* y, int64_t M);
int validate_dequant_pointers(const void* qweight, const void* qzeros,
                              const void* scales, const void* w);

// The unquantised baseline (awq_dense_gemv): 1 <= M <= kDenseMaxM (M == 0 is
// a no-op), K % 8 == 0, M * K <= kDenseMaxMK (x is staged in LDS), x and w
// 16-byte aligned, bias and y 2-byte aligned.  Returns an awq_status value.
constexpr int kDenseMaxM = 4;
constexpr int64_t kDenseMaxMK = 65536;
int validate_dense(const void* x, const void* w, const void* bias, const void* y, int64_t M,
                   int64_t K, int64_t N);

// Alignment flags: whether x, scales and qweight start on a 16-byte boundary.
struct Alignment {
  bool x, scales, qweight;
};

bool decode_supported(const Problem& p, const Alignment& al);
bool prefill_supported(const Problem& p, const Alignment& al);

// awq_gemm_workspace_size: the larger of the decode and prefill plans' needs
// (0 for invalid shapes).
size_t gemm_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size);

// force: 0 = automatic, otherwise an awq_path value.  Returns an awq_status.
int make_plan(const Problem& p, const Alignment& al, int force, Plan* out);

// Planner overrides for tests and tuning (awq_set_option / awq_get_option):
// process-wide values, each initialised once from its environment variable
// (AWQ_FORCE_PATH = decode | prefill | generic, AWQ_DECODE_STEPS,
// AWQ_DECODE_GATHER_MAX_M, AWQ_PREFILL_BM, AWQ_PREFILL_BN,
// AWQ_PREFILL_SPLITS) on first use.  kOptAuto = the planner's own choice.
constexpr int kOptAuto = -1;
int option(int opt);
int set_option(int opt, int64_t value);
int get_option(int opt, int64_t* value);

// Largest batch for which the LDS decode kernel gathers an act-order x
// itself (each column tile gathers its K range again, so the scattered loads
// grow with M x N / 256; beyond this a separate reorder pass is cheaper).
// AWQ_OPT_DECODE_GATHER_MAX_M overrides it (0 disables).
int decode_gather_max_m();

// The forced kernel family: 0 (automatic), an awq_path value, or -1 when
// AWQ_FORCE_PATH held an unrecognised value.
int forced_path();

// Row-to-group map problems (awq_dequant_gidx, awq_gemm_gidx): M >= 0,
// K > 0, N > 0 with N % 8 == 0, num_groups >= 1, every operand (including
// scales, num_groups x N) below 2^31 elements.  Fills p with g = 0 (no
// contiguous grouping) and G = num_groups.  Returns an awq_status value.
int validate_gidx_shape(int64_t M, int64_t K, int64_t N, int64_t num_groups, Problem* out);

// Sorted layout of a row-to-group map (awq_gidx_layout): rows stably sorted
// by group, then cut into blocks that each lie in one group.  When every
// group holds K / num_groups rows and that count is a power of two of at
// least kGidxBlockRows (activation order), a block is a whole group and no
// row is added; otherwise blocks are kGidxBlockRows rows and the last block
// of each group is padded with null rows (perm entry -1).  Writes *rows
// (rows of the sorted weight), *block_rows and *blocks always (on success
// or AWQ_ERROR_SHAPE); perm (rows entries) and block_group (blocks entries:
// the map's group of each block) when non-NULL and their capacities
// suffice, else AWQ_ERROR_SHAPE.  Entries of g_idx outside [0, num_groups)
// give AWQ_ERROR_INVALID_VALUE.
constexpr int64_t kGidxBlockRows = 32;
int gidx_layout(const int32_t* g_idx, int64_t K, int64_t num_groups, int32_t* perm,
                int64_t perm_capacity, int32_t* block_group, int64_t block_capacity,
                int64_t* rows, int64_t* block_rows, int64_t* blocks);

// Workspace of awq_gemm_sorted: the awq_gemm workspace of the sorted problem
// (M, rows, N, block_rows), at least the fixed accumulator region, rounded
// up to 256 bytes, then room for x with its columns reordered (M x rows
// float16, rounded up to 256 bytes).  0 for M == 0 or invalid shapes.
size_t sorted_workspace_size(int64_t M, int64_t rows, int64_t N, int64_t block_rows);
// Byte offset of the reordered x inside that workspace.
size_t sorted_x_offset(int64_t M, int64_t rows, int64_t N, int64_t block_rows);

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace awq
