/*
 * awq.h -- C ABI of the MI355X (gfx950) W4A16 weight-quantised linear forward.
 *
 * The operation is the forward of the AWQ WQLinear layer described on the page
 * "Predibase Lorax AWQ WQLinear" (sections Description and I/O Contract):
 *
 *     y[M, N] = x[M, K] . W[K, N] (+ bias[N]),
 *     W[k, n] = float16_RNE((q[k, n] - z[k / g, n]) * s[k / g, n])
 *
 * with K = in_features, N = out_features, g = group_size (g = K when -1 is
 * passed, G = K / g groups).  Data formats (row-major, contiguous):
 *
 *   x        float16  (M, K)
 *   qweight  int32    (K, N / 8)  eight unsigned 4-bit values per word along
 *                                 the output dimension; bits [4j, 4j+3] of
 *                                 word (k, c) hold q[k, 8c + j]
 *   qzeros   int32    (G, N / 8)  zero points z, packed like qweight
 *   scales   float16  (G, N)      scales s
 *   bias     float16  (N) or NULL
 *   y        float16  (M, N)
 *
 * The page fixes the packing (eight 4-bit values per int32 along the output
 * dimension), the shape of qweight, the -1 rule for group_size and the checks
 * K % group_size == 0 and N % 8 == 0.  It does not fix the nibble order inside
 * a word, the layouts of qzeros and scales, or the dequantisation rounding;
 * the readings above are the ones this library implements.
 *
 * Conventions for every entry point:
 *   - Pointers named x, qweight, qzeros, scales, bias, y, w and workspace are
 *     DEVICE pointers owned by the caller.  The library allocates nothing and
 *     keeps no pointer after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; nothing synchronises.
 *   - Arguments are validated on the host before any HIP call.  On a non-zero
 *     return nothing was enqueued and no output was written, except
 *     AWQ_ERROR_HIP, which reports a failed launch.
 *   - Element alignment is required (2 bytes for float16 pointers, 4 bytes for
 *     int32 pointers).  Faster kernels are chosen when x, scales and qweight
 *     are 16-byte aligned and K % 8 == 0; other legal inputs take a general
 *     kernel.
 *   - Every operand must hold fewer than 2^31 elements (M*K, M*N, K*N).
 */
#ifndef AWQ_MI355X_AWQ_H_
#define AWQ_MI355X_AWQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AWQ_ABI_VERSION 5

/* Status codes returned by every entry point. */
enum awq_status {
  AWQ_SUCCESS = 0,
  AWQ_ERROR_INVALID_VALUE = 1, /* NULL required pointer, M < 0, K <= 0, N <= 0,
                                  group_size == 0 or < -1, unknown path request */
  AWQ_ERROR_SHAPE = 2,         /* N % 8 != 0, K % group_size != 0 (page checks),
                                  or an operand with 2^31 or more elements */
  AWQ_ERROR_MISALIGNED = 3,    /* a pointer not aligned to its element size */
  AWQ_ERROR_WORKSPACE = 4,     /* workspace smaller than awq_gemm_workspace_size */
  AWQ_ERROR_HIP = 5,           /* a HIP launch reported an error */
  AWQ_ERROR_SCRATCH = 6        /* awq_gemm_noalloc: the problem's split-K workspace
                                  exceeds AWQ_NOALLOC_SCRATCH_BYTES */
};

/* Kernel families that awq_gemm can run (see awq_gemm_plan). */
enum awq_path {
  AWQ_PATH_DECODE = 1,  /* split-K MFMA skinny GEMM, M <= 16 (17-32 on large weights) */
  AWQ_PATH_PREFILL = 2, /* LDS-tiled MFMA GEMM with dequantisation into LDS */
  AWQ_PATH_GENERIC = 3  /* any legal shape or alignment; slow */
};

/* Planner overrides, for tests and tuning (awq_set_option). */
enum awq_option {
  AWQ_OPT_FORCE_PATH = 1,          /* an awq_path value: run that kernel family */
  AWQ_OPT_DECODE_STEPS = 2,        /* 1, 2, 4 or 8: 32-row steps per decode wave */
  AWQ_OPT_DECODE_GATHER_MAX_M = 3, /* 0..16: largest batch whose sorted-weight
                                      forward gathers x inside the decode kernel */
  AWQ_OPT_PREFILL_BM = 4,          /* 64, 128 or 256: prefill tile rows */
  AWQ_OPT_PREFILL_BN = 5,          /* 128, 192 or 256: prefill tile columns
                                      (256 for the packed-weight tile only) */
  AWQ_OPT_PREFILL_SPLITS = 6,      /* 1..8: prefill work-groups along K per tile */
  AWQ_OPT_DECODE_WAVES = 7,        /* 4 or 8: waves along K per decode work-group */
  AWQ_OPT_PREFILL_PACKED = 8       /* 0: never the packed-weight 256-row prefill
                                      tile; 1: wherever it applies; 2: the same
                                      with two waves along M (tuning) */
};
#define AWQ_OPT_AUTO (-1)          /* the planner's own choice */

/* AWQ_ABI_VERSION of the built library. */
int awq_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* awq_status_string(int status);

/* Sets a planner override, process-wide, for every later call from any
 * thread (a relaxed atomic store; calls already planned are unaffected).
 * value is AWQ_OPT_AUTO or one of the values listed with the option;
 * anything else, or an unknown option, is AWQ_ERROR_INVALID_VALUE and
 * changes nothing.  Each override starts from an environment variable read
 * once, on the library's first planning call: AWQ_FORCE_PATH (decode |
 * prefill | generic; any other text makes every awq_gemm and awq_gemm_plan
 * call fail with AWQ_ERROR_INVALID_VALUE until the option is set),
 * AWQ_DECODE_STEPS, AWQ_DECODE_GATHER_MAX_M, AWQ_PREFILL_BM,
 * AWQ_PREFILL_BN, AWQ_PREFILL_SPLITS, AWQ_DECODE_WAVES, AWQ_PREFILL_PACKED
 * (numbers; unusable ones are ignored).
 * No call reads the environment after that.  Host only. */
int awq_set_option(int option, int64_t value);

/* Writes the current value of an override (AWQ_OPT_AUTO when none) to
 * *value.  Unknown option or NULL value: AWQ_ERROR_INVALID_VALUE. */
int awq_get_option(int option, int64_t* value);

/* Bytes of workspace awq_gemm needs for this problem whatever the pointers'
 * alignment and whichever kernel family runs it (also one forced through
 * AWQ_OPT_FORCE_PATH): the larger of the split-K decode and split-K prefill
 * needs.  0 means none.  Returns 0 for invalid shapes (awq_gemm then reports
 * the error). */
size_t awq_gemm_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* Host-only planning, no HIP call and no dereference of x, qweight or scales
 * (only their addresses' alignment is inspected; NULL counts as aligned).
 * Writes the kernel family awq_gemm would run to *path and its workspace need
 * to *workspace_bytes (either may be NULL).  AWQ_OPT_FORCE_PATH
 * (awq_set_option) overrides the choice for testing; a forced family that
 * cannot run the problem yields AWQ_ERROR_INVALID_VALUE. */
int awq_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t group_size,
                  const void* x, const void* qweight, const void* scales, int* path,
                  size_t* workspace_bytes);

/* The WQLinear forward (page "Predibase Lorax AWQ WQLinear", Description,
 * forward steps 1-3), with the bias addition fused into the kernel epilogue:
 * y = float16_RNE(fp32 accumulation of x . W + bias).
 *
 * workspace: device memory of at least awq_gemm_workspace_size(...) bytes, or
 * NULL when that is 0.  It must be zero-filled once before its first use; the
 * kernels leave it re-usable (all counters back at zero) on exit, so the same
 * buffer serves later calls on the same stream.  Two calls that may run
 * concurrently (different streams) must not share a workspace.  A HIP graph
 * that captured a call keeps its workspace pointer: the buffer must stay
 * allocated (and unused by anything else) for as long as the graph may be
 * replayed.  A split prefill call, and a split decode call of more than
 * four rows or of so many splits x rows x columns that the atomic exchange
 * would issue 380K or more atomics, enqueue two kernels on `stream` (the
 * second sums the fp32 split partials in split order); every other call
 * enqueues one.
 * M == 0 is a no-op that returns AWQ_SUCCESS (x and y may then be NULL). */
int awq_gemm(const void* x, const void* qweight, const void* qzeros,
             const void* scales, const void* bias, void* y,
             int64_t M, int64_t K, int64_t N, int64_t group_size,
             void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): awq_gemm
 * without a workspace argument.  The split-K workspace is the library's own
 * file-scope device array of AWQ_NOALLOC_SCRATCH_BYTES (16 MiB), one copy per
 * device, held from the library's first use on that device until the
 * process ends; no call allocates or frees anything.  Same arguments,
 * kernels, results (bit for bit), errors and stream behaviour as awq_gemm,
 * with two exceptions: a batch of 17-32 rows whose decode plan needs more
 * workspace than the scratch holds runs awq_gemm's prefill kernel instead
 * (same tolerance, other rounding), and AWQ_ERROR_SCRATCH when the plan
 * still needs more workspace than the scratch holds (decode batches at the
 * shapes this library targets fit; large split prefill problems may not).
 * The first call on a device looks
 * up the array's address on that device (hipGetSymbolAddress) and enqueues
 * a small fill kernel on `stream` that zeroes the exchange counters (inside
 * a graph capture that kernel is captured too); every exchange leaves them
 * zero again.  All calls on one device share the one array: calls that may
 * run concurrently on that device (different streams, or graphs replayed
 * concurrently) race and must not overlap. */
#define AWQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int awq_gemm_noalloc(const void* x, const void* qweight, const void* qzeros,
                     const void* scales, const void* bias, void* y,
                     int64_t M, int64_t K, int64_t N, int64_t group_size, void* stream);

/* The dequantised weight on its own: w[K, N] float16 with
 * w[k, n] = float16_RNE((q[k, n] - z[k / g, n]) * s[k / g, n]), bit-exact
 * (the page's "per-group dequantization", Description). */
int awq_dequant(const void* qweight, const void* qzeros, const void* scales,
                void* w, int64_t K, int64_t N, int64_t group_size, void* stream);

/* The unquantised float16 linear, as a baseline for the W4A16 decode: the
 * FastLinear of the page "Predibase Lorax Linear Layer Factory"
 * (Description), F.linear(x, w, bias):
 *   y[m, n] = float16_RNE(fp32 sum_k x[m, k] * w[n, k] + bias[n]).
 * Its ROCm variant sends single-token products at K = 8192, N = 1280 or
 * 7168 to a custom skinny kernel; this one covers 1 <= M <= 4.
 *
 * x: float16 (M, K) row-major, 16-byte aligned.  w: float16 (N, K)
 * row-major (out_features x in_features), 16-byte aligned.  bias: float16
 * (N) or NULL.  y: float16 (M, N), written.  All device pointers owned by
 * the caller; no workspace; deterministic.  K % 8 == 0 and M * K <= 65536
 * (x is staged in LDS), else AWQ_ERROR_SHAPE; M > 4 is AWQ_ERROR_SHAPE;
 * M == 0 is a no-op.  Enqueued on `stream`, nothing synchronises. */
int awq_dense_gemv(const void* x, const void* w, const void* bias, void* y,
                   int64_t M, int64_t K, int64_t N, void* stream);

/* ------------------------------------------------------------------------
 * Row-to-group map (g_idx).  The page "Predibase Lorax Linear Layer Factory"
 * (Description, the get_linear bullets) lists g_idx among the components of
 * a GPTQ-quantised weight and says nothing more.  This library reads it as
 * the per-row generalisation of the contiguous groups above: g_idx is int32
 * (K) and input row k takes zero row and scale row g_idx[k],
 *
 *     W[k, n] = float16_RNE((q[k, n] - z[g_idx[k], n]) * s[g_idx[k], n]),
 *
 * with qweight/qzeros packed as above, qzeros (G, N/8) and scales (G, N),
 * G = num_groups >= 1.  g_idx[k] = k / g is the contiguous case.
 *
 * Two routes.  Directly: awq_dequant_gidx and awq_gemm_gidx look the group
 * up per row (the latter in the general kernel: correct, slow).  Fast: at
 * load time, awq_gidx_layout (host) sorts the rows by group and cuts them
 * into blocks that each lie in one group, and awq_gather_rows (device)
 * builds the sorted weight and each block's zero and scale rows; the result
 * is an ordinary grouped weight, and awq_gemm_sorted runs it on the grouped
 * kernels with x's columns brought into the same order.
 * ------------------------------------------------------------------------ */

/* w[K, N] float16 dequantised under a row-to-group map, bit-exact.
 * g_idx: DEVICE int32 (K), 4-byte aligned.  The map lives in device memory,
 * so its entries are not checked on the host: an entry outside
 * [0, num_groups) is read as zero point 0 and scale 0 (that row of w is
 * zero); no access goes outside the operands.  Other arguments, errors and
 * stream behaviour as awq_dequant; num_groups <= 0 is AWQ_ERROR_INVALID_VALUE. */
int awq_dequant_gidx(const void* qweight, const void* qzeros, const void* scales,
                     const void* g_idx, void* w, int64_t K, int64_t N, int64_t num_groups,
                     void* stream);

/* y[M, N] = float16_RNE(fp32 accumulation of x . W + bias) under any
 * row-to-group map (W as above), looking the group up per row in the
 * general kernel (plain fp32 FMA): the direct form of the definition, slow;
 * awq_gemm_sorted is the fast route for every map.  g_idx as in
 * awq_dequant_gidx.  No workspace.  Other arguments, errors and stream
 * behaviour as awq_gemm. */
int awq_gemm_gidx(const void* x, const void* qweight, const void* qzeros, const void* scales,
                  const void* g_idx, const void* bias, void* y, int64_t M, int64_t K, int64_t N,
                  int64_t num_groups, void* stream);

/* Host-only, no HIP call.  Sorted layout of a row-to-group map.
 * g_idx: HOST int32 (K), entries in [0, num_groups).  The rows are sorted
 * stably by group (ties in increasing row order), then cut into blocks:
 *   - when every group holds exactly K / num_groups rows and that count is a
 *     power of two >= 32 (activation order), one block per group, no rows
 *     added: *rows = K, *block_rows = K / num_groups, *blocks = num_groups;
 *   - otherwise blocks of 32 rows, each group's last block padded with null
 *     rows, and one block of null rows appended when the count is odd (with
 *     the last group), so that *rows is a multiple of 64:
 *     *block_rows = 32, *rows = 32 * *blocks.
 * perm (HOST int32, *rows entries): the input row placed j-th, or -1 for a
 * null row.  block_group (HOST int32, *blocks entries): the map's group of
 * each block.  Call with perm and block_group NULL to get the sizes; with
 * both non-NULL, capacities (entries) below *rows / *blocks give
 * AWQ_ERROR_SHAPE (sizes still written).  rows, block_rows and blocks must be
 * non-NULL.  An entry outside [0, num_groups), K <= 0 or num_groups <= 0 is
 * AWQ_ERROR_INVALID_VALUE (as is a failed host allocation of K indices). */
int awq_gidx_layout(const int32_t* g_idx, int64_t K, int64_t num_groups, int32_t* perm,
                    int64_t perm_capacity, int32_t* block_group, int64_t block_capacity,
                    int64_t* rows, int64_t* block_rows, int64_t* blocks);

/* Device row gather: dst row j = src row idx[j] for j < dst_rows, rows of
 * row_bytes bytes (row_bytes % 4 == 0, else AWQ_ERROR_SHAPE); an index
 * outside [0, src_rows) writes a row of zeros.  src, dst (must not overlap)
 * and idx (DEVICE int32, dst_rows entries) 4-byte aligned.  Builds a sorted
 * weight from awq_gidx_layout's output: qweight_sorted = rows of qweight by
 * perm (row_bytes = N / 2), qzeros_sorted and scales_sorted = rows of qzeros
 * and scales by block_group (row_bytes N / 2 and 2 N).  Enqueued on
 * `stream`; a load-time step. */
int awq_gather_rows(const void* src, int64_t src_rows, const void* idx, void* dst,
                    int64_t dst_rows, int64_t row_bytes, void* stream);

/* Workspace bytes of awq_gemm_sorted: the awq_gemm workspace of the sorted
 * problem (M, rows, N, block_rows), at least its fixed zero-filled regions,
 * then M x rows float16 for x with its columns reordered.  0 for M == 0 or
 * invalid shapes. */
size_t awq_gemm_sorted_workspace_size(int64_t M, int64_t rows, int64_t N, int64_t block_rows);

/* Forward of a sorted weight:
 *   y = float16_RNE(fp32 accumulation of x[:, perm] . W_sorted + bias),
 * x float16 (M, K_in); perm DEVICE int32 (rows), 4-byte aligned, an entry
 * outside [0, K_in) reading x as 0; W_sorted the grouped weight (group size
 * block_rows) of qweight_sorted (rows, N/8), qzeros_sorted (rows/block_rows,
 * N/8) and scales_sorted (rows/block_rows, N).  With those built by
 * awq_gidx_layout and awq_gather_rows this equals x . W (+ bias) for the
 * original (qweight, qzeros, scales, g_idx): the same products summed in
 * another order, null rows adding exact zeros.  workspace: at least
 * awq_gemm_sorted_workspace_size(...) bytes, 256-byte aligned, zero-filled
 * once like awq_gemm's (the same buffer may serve both); the reordered x is
 * written into it, so concurrent calls must not share it.  One or two
 * launches on `stream` (small batches gather x inside the decode kernel).
 * Other arguments, errors and stream behaviour as awq_gemm with K = rows and
 * group_size = block_rows. */
int awq_gemm_sorted(const void* x, const void* perm, const void* qweight_sorted,
                    const void* qzeros_sorted, const void* scales_sorted, const void* bias,
                    void* y, int64_t M, int64_t K_in, int64_t rows, int64_t N, int64_t block_rows,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* AWQ_MI355X_AWQ_H_ */
