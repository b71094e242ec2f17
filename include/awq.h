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

#define AWQ_ABI_VERSION 3

/* Status codes returned by every entry point. */
enum awq_status {
  AWQ_SUCCESS = 0,
  AWQ_ERROR_INVALID_VALUE = 1, /* NULL required pointer, M < 0, K <= 0, N <= 0,
                                  group_size == 0 or < -1, unknown path request */
  AWQ_ERROR_SHAPE = 2,         /* N % 8 != 0, K % group_size != 0 (page checks),
                                  or an operand with 2^31 or more elements */
  AWQ_ERROR_MISALIGNED = 3,    /* a pointer not aligned to its element size */
  AWQ_ERROR_WORKSPACE = 4,     /* workspace smaller than awq_gemm_workspace_size */
  AWQ_ERROR_HIP = 5            /* a HIP launch reported an error */
};

/* Kernel families that awq_gemm can run (see awq_gemm_plan). */
enum awq_path {
  AWQ_PATH_DECODE = 1,  /* split-K MFMA skinny GEMM, M <= 16 */
  AWQ_PATH_PREFILL = 2, /* LDS-tiled MFMA GEMM with dequantisation into LDS */
  AWQ_PATH_GENERIC = 3  /* any legal shape or alignment; slow */
};

/* AWQ_ABI_VERSION of the built library. */
int awq_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* awq_status_string(int status);

/* Bytes of workspace awq_gemm needs for this problem whatever the pointers'
 * alignment and whichever kernel family runs it (also one forced through
 * AWQ_FORCE_PATH): the larger of the split-K decode and split-K prefill
 * needs.  0 means none.  Returns 0 for invalid shapes (awq_gemm then reports
 * the error). */
size_t awq_gemm_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* Host-only planning, no HIP call and no dereference of x, qweight or scales
 * (only their addresses' alignment is inspected; NULL counts as aligned).
 * Writes the kernel family awq_gemm would run to *path and its workspace need
 * to *workspace_bytes (either may be NULL).  The environment variable
 * AWQ_FORCE_PATH = decode | prefill | generic overrides the choice for
 * testing; a forced family that cannot run the problem yields
 * AWQ_ERROR_INVALID_VALUE. */
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
 * concurrently (different streams) must not share a workspace.
 * M == 0 is a no-op that returns AWQ_SUCCESS (x and y may then be NULL). */
int awq_gemm(const void* x, const void* qweight, const void* qzeros,
             const void* scales, const void* bias, void* y,
             int64_t M, int64_t K, int64_t N, int64_t group_size,
             void* workspace, size_t workspace_bytes, void* stream);

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
 * Two routes.  Any map: awq_dequant_gidx, awq_gemm_gidx (general kernel,
 * slow).  A map that gives every group the same number of rows (activation
 * order, where the rows of each group are scattered over the input): sort
 * the rows by group once at load time (awq_gidx_order on the host, then
 * awq_permute_rows on the device), after which awq_gemm_act_order runs the
 * fast grouped kernels.
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
 * row-to-group map (W as above).  The general kernel (plain fp32 FMA): a
 * correctness route for maps with groups of unequal size; activation-order
 * maps should take awq_gemm_act_order.  g_idx as in awq_dequant_gidx.  No
 * workspace.  Other arguments, errors and stream behaviour as awq_gemm. */
int awq_gemm_gidx(const void* x, const void* qweight, const void* qzeros, const void* scales,
                  const void* g_idx, const void* bias, void* y, int64_t M, int64_t K, int64_t N,
                  int64_t num_groups, void* stream);

/* Host-only, no HIP call.  Stable order of the K input rows by group:
 * perm[j] (HOST int32 (K), written) is the row placed j-th, so the rows of
 * group 0 come first in increasing row order, then those of group 1, ...
 * g_idx: HOST int32 (K).  *group_size (may be NULL) receives K / num_groups
 * when every group holds exactly that many rows (the reordered weight is then
 * a grouped weight of that group size), else 0.  An entry outside
 * [0, num_groups), NULL pointers, K <= 0 or num_groups <= 0 give
 * AWQ_ERROR_INVALID_VALUE and leave perm untouched (as does a failed host
 * allocation of K indices). */
int awq_gidx_order(const int32_t* g_idx, int64_t K, int64_t num_groups, int32_t* perm,
                   int64_t* group_size);

/* Reorders the rows of a packed weight: qweight_out[j, :] = qweight[perm[j], :]
 * for int32 (K, N/8) matrices (DEVICE pointers, 4-byte aligned; must not
 * overlap).  perm: DEVICE int32 (K), e.g. awq_gidx_order's output copied to
 * the device; an entry outside [0, K) writes a row of zeros.  N % 8 != 0 is
 * AWQ_ERROR_SHAPE.  Enqueued on `stream`; a load-time step. */
int awq_permute_rows(const void* qweight, const void* perm, void* qweight_out, int64_t K,
                     int64_t N, void* stream);

/* Workspace bytes of awq_gemm_act_order: the awq_gemm workspace of the same
 * problem (at least its fixed zero-filled regions), then M x K float16 for x
 * with its columns reordered.  0 for M == 0 or invalid shapes. */
size_t awq_gemm_act_order_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* Forward of an activation-order weight after the load-time reorder:
 *   y = float16_RNE(fp32 accumulation of x[:, perm] . W_sorted + bias),
 * W_sorted the grouped weight (group_size) of qweight_sorted, qzeros and
 * scales.  With perm and group_size from awq_gidx_order and qweight_sorted =
 * awq_permute_rows(qweight, perm), this equals x . W (+ bias) for the
 * original (qweight, g_idx): the same products summed in another order.
 * perm: DEVICE int32 (K), 4-byte aligned (entries outside [0, K) read x as 0).
 * workspace: at least awq_gemm_act_order_workspace_size(...) bytes, 256-byte
 * aligned, zero-filled once like awq_gemm's (the same buffer may serve both);
 * the reordered x is written into it, so concurrent calls must not share it.
 * Two launches on `stream`: the column reorder of x, then the awq_gemm kernel
 * family for the problem.  Other arguments, errors and stream behaviour as
 * awq_gemm. */
int awq_gemm_act_order(const void* x, const void* perm, const void* qweight_sorted,
                       const void* qzeros, const void* scales, const void* bias, void* y,
                       int64_t M, int64_t K, int64_t N, int64_t group_size, void* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* AWQ_MI355X_AWQ_H_ */
