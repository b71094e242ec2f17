// C-ABI entry points (include/awq.h): host validation, planning, launch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "awq.h"
#include "awq_device.h"
#include "awq_plan.h"

using awq::Plan;
using awq::Problem;

extern "C" {

int awq_abi_version(void) { return AWQ_ABI_VERSION; }

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_SUCCESS: return "success";
    case AWQ_ERROR_INVALID_VALUE:
      return "invalid value (NULL pointer, negative or zero size, bad group_size, "
             "or a kernel path that cannot run this problem)";
    case AWQ_ERROR_SHAPE:
      return "shape error (out_features % 8 != 0, in_features % group_size != 0, "
             "or an operand with 2^31 or more elements)";
    case AWQ_ERROR_MISALIGNED: return "pointer not aligned to its element size";
    case AWQ_ERROR_WORKSPACE: return "workspace missing or smaller than awq_gemm_workspace_size";
    case AWQ_ERROR_HIP: return "HIP launch error";
    case AWQ_ERROR_SCRATCH:
      return "problem needs more split-K workspace than awq_gemm_noalloc's fixed scratch "
             "(AWQ_NOALLOC_SCRATCH_BYTES); use awq_gemm with a workspace";
    default: return "unknown status";
  }
}

int awq_set_option(int option, int64_t value) { return awq::set_option(option, value); }

int awq_get_option(int option, int64_t* value) { return awq::get_option(option, value); }

size_t awq_gemm_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  return awq::gemm_workspace_size(M, K, N, group_size);
}

int awq_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t group_size, const void* x,
                  const void* qweight, const void* scales, int* path,
                  size_t* workspace_bytes) {
  Problem p;
  int st = awq::validate_shape(M, K, N, group_size, &p);
  if (st != AWQ_SUCCESS) return st;
  const int force = awq::forced_path();
  if (force < 0) return AWQ_ERROR_INVALID_VALUE;
  Plan pl;
  const awq::Alignment al{awq::aligned(x, 16), awq::aligned(scales, 16),
                          awq::aligned(qweight, 16)};
  st = awq::make_plan(p, al, force, &pl);
  if (st != AWQ_SUCCESS) return st;
  if (path) *path = pl.path;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  return AWQ_SUCCESS;
}

}  // extern "C"

namespace {

// Plans and launches the grouped forward for a validated problem p (x, y
// non-NULL and M > 0).  Shared by awq_gemm and awq_gemm_sorted.  With a
// column order perm (sorted weight), x (M x Kx) is read as x[:, perm] with
// 0 where perm is outside [0, Kx): the LDS decode kernel gathers it itself
// (small batches); every other kernel reads a copy reordered into xp first
// (M x K float16, 16-byte aligned).
// The plan awq_gemm follows for problem p with these operand addresses (a
// reordered x is 16-byte aligned wherever it is read from).  ws_limit: the
// workspace the caller can offer at most (awq_gemm_noalloc's scratch); a
// two-block decode plan (17-32 rows) that needs more falls back to the
// prefill kernel, whose split partials are fewer.
int plan_gemm(const Problem& p, const void* x, const void* qweight, const void* scales,
              bool reordered_x, size_t ws_limit, Plan* pl) {
  const int force = awq::forced_path();
  if (force < 0) return AWQ_ERROR_INVALID_VALUE;
  const awq::Alignment al{reordered_x ? true : awq::aligned(x, 16), awq::aligned(scales, 16),
                          awq::aligned(qweight, 16)};
  const int st = awq::make_plan(p, al, force, pl);
  if (st != AWQ_SUCCESS || force != 0 || pl->ws_bytes <= ws_limit ||
      pl->path != AWQ_PATH_DECODE || p.M <= awq::kDecodeBlockM || !awq::prefill_supported(p, al))
    return st;
  return awq::make_plan(p, al, AWQ_PATH_PREFILL, pl);
}

int run_gemm(const Problem& p, const void* x, const void* qweight, const void* qzeros,
             const void* scales, const void* bias, void* y, void* workspace,
             size_t workspace_bytes, const int32_t* perm, int64_t Kx, _Float16* xp,
             size_t ws_limit, hipStream_t s) {
  Plan pl;
  const int st = plan_gemm(p, x, qweight, scales, perm != nullptr, ws_limit, &pl);
  if (st != AWQ_SUCCESS) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes) return AWQ_ERROR_WORKSPACE;
    if (!awq::aligned(workspace, 16)) return AWQ_ERROR_MISALIGNED;
  }
  const bool fused_gather = perm && pl.path == AWQ_PATH_DECODE && pl.decode_lds &&
                            pl.steps <= 4 && p.M <= awq::decode_gather_max_m();
  if (perm && !fused_gather) {
    const hipError_t e = awq::launch_gather_cols(static_cast<const _Float16*>(x), perm, xp,
                                                 static_cast<int>(p.M), static_cast<int>(Kx),
                                                 static_cast<int>(p.K), s);
    if (e != hipSuccess) return AWQ_ERROR_HIP;
    x = xp;
  }

  const auto* xh = static_cast<const _Float16*>(x);
  const auto* qw = static_cast<const uint32_t*>(qweight);
  const auto* qz = static_cast<const uint32_t*>(qzeros);
  const auto* sc = static_cast<const _Float16*>(scales);
  const auto* bh = static_cast<const _Float16*>(bias);
  auto* yh = static_cast<_Float16*>(y);
  const int iM = static_cast<int>(p.M), iK = static_cast<int>(p.K), iN = static_cast<int>(p.N);
  const int ig = static_cast<int>(p.g), iG = static_cast<int>(p.G);

  hipError_t e = hipErrorInvalidValue;
  switch (pl.path) {
    case AWQ_PATH_DECODE:
      e = awq::launch_decode(xh, qw, qz, sc, bh, yh, iM, iK, iN, ig, iG, pl.steps, pl.splits,
                             pl.n_tiles, pl.decode_lds, pl.decode_waves, pl.decode_atomic,
                             workspace,
                             fused_gather ? perm : nullptr,
                             fused_gather ? static_cast<int>(Kx) : iK, s);
      break;
    case AWQ_PATH_PREFILL:
      if (pl.prefill_packed) {
        e = awq::launch_prefill_packed(xh, qw, qz, sc, bh, yh, iM, iK, iN, pl.group_shift,
                                       pl.prefill_bn, pl.packed_wm, pl.m_tiles, pl.n_tiles, s);
        break;
      }
      e = awq::launch_prefill(xh, qw, qz, sc, bh, yh, iM, iK, iN, pl.group_shift, pl.prefill_bm,
                              pl.prefill_bn, pl.m_tiles, pl.n_tiles, pl.splits, pl.steps,
                              workspace, s);
      break;
    case AWQ_PATH_GENERIC:
      e = awq::launch_generic(xh, qw, qz, sc, bh, yh, iM, iK, iN, ig, nullptr, iG, s);
      break;
    default:
      return AWQ_ERROR_INVALID_VALUE;
  }
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

// ---------------------------------------------------------------------------
// awq_gemm_noalloc: awq_gemm for callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc).  Its
// split-K workspace is this file-scope array, one copy per device, held
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the per-device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current.
constexpr size_t kScratchBytes = AWQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= awq::kAtomicRegionBytes,
              "the scratch holds at least the exchange's fixed region");
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  int status = AWQ_ERROR_HIP;
};
ScratchSlot g_scratch[kMaxDevices];

// Zeroes n16 16-byte words at p (the atomic exchange's accumulator region
// must start at zero; every exchange leaves it zero again).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch address on the device of stream s, set up on first use: the
// symbol's address with that device current, and a fill kernel on s that
// zeroes the fixed region before any exchange uses it.
int scratch_for_stream(hipStream_t s, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return AWQ_ERROR_HIP;
  int dev = cur;
  if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return AWQ_ERROR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return AWQ_ERROR_INVALID_VALUE;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr != nullptr) {
      const size_t n16 = awq::kAtomicRegionBytes / 16;
      hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, s,
                         static_cast<uint4*>(ptr), n16);
      if (hipGetLastError() == hipSuccess) {
        slot.ptr = ptr;
        slot.status = AWQ_SUCCESS;
      }
    }
    if (dev != cur) (void)hipSetDevice(cur);
  });
  if (slot.status != AWQ_SUCCESS) return slot.status;
  *out = slot.ptr;
  return AWQ_SUCCESS;
}

}  // namespace

extern "C" {

int awq_gemm_noalloc(const void* x, const void* qweight, const void* qzeros, const void* scales,
                     const void* bias, void* y, int64_t M, int64_t K, int64_t N,
                     int64_t group_size, void* stream) {
  Problem p;
  int st = awq::validate_shape(M, K, N, group_size, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_gemm_pointers(x, qweight, qzeros, scales, bias, y, M);
  if (st != AWQ_SUCCESS) return st;
  if (M == 0) return AWQ_SUCCESS;
  Plan pl;
  st = plan_gemm(p, x, qweight, scales, false, kScratchBytes, &pl);
  if (st != AWQ_SUCCESS) return st;
  if (pl.ws_bytes > kScratchBytes) return AWQ_ERROR_SCRATCH;
  const auto s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_for_stream(s, &ws);
  if (st != AWQ_SUCCESS) return st;
  return run_gemm(p, x, qweight, qzeros, scales, bias, y, ws, kScratchBytes, nullptr, K,
                  nullptr, kScratchBytes, s);
}

int awq_gemm(const void* x, const void* qweight, const void* qzeros, const void* scales,
             const void* bias, void* y, int64_t M, int64_t K, int64_t N, int64_t group_size,
             void* workspace, size_t workspace_bytes, void* stream) {
  Problem p;
  int st = awq::validate_shape(M, K, N, group_size, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_gemm_pointers(x, qweight, qzeros, scales, bias, y, M);
  if (st != AWQ_SUCCESS) return st;
  if (M == 0) return AWQ_SUCCESS;
  return run_gemm(p, x, qweight, qzeros, scales, bias, y, workspace, workspace_bytes, nullptr,
                  K, nullptr, SIZE_MAX, static_cast<hipStream_t>(stream));
}

int awq_dense_gemv(const void* x, const void* w, const void* bias, void* y, int64_t M, int64_t K,
                   int64_t N, void* stream) {
  const int st = awq::validate_dense(x, w, bias, y, M, K, N);
  if (st != AWQ_SUCCESS) return st;
  if (M == 0) return AWQ_SUCCESS;
  const hipError_t e = awq::launch_dense_gemv(
      static_cast<const _Float16*>(x), static_cast<const _Float16*>(w),
      static_cast<const _Float16*>(bias), static_cast<_Float16*>(y), static_cast<int>(M),
      static_cast<int>(K), static_cast<int>(N), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

int awq_dequant(const void* qweight, const void* qzeros, const void* scales, void* w,
                int64_t K, int64_t N, int64_t group_size, void* stream) {
  Problem p;
  int st = awq::validate_shape(0, K, N, group_size, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_dequant_pointers(qweight, qzeros, scales, w);
  if (st != AWQ_SUCCESS) return st;
  hipError_t e = awq::launch_dequant(static_cast<const uint32_t*>(qweight),
                                     static_cast<const uint32_t*>(qzeros),
                                     static_cast<const _Float16*>(scales),
                                     static_cast<_Float16*>(w), static_cast<int>(p.K),
                                     static_cast<int>(p.N), static_cast<int>(p.g), nullptr,
                                     static_cast<int>(p.G), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

int awq_dequant_gidx(const void* qweight, const void* qzeros, const void* scales,
                     const void* g_idx, void* w, int64_t K, int64_t N, int64_t num_groups,
                     void* stream) {
  Problem p;
  int st = awq::validate_gidx_shape(0, K, N, num_groups, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_dequant_pointers(qweight, qzeros, scales, w);
  if (st != AWQ_SUCCESS) return st;
  if (!g_idx) return AWQ_ERROR_INVALID_VALUE;
  if (!awq::aligned(g_idx, 4)) return AWQ_ERROR_MISALIGNED;
  const hipError_t e = awq::launch_dequant(
      static_cast<const uint32_t*>(qweight), static_cast<const uint32_t*>(qzeros),
      static_cast<const _Float16*>(scales), static_cast<_Float16*>(w), static_cast<int>(p.K),
      static_cast<int>(p.N), 1, static_cast<const int32_t*>(g_idx), static_cast<int>(p.G),
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

int awq_gemm_gidx(const void* x, const void* qweight, const void* qzeros, const void* scales,
                  const void* g_idx, const void* bias, void* y, int64_t M, int64_t K, int64_t N,
                  int64_t num_groups, void* stream) {
  Problem p;
  int st = awq::validate_gidx_shape(M, K, N, num_groups, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_gemm_pointers(x, qweight, qzeros, scales, bias, y, M);
  if (st != AWQ_SUCCESS) return st;
  if (!g_idx) return AWQ_ERROR_INVALID_VALUE;
  if (!awq::aligned(g_idx, 4)) return AWQ_ERROR_MISALIGNED;
  if (M == 0) return AWQ_SUCCESS;
  const hipError_t e = awq::launch_generic(
      static_cast<const _Float16*>(x), static_cast<const uint32_t*>(qweight),
      static_cast<const uint32_t*>(qzeros), static_cast<const _Float16*>(scales),
      static_cast<const _Float16*>(bias), static_cast<_Float16*>(y), static_cast<int>(p.M),
      static_cast<int>(p.K), static_cast<int>(p.N), 1, static_cast<const int32_t*>(g_idx),
      static_cast<int>(p.G), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

int awq_gidx_layout(const int32_t* g_idx, int64_t K, int64_t num_groups, int32_t* perm,
                    int64_t perm_capacity, int32_t* block_group, int64_t block_capacity,
                    int64_t* rows, int64_t* block_rows, int64_t* blocks) {
  return awq::gidx_layout(g_idx, K, num_groups, perm, perm_capacity, block_group,
                          block_capacity, rows, block_rows, blocks);
}

int awq_gather_rows(const void* src, int64_t src_rows, const void* idx, void* dst,
                    int64_t dst_rows, int64_t row_bytes, void* stream) {
  if (!src || !idx || !dst || src_rows <= 0 || dst_rows <= 0 || row_bytes <= 0)
    return AWQ_ERROR_INVALID_VALUE;
  if (row_bytes % 4 != 0) return AWQ_ERROR_SHAPE;
  const int64_t lim = (int64_t{1} << 31) - 1;
  const int64_t words = row_bytes / 4;
  if (src_rows > lim || dst_rows > lim || src_rows * words > lim || dst_rows * words > lim)
    return AWQ_ERROR_SHAPE;
  if (!awq::aligned(src, 4) || !awq::aligned(idx, 4) || !awq::aligned(dst, 4))
    return AWQ_ERROR_MISALIGNED;
  const hipError_t e = awq::launch_gather_rows(
      static_cast<const uint32_t*>(src), static_cast<int>(src_rows),
      static_cast<const int32_t*>(idx), static_cast<uint32_t*>(dst), static_cast<int>(dst_rows),
      static_cast<int>(words), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

size_t awq_gemm_sorted_workspace_size(int64_t M, int64_t rows, int64_t N, int64_t block_rows) {
  return awq::sorted_workspace_size(M, rows, N, block_rows);
}

int awq_gemm_sorted(const void* x, const void* perm, const void* qweight_sorted,
                    const void* qzeros_sorted, const void* scales_sorted, const void* bias,
                    void* y, int64_t M, int64_t K_in, int64_t rows, int64_t N, int64_t block_rows,
                    void* workspace, size_t workspace_bytes, void* stream) {
  Problem p;
  int st = awq::validate_shape(M, rows, N, block_rows, &p);
  if (st != AWQ_SUCCESS) return st;
  st = awq::validate_gemm_pointers(x, qweight_sorted, qzeros_sorted, scales_sorted, bias, y, M);
  if (st != AWQ_SUCCESS) return st;
  if (!perm || K_in <= 0) return AWQ_ERROR_INVALID_VALUE;
  if (K_in > (int64_t{1} << 31) - 1 || M * K_in > (int64_t{1} << 31) - 1) return AWQ_ERROR_SHAPE;
  if (!awq::aligned(perm, 4)) return AWQ_ERROR_MISALIGNED;
  if (M == 0) return AWQ_SUCCESS;
  const size_t need = awq::sorted_workspace_size(M, rows, N, block_rows);
  if (!workspace || workspace_bytes < need) return AWQ_ERROR_WORKSPACE;
  if (!awq::aligned(workspace, 256)) return AWQ_ERROR_MISALIGNED;
  const size_t xoff = awq::sorted_x_offset(M, rows, N, block_rows);
  auto* xp = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + xoff);
  return run_gemm(p, x, qweight_sorted, qzeros_sorted, scales_sorted, bias, y, workspace, xoff,
                  static_cast<const int32_t*>(perm), K_in, xp, SIZE_MAX,
                  static_cast<hipStream_t>(stream));
}

}  // extern "C"
