// Device helpers shared by the gfx950 kernels: vector types, nibble unpacking
// into packed float16 pairs, and the launch entry points of each kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// float16 1024.0 is 0x6400; its ulp is 1, so OR-ing a nibble q into the low
// mantissa bits yields exactly 1024 + q.  Two such values sit in one 32-bit
// register as a packed pair.
constexpr uint32_t kMagicPair = 0x64006400u;
constexpr uint32_t kNibblePairMask = 0x000F000Fu;

// Byte shuffles that place, for two words a (low half) and b (high half),
// bytes {a.b0, a.b1, b.b0, b.b1} (lo) or {a.b2, a.b3, b.b2, b.b3} (hi) in one
// register.  Nibble j < 4 of a and b then sits at bit 4j of each 16-bit half
// of `lo`, nibble j >= 4 at bit 4(j-4) of each half of `hi`.
__device__ __forceinline__ uint32_t pair_bytes_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_bytes_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// (v & mask) | bits in one VALU instruction.  The compiler splits this
// pattern into two when the operands are constants; gfx9 encodings allow at
// most one scalar operand, so the mask travels in a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(v), "v"(mask), "s"(bits));
  return d;
}

// (1024 + nibble, 1024 + nibble) float16 pair from a pair_bytes_* register.
__device__ __forceinline__ uint32_t magic_pair(uint32_t paired, int shift) {
  return and_or(paired >> shift, kNibblePairMask, kMagicPair);
}

// Buffer resource over [base, base + bytes): loads at offsets outside that
// range return zero instead of touching memory, so tails need no branches.
// Offsets are in bytes and must stay below 2^32.
// Loads a kernel argument into SGPRs now.  The compiler otherwise defers
// loads of arguments used only in an epilogue until then, where the
// kernel-argument fetch (~1 us) lands on the critical path; an asm that
// claims to modify the value also keeps it from being reloaded later.
template <class T>
__device__ __forceinline__ void pin_arg(T& v) {
  asm volatile("" : "+s"(v));
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset >= the range reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Branch-free "offset if valid, else out of range": valid offsets are below
// 2^31 (operands stay under 1 GiB), so setting bit 31 moves an invalid lane
// past the end of every buffer.  A select written as a ternary may be turned
// into divergent branches, each issuing its own load; this cannot.
__device__ __forceinline__ uint32_t offset_or_oob(bool valid, uint32_t off) {
  return off | (static_cast<uint32_t>(!valid) << 31);
}
__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_load_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// (1024 + z_j) in both halves, for nibble j of zero word zw.
__device__ __forceinline__ uint32_t zero_pair(uint32_t zw, int j) {
  const uint32_t dup = (j < 4) ? pair_bytes_lo(zw, zw) : pair_bytes_hi(zw, zw);
  return magic_pair(dup, 4 * (j & 3));
}

}  // namespace awq

// Launchers implemented in the .hip files; called by awq_api.cpp.
namespace awq {
struct Problem;
struct Plan;
hipError_t launch_dequant(const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, _Float16* w, int K, int N, int g,
                          const int32_t* gidx, int G, hipStream_t stream);
hipError_t launch_generic(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, const _Float16* bias, _Float16* y,
                          int M, int K, int N, int g, const int32_t* gidx, int G,
                          hipStream_t stream);
// Row gather of a word matrix: dst[j] = src[idx[j]] (zeros out of range).
hipError_t launch_gather_rows(const uint32_t* src, int src_rows, const int32_t* idx,
                              uint32_t* dst, int dst_rows, int row_words, hipStream_t stream);
// Column reorder of x (M, Kin) into xp (M, Kout): xp[m, j] = x[m, perm[j]].
hipError_t launch_gather_cols(const _Float16* x, const int32_t* perm, _Float16* xp, int M,
                              int Kin, int Kout, hipStream_t stream);
hipError_t launch_decode(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                         const _Float16* scales, const _Float16* bias, _Float16* y,
                         int M, int K, int N, int g, int G, int steps, int splits,
                         int n_tiles, bool lds_variant, int waves, bool atomic,
                         void* workspace, const int32_t* perm, int Kx, hipStream_t stream);
hipError_t launch_prefill(const _Float16* x, const uint32_t* qweight, const uint32_t* qzeros,
                          const _Float16* scales, const _Float16* bias, _Float16* y,
                          int M, int K, int N, int group_shift, int bm, int bn,
                          int m_tiles, int n_tiles, int splits, int ksteps, void* workspace,
                          hipStream_t stream);
hipError_t launch_prefill_packed(const _Float16* x, const uint32_t* qweight,
                                 const uint32_t* qzeros, const _Float16* scales,
                                 const _Float16* bias, _Float16* y, int M, int K, int N,
                                 int group_shift, int bn, int wm, int m_tiles, int n_tiles,
                                 hipStream_t stream);
hipError_t launch_dense_gemv(const _Float16* x, const _Float16* w, const _Float16* bias,
                             _Float16* y, int M, int K, int N, hipStream_t stream);
}  // namespace awq
