// Drives the HIP-free validation and planning code over a grid of arguments,
// including every error path and extreme sizes, under ASan/UBSan.  Prints
// "plan_check ok" and exits 0 when every expectation holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "awq.h"
#include "awq_plan.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
              __LINE__, #cond);                                        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  using namespace awq;
  Problem p;
  EXPECT(validate_shape(4, 256, 128, 64, &p) == AWQ_SUCCESS);
  EXPECT(p.g == 64 && p.G == 4);
  EXPECT(validate_shape(4, 256, 128, -1, &p) == AWQ_SUCCESS && p.g == 256 && p.G == 1);
  EXPECT(validate_shape(-1, 256, 128, 64, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_shape(4, 0, 128, 64, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_shape(4, 256, 0, 64, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_shape(4, 256, 128, 0, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_shape(4, 256, 128, -7, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_shape(4, 256, 130, 64, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_shape(4, 256, 128, 48, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_shape(INT64_MAX, INT64_MAX, 8, -1, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_shape(1, INT64_MAX - 7, 8, -1, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_shape(1, (int64_t)1 << 40, (int64_t)1 << 40, -1, &p) == AWQ_ERROR_SHAPE);

  int x;
  EXPECT(validate_gemm_pointers(&x, &x, &x, &x, nullptr, &x, 1) == AWQ_SUCCESS);
  EXPECT(validate_gemm_pointers(nullptr, &x, &x, &x, nullptr, nullptr, 0) == AWQ_SUCCESS);
  EXPECT(validate_gemm_pointers(nullptr, &x, &x, &x, nullptr, &x, 1) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_gemm_pointers(&x, (char*)&x + 2, &x, &x, nullptr, &x, 1) ==
         AWQ_ERROR_MISALIGNED);
  EXPECT(validate_dequant_pointers(&x, &x, &x, nullptr) == AWQ_ERROR_INVALID_VALUE);

  // Every shape in a grid plans without overflow, and a plan's workspace
  // covers its split-K partials.
  const int64_t Ms[] = {0, 1, 2, 15, 16, 17, 255, 256, 4096};
  const int64_t Ks[] = {8, 32, 40, 96, 256, 4096, 8192, 14336};
  const int64_t Ns[] = {8, 24, 128, 1280, 7168, 12288};
  const int64_t gs[] = {-1, 1, 4, 8, 12, 32, 64, 96, 128};
  for (int64_t M : Ms)
    for (int64_t K : Ks)
      for (int64_t N : Ns)
        for (int64_t g : gs) {
          if (validate_shape(M, K, N, g, &p) != AWQ_SUCCESS) continue;
          for (int force = 0; force <= 3; ++force) {
            for (int al = 0; al < 8; ++al) {
              Plan pl;
              const Alignment a{(al & 1) != 0, (al & 2) != 0, (al & 4) != 0};
              const int st = make_plan(p, a, force, &pl);
              if (st != AWQ_SUCCESS) {
                EXPECT(force != 0 && force != AWQ_PATH_GENERIC);
                continue;
              }
              if (pl.path == AWQ_PATH_DECODE) {
                EXPECT(M <= kDecodeMaxM);
                EXPECT(pl.splits >= 1 && pl.n_tiles * kDecodeCols >= N);
                EXPECT(pl.decode_lds == (N % 32 == 0));
                EXPECT(!pl.decode_lds || a.qweight);
                EXPECT(pl.decode_waves == 4 || (pl.decode_lds && pl.decode_waves == 8));
                EXPECT(pl.decode_waves == 4 || pl.steps <= 4);
                const int waves_k = pl.decode_lds ? pl.decode_waves : 2;
                EXPECT((int64_t)pl.splits * waves_k * kDecodeRowsPerStep * pl.steps >= K);
                EXPECT((int64_t)(pl.splits - 1) * waves_k * kDecodeRowsPerStep * pl.steps < K);
                EXPECT(pl.splits <= kDecodeMaxSplits);
                if (pl.splits > 1)
                  EXPECT(pl.ws_bytes == kAtomicRegionBytes +
                                        (size_t)pl.splits * M * N * 4);
                else
                  EXPECT(pl.ws_bytes == 0);
              } else if (pl.path == AWQ_PATH_PREFILL) {
                EXPECT(pl.prefill_bm == 64 || pl.prefill_bm == 128 || pl.prefill_bm == kPrefillBM);
                EXPECT(pl.prefill_bn == kPrefillBN || pl.prefill_bm == kPrefillBM);
                EXPECT((int64_t)pl.m_tiles * pl.prefill_bm >= M);
                const int64_t nkt = (K + kPrefillBK - 1) / kPrefillBK;
                // The smallest of 64 / 128 / 256 rows covering M; for short K
                // (a 256-row plan that would split) also 128, or 64 for at
                // most 256 rows.
                const int def_bm = M <= 64 ? 64 : (M <= 128 ? 128 : 256);
                EXPECT(pl.prefill_bm == def_bm ||
                       (def_bm == 256 && nkt <= kPrefillShortKSteps &&
                        (pl.prefill_bm == 128 || (pl.prefill_bm == 64 && M <= 256))));
                EXPECT(pl.prefill_bn == kPrefillBN || pl.prefill_bn == kPrefillWideBN);
                EXPECT((int64_t)pl.n_tiles * pl.prefill_bn >= N);
                EXPECT((int64_t)(pl.n_tiles - 1) * pl.prefill_bn < N);
                const int64_t tiles = (int64_t)pl.m_tiles * pl.n_tiles;
                EXPECT(pl.splits >= 1 && pl.splits <= kPrefillMaxSplits);
                EXPECT((int64_t)pl.splits * pl.steps >= nkt);
                EXPECT((int64_t)(pl.splits - 1) * pl.steps < nkt);
                EXPECT(pl.splits == 1 || (tiles * pl.splits <= kPrefillTargetWGs &&
                                          pl.steps >= kPrefillMinSplitSteps));
                EXPECT((tiles > 0 && tiles < kPrefillTargetWGs) || pl.splits == 1);
                if (pl.splits > 1)
                  EXPECT(pl.ws_bytes == kAtomicRegionBytes +
                                        (size_t)pl.splits * M * N * 4);
                else
                  EXPECT(pl.ws_bytes == 0);
                EXPECT(p.G == 1 ? pl.group_shift == 31 : (int64_t{1} << pl.group_shift) == p.g);
              }
            }
          }
        }
  // Row-to-group maps: validation, the stable counting sort and its group
  // size report, bad entries, and the act-order workspace rule.
  EXPECT(validate_gidx_shape(4, 256, 128, 4, &p) == AWQ_SUCCESS && p.G == 4 && p.g == 0);
  EXPECT(validate_gidx_shape(4, 256, 128, 0, &p) == AWQ_ERROR_INVALID_VALUE);
  EXPECT(validate_gidx_shape(4, 256, 121, 4, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_gidx_shape(1, 8, 8, INT64_MAX, &p) == AWQ_ERROR_SHAPE);
  EXPECT(validate_gidx_shape(1, 8, (int64_t)1 << 20, (int64_t)1 << 12, &p) == AWQ_ERROR_SHAPE);
  {
    // Uneven map: blocks of 32 rows padded with -1, in group order.
    const int32_t gi[6] = {2, 0, 1, 0, 2, 1};
    int64_t rows = 0, brows = 0, nblk = 0;
    EXPECT(gidx_layout(gi, 6, 3, nullptr, 0, nullptr, 0, &rows, &brows, &nblk) == AWQ_SUCCESS);
    // Three blocks, and a fourth of null rows so that rows % 64 == 0.
    EXPECT(rows == 128 && brows == 32 && nblk == 4);
    std::vector<int32_t> perm(128, 7), blk(4, 7);
    EXPECT(gidx_layout(gi, 6, 3, perm.data(), 128, blk.data(), 4, &rows, &brows, &nblk) ==
           AWQ_SUCCESS);
    EXPECT(perm[0] == 1 && perm[1] == 3 && perm[2] == -1 && perm[31] == -1);
    EXPECT(perm[32] == 2 && perm[33] == 5 && perm[64] == 0 && perm[65] == 4 && perm[95] == -1);
    EXPECT(perm[96] == -1 && perm[127] == -1);
    EXPECT(blk[0] == 0 && blk[1] == 1 && blk[2] == 2 && blk[3] == 2);
    EXPECT(gidx_layout(gi, 6, 3, perm.data(), 127, blk.data(), 4, &rows, &brows, &nblk) ==
           AWQ_ERROR_SHAPE);
    EXPECT(gidx_layout(gi, 6, 3, perm.data(), 128, blk.data(), 3, &rows, &brows, &nblk) ==
           AWQ_ERROR_SHAPE);
    // Activation order with 32-row groups: whole groups, no padding.
    std::vector<int32_t> ao(128);
    for (int k = 0; k < 128; ++k) ao[k] = (k * 37) % 128 / 32;
    EXPECT(gidx_layout(ao.data(), 128, 4, perm.data(), 96, blk.data(), 3, &rows, &brows, &nblk) ==
           AWQ_ERROR_SHAPE);
    EXPECT(rows == 128 && brows == 32 && nblk == 4);
    std::vector<int32_t> perm2(128), blk2(4);
    EXPECT(gidx_layout(ao.data(), 128, 4, perm2.data(), 128, blk2.data(), 4, &rows, &brows,
                       &nblk) == AWQ_SUCCESS);
    for (int j = 0; j < 128; ++j) EXPECT(ao[perm2[j]] == j / 32);
    const int32_t bad[3] = {0, 3, 1};
    EXPECT(gidx_layout(bad, 3, 3, nullptr, 0, nullptr, 0, &rows, &brows, &nblk) ==
           AWQ_ERROR_INVALID_VALUE);
    const int32_t neg[2] = {0, -1};
    EXPECT(gidx_layout(neg, 2, 2, nullptr, 0, nullptr, 0, &rows, &brows, &nblk) ==
           AWQ_ERROR_INVALID_VALUE);
    EXPECT(gidx_layout(nullptr, 2, 2, nullptr, 0, nullptr, 0, &rows, &brows, &nblk) ==
           AWQ_ERROR_INVALID_VALUE);
    EXPECT(gidx_layout(gi, 6, 0, nullptr, 0, nullptr, 0, &rows, &brows, &nblk) ==
           AWQ_ERROR_INVALID_VALUE);
    EXPECT(gidx_layout(gi, 6, 3, nullptr, 0, nullptr, 0, nullptr, &brows, &nblk) ==
           AWQ_ERROR_INVALID_VALUE);
  }
  {
    const size_t fixed = kAtomicRegionBytes;
    EXPECT(sorted_workspace_size(0, 256, 128, 64) == 0);
    EXPECT(sorted_workspace_size(4, 256, 128, 48) == 0);
    EXPECT(sorted_x_offset(4, 256, 128, 64) >= fixed);
    EXPECT(sorted_x_offset(16, 8192, 7168, 128) >= gemm_workspace_size(16, 8192, 7168, 128));
    EXPECT(sorted_x_offset(16, 8192, 7168, 128) % 256 == 0);
    EXPECT(sorted_workspace_size(16, 8192, 7168, 128) ==
           sorted_x_offset(16, 8192, 7168, 128) + 16 * 8192 * 2);
  }

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("plan_check ok\n");
  return 0;
}
