// Host-side validation and kernel planning (HIP-free).
#include "awq_plan.h"

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "awq.h"

namespace awq {

namespace {
constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;
// Work-groups to aim for in the decode grid: enough resident waves on 256
// CUs to keep many weight loads in flight, without multiplying the split-K
// partial sums more than needed.
constexpr int64_t kDecodeTargetWGs = 800;
constexpr int64_t kDecodeLdsTargetWGs = 384;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }
}  // namespace

int validate_shape(int64_t M, int64_t K, int64_t N, int64_t group_size, Problem* out) {
  if (M < 0 || K <= 0 || N <= 0) return AWQ_ERROR_INVALID_VALUE;
  if (group_size == 0 || group_size < -1) return AWQ_ERROR_INVALID_VALUE;
  if (N % 8 != 0) return AWQ_ERROR_SHAPE;
  const int64_t g = (group_size == -1) ? K : group_size;
  if (K % g != 0) return AWQ_ERROR_SHAPE;
  if (K > kMaxElems || N > kMaxElems || M > kMaxElems) return AWQ_ERROR_SHAPE;
  if (K * N > kMaxElems) return AWQ_ERROR_SHAPE;
  if (M * K > kMaxElems || M * N > kMaxElems) return AWQ_ERROR_SHAPE;
  if (out) {
    out->M = M;
    out->K = K;
    out->N = N;
    out->g = g;
    out->G = K / g;
  }
  return AWQ_SUCCESS;
}

int validate_gemm_pointers(const void* x, const void* qweight, const void* qzeros,
                           const void* scales, const void* bias, const void* y, int64_t M) {
  if (!qweight || !qzeros || !scales) return AWQ_ERROR_INVALID_VALUE;
  if (M > 0 && (!x || !y)) return AWQ_ERROR_INVALID_VALUE;
  if (!aligned(qweight, 4) || !aligned(qzeros, 4)) return AWQ_ERROR_MISALIGNED;
  if (!aligned(scales, 2)) return AWQ_ERROR_MISALIGNED;
  if (bias && !aligned(bias, 2)) return AWQ_ERROR_MISALIGNED;
  if (x && !aligned(x, 2)) return AWQ_ERROR_MISALIGNED;
  if (y && !aligned(y, 2)) return AWQ_ERROR_MISALIGNED;
  return AWQ_SUCCESS;
}

int validate_dequant_pointers(const void* qweight, const void* qzeros,
                              const void* scales, const void* w) {
  if (!qweight || !qzeros || !scales || !w) return AWQ_ERROR_INVALID_VALUE;
  if (!aligned(qweight, 4) || !aligned(qzeros, 4)) return AWQ_ERROR_MISALIGNED;
  if (!aligned(scales, 2) || !aligned(w, 2)) return AWQ_ERROR_MISALIGNED;
  return AWQ_SUCCESS;
}

int validate_dense(const void* x, const void* w, const void* bias, const void* y, int64_t M,
                   int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0) return AWQ_ERROR_INVALID_VALUE;
  if (!w) return AWQ_ERROR_INVALID_VALUE;
  if (M > 0 && (!x || !y)) return AWQ_ERROR_INVALID_VALUE;
  if (M > kDenseMaxM || K % 8 != 0 || M * K > kDenseMaxMK) return AWQ_ERROR_SHAPE;
  if (K > kMaxElems || N > kMaxElems || K * N > kMaxElems || M * N > kMaxElems)
    return AWQ_ERROR_SHAPE;
  if (!aligned(w, 16) || (x && !aligned(x, 16))) return AWQ_ERROR_MISALIGNED;
  if ((y && !aligned(y, 2)) || (bias && !aligned(bias, 2))) return AWQ_ERROR_MISALIGNED;
  return AWQ_SUCCESS;
}

// The fast kernels address every operand with 32-bit byte offsets (buffer
// loads whose out-of-range offsets read zero): keep each operand below 1 GiB.
static bool fits_32bit_offsets(const Problem& p) {
  const int64_t lim = int64_t{1} << 29;  // elements of 2 bytes
  return p.M * p.K <= lim && p.M * p.N <= lim && p.K * p.N / 4 <= lim;
}

// Split-K work-groups per column tile for a step count: rows per work-group
// are `waves` waves (LDS variant: 4 or 8) or 2 waves (register variant)
// x 32 x steps.
static int64_t decode_splits(const Problem& p, bool lds, int steps, int waves = 4) {
  const int waves_k = lds ? waves : 2;
  return ceil_div(p.K, static_cast<int64_t>(waves_k) * kDecodeRowsPerStep * steps);
}

// Whether every wave's rows lie in one quantisation group at `steps` steps
// per wave (work-group row ranges start at multiples of the wave's rows).
static bool decode_single_group(const Problem& p, int steps) {
  return p.G == 1 || p.g % (static_cast<int64_t>(kDecodeRowsPerStep) * steps) == 0;
}

// More than one MFMA row block (17-32 rows) runs only in the LDS variant
// with one group per wave: some step count must give that within the split
// limit.
static bool decode_two_blocks_fit(const Problem& p) {
  for (int s = 8; s >= 1; s /= 2)
    if (decode_single_group(p, s) && decode_splits(p, true, s) <= kDecodeMaxSplits) return true;
  return false;
}

bool decode_supported(const Problem& p, const Alignment& al) {
  // 16-byte x loads need K % 8 == 0; a group must not change inside a wave's
  // 32-row step; the LDS-streaming variant (N % 32 == 0) copies 16-byte row
  // segments; the split-K exchange counts at most kDecodeMaxSplits splits
  // (at 8 steps per wave).
  const bool lds = p.N % 32 == 0;
  return fits_32bit_offsets(p) && p.M <= kDecodeMaxM && p.K % 8 == 0 && al.x && al.scales &&
         (!lds || al.qweight) && (p.g % kDecodeRowsPerStep == 0 || p.G == 1) &&
         decode_splits(p, lds, 8) <= kDecodeMaxSplits &&
         (p.M <= kDecodeBlockM || (lds && decode_two_blocks_fit(p)));
}

static int log2_exact(int64_t v) {
  int s = 0;
  while ((int64_t{1} << s) < v) ++s;
  return (int64_t{1} << s) == v ? s : -1;
}

bool prefill_supported(const Problem& p, const Alignment& al) {
  // Dequantisation works on 4-row blocks that must share a group, and the
  // kernel finds a row's group with a shift: a power-of-two group size of at
  // least 4, or a single group.
  return fits_32bit_offsets(p) && p.K % 8 == 0 && al.x && al.scales &&
         (p.G == 1 || (p.g >= 4 && log2_exact(p.g) >= 0));
}

// Planner overrides (awq_set_option).  Each starts from its environment
// variable, read once on first use, and can be changed later through the
// C ABI; planning reads them with relaxed atomic loads, so a call never
// touches the environment.  kOptAuto means "the planner's own choice";
// kOptInvalid marks an unrecognised AWQ_FORCE_PATH, which fails every plan.
namespace {
constexpr int kOptInvalid = -2;
constexpr int kNumOptions = AWQ_OPT_PREFILL_PACKED + 1;

bool option_value_ok(int opt, int64_t v) {
  if (v == kOptAuto) return true;
  switch (opt) {
    case AWQ_OPT_FORCE_PATH:
      return v == AWQ_PATH_DECODE || v == AWQ_PATH_PREFILL || v == AWQ_PATH_GENERIC;
    case AWQ_OPT_DECODE_STEPS: return v == 1 || v == 2 || v == 4 || v == 8;
    case AWQ_OPT_DECODE_GATHER_MAX_M: return v >= 0 && v <= kDecodeBlockM;
    case AWQ_OPT_PREFILL_BM: return v == kPrefillMinBM || v == 2 * kPrefillMinBM || v == kPrefillBM;
    case AWQ_OPT_PREFILL_BN: return v == kPrefillBN || v == kPrefillWideBN || v == kPackedBN;
    case AWQ_OPT_PREFILL_SPLITS: return v >= 1 && v <= kPrefillMaxSplits;
    case AWQ_OPT_DECODE_WAVES: return v == 4 || v == 8;
    case AWQ_OPT_PREFILL_PACKED: return v >= 0 && v <= 3;
    default: return false;
  }
}

int option_from_env(int opt) {
  static const char* const names[kNumOptions] = {
      nullptr, "AWQ_FORCE_PATH", "AWQ_DECODE_STEPS", "AWQ_DECODE_GATHER_MAX_M",
      "AWQ_PREFILL_BM", "AWQ_PREFILL_BN", "AWQ_PREFILL_SPLITS", "AWQ_DECODE_WAVES", "AWQ_PREFILL_PACKED"};
  const char* s = getenv(names[opt]);
  if (!s || !*s) return kOptAuto;
  if (opt == AWQ_OPT_FORCE_PATH) {
    if (!strcmp(s, "decode")) return AWQ_PATH_DECODE;
    if (!strcmp(s, "prefill")) return AWQ_PATH_PREFILL;
    if (!strcmp(s, "generic")) return AWQ_PATH_GENERIC;
    return kOptInvalid;
  }
  const int v = atoi(s);   // unusable numeric values leave the automatic choice
  return option_value_ok(opt, v) ? v : kOptAuto;
}

std::atomic<int>* option_table() {
  static std::atomic<int> table[kNumOptions];
  static const bool loaded = [] {
    for (int o = 1; o < kNumOptions; ++o) table[o].store(option_from_env(o));
    return true;
  }();
  (void)loaded;
  return table;
}
}  // namespace

int option(int opt) { return option_table()[opt].load(std::memory_order_relaxed); }

int set_option(int opt, int64_t value) {
  if (opt < 1 || opt >= kNumOptions) return AWQ_ERROR_INVALID_VALUE;
  if (!option_value_ok(opt, value)) return AWQ_ERROR_INVALID_VALUE;
  option_table()[opt].store(static_cast<int>(value), std::memory_order_relaxed);
  return AWQ_SUCCESS;
}

int get_option(int opt, int64_t* value) {
  if (opt < 1 || opt >= kNumOptions || !value) return AWQ_ERROR_INVALID_VALUE;
  *value = option(opt);
  return AWQ_SUCCESS;
}

static int override_or_zero(int opt) {
  const int v = option(opt);
  return v > 0 ? v : 0;
}

int make_plan(const Problem& p, const Alignment& al, int force, Plan* out) {
  Plan pl;
  memset(&pl, 0, sizeof(pl));
  const bool dec = decode_supported(p, al);
  const bool pre = prefill_supported(p, al);
  int path;
  if (force == 0) {
    // 17-32 rows: the decode kernel's two-block form where the weight is
    // large and its split partials (written, then read back by the sum
    // kernel) are at most half the packed weight's bytes, else the prefill
    // kernel.
    bool dec_auto = dec;
    if (dec && pre && p.M > kDecodeBlockM) {
      Plan d;
      dec_auto = p.K * p.N >= kDecodeTwoBlockMinWeights &&
                 make_plan(p, al, AWQ_PATH_DECODE, &d) == AWQ_SUCCESS &&
                 16 * static_cast<int64_t>(d.splits) * p.M <= p.K;
    }
    path = dec_auto ? AWQ_PATH_DECODE : (pre ? AWQ_PATH_PREFILL : AWQ_PATH_GENERIC);
  } else {
    path = force;
    if ((force == AWQ_PATH_DECODE && !dec) || (force == AWQ_PATH_PREFILL && !pre))
      return AWQ_ERROR_INVALID_VALUE;
    if (force != AWQ_PATH_DECODE && force != AWQ_PATH_PREFILL && force != AWQ_PATH_GENERIC)
      return AWQ_ERROR_INVALID_VALUE;
  }
  pl.path = path;
  if (path == AWQ_PATH_DECODE) {
    pl.n_tiles = static_cast<int>(ceil_div(p.N, kDecodeCols));
    pl.decode_lds = (p.N % 32 == 0);
    pl.decode_waves = 4;
    const int waves_opt = override_or_zero(AWQ_OPT_DECODE_WAVES);
    if (pl.decode_lds && waves_opt == 8) pl.decode_waves = 8;
    const int waves = pl.decode_waves;
    // Two row blocks need one group per wave.
    const bool two_blocks = p.M > kDecodeBlockM;
    const int steps_opt = override_or_zero(AWQ_OPT_DECODE_STEPS);
    int steps = steps_opt;
    if (steps != 0 && (decode_splits(p, pl.decode_lds, steps, waves) > kDecodeMaxSplits ||
                       (two_blocks && !decode_single_group(p, steps))))
      steps = 0;
    if (steps == 0) {
      // The largest step count whose rows stay in one quantisation group and
      // that still gives enough work-groups; failing that, the largest that
      // gives enough work-groups (a wave whose rows span groups scales each
      // step on its own whatever the count, and fewer splits mean less to
      // exchange); failing that, the one with the most work-groups.  8 steps
      // only when fewer would need more than kDecodeMaxSplits splits.
      const int64_t target = pl.decode_lds ? kDecodeLdsTargetWGs : kDecodeTargetWGs;
      int single_enough = 0, enough = 0, most = 0;
      for (int s = 4; s >= 1; s /= 2) {
        const bool single = decode_single_group(p, s);
        const int64_t splits = decode_splits(p, pl.decode_lds, s, waves);
        if (splits > kDecodeMaxSplits) break;
        if (two_blocks && !single) continue;
        most = s;
        if (pl.n_tiles * splits >= target) {
          if (single && single_enough == 0) single_enough = s;
          if (enough == 0) enough = s;
        }
      }
      steps = single_enough ? single_enough : (enough ? enough : (most ? most : 8));
    }
    // Above the atomic exchange every split's partials are stored and read
    // back by the sum kernel, so eight waves of four steps (half the splits
    // of four waves, one group per wave) are taken whenever their work-groups
    // make one resident round that fills the CUs: K = 8192, N = 7168, M = 16:
    // 14.7 -> 14.0 us, M = 32: 19.6 -> 18.2 us; K = 4096, N = 11008, M = 16
    // (against 2 steps of four waves): 16.5 -> 13.3 us; K = 14336, N = 4096,
    // M = 16: 16.1 -> 15.3 us.  Two rounds (K = 8192, N = 14336, 448
    // work-groups) or idle CUs (56-64 work-groups) lose.
    pl.decode_atomic = decode_atomic_capable(p.M, p.N) &&
                       decode_splits(p, pl.decode_lds, steps, pl.decode_waves) * p.M * p.N <
                           kDecodeAtomicMaxOps;
    if (pl.decode_lds && waves_opt == 0 && steps_opt == 0 && !pl.decode_atomic &&
        decode_single_group(p, 4)) {
      const int64_t s8 = decode_splits(p, true, 4, 8);
      const int64_t wg8 = pl.n_tiles * s8;
      if (s8 <= kDecodeMaxSplits && wg8 >= kDecodeEightWaveMinWGs &&
          wg8 <= kDecodeEightWaveMaxWGs) {
        steps = 4;
        pl.decode_waves = 8;
      }
    }
    // One row on the atomic exchange: four waves of four steps become eight
    // waves of two (the same work-groups and splits), so the arithmetic left
    // when the last copies land is at most two steps per wave.  Same box:
    // K = 14336, N = 4096: 10.06 -> 9.62 us; K = 4096, N = 12288: 9.62 ->
    // 9.46 us; K = 28672, N = 8192: 28.9 -> 28.1 us; K = 8192, N = 28672:
    // 29.2 -> 28.8 us; K = 8192, N = 7168: 9.38 -> 9.43 us.  Not for more
    // rows (M = 2, 3: 0.4 us slower) nor from two steps to one (slower).
    if (pl.decode_lds && waves_opt == 0 && steps_opt == 0 && pl.decode_atomic && p.M == 1 &&
        steps == 4 && decode_single_group(p, 2)) {
      steps = 2;
      pl.decode_waves = 8;
    }
    // Eight waves of eight steps would need 272 KiB of LDS: four waves then.
    if (pl.decode_waves == 8 && steps == 8) pl.decode_waves = 4;
    pl.steps = steps;
    pl.splits = static_cast<int>(decode_splits(p, pl.decode_lds, steps, pl.decode_waves));
    if (pl.splits > 1)
      pl.ws_bytes = kAtomicRegionBytes +
                    static_cast<size_t>(pl.splits) * p.M * p.N * sizeof(float);
  } else if (path == AWQ_PATH_PREFILL) {
    // The packed-weight tile where it applies and fills the CUs without a
    // split; its width is the one whose rounds of work-groups over the CUs
    // cost less (rounds x columns per tile).
    const int packed_opt = option(AWQ_OPT_PREFILL_PACKED);
    const int64_t m_tiles_p = ceil_div(p.M, kPackedBM);
    const int64_t t256 = m_tiles_p * ceil_div(p.N, kPackedBN);
    const int64_t t192 = m_tiles_p * ceil_div(p.N, kPackedNarrowBN);
    // Automatic: where it applies and its tiles fill the CUs; forced (1):
    // wherever it applies; 0: never.
    const bool packed_fits = p.M > 2 * kPrefillMinBM && p.K % kPrefillBK == 0 &&
                             p.N % 32 == 0 && al.qweight && (p.G == 1 || p.g % kPrefillBK == 0) &&
                             override_or_zero(AWQ_OPT_PREFILL_SPLITS) <= 1 &&
                             override_or_zero(AWQ_OPT_PREFILL_BM) == 0;
    const bool packed_ok = packed_fits && (packed_opt >= 1 || (packed_opt == kOptAuto &&
                                                               kPackedAuto &&
                                                               t192 >= kPrefillTargetWGs));
    if (packed_ok) {
      const int64_t c256 = ceil_div(t256, kPrefillTargetWGs) * kPackedBN;
      const int64_t c192 = ceil_div(t192, kPrefillTargetWGs) * kPackedNarrowBN;
      int bn = c192 < c256 ? kPackedNarrowBN : kPackedBN;
      const int o = override_or_zero(AWQ_OPT_PREFILL_BN);
      if (o == kPackedBN || o == kPackedNarrowBN) bn = o;
      pl.prefill_packed = true;
      // Waves along M: one (each wave all 256 rows of 64 columns) for the
      // 256-column tile, two for the 192-column one; option value 2 takes two
      // for either (tuning).
      pl.packed_wm = bn == kPackedNarrowBN ? 2 : (packed_opt >= 2 ? packed_opt : 1);
      pl.prefill_bm = kPackedBM;
      pl.prefill_bn = bn;
      pl.m_tiles = static_cast<int>(m_tiles_p);
      pl.n_tiles = static_cast<int>(ceil_div(p.N, bn));
      pl.group_shift = p.G == 1 ? 31 : log2_exact(p.g);
      pl.splits = 1;
      pl.steps = static_cast<int>(p.K / kPrefillBK);
      *out = pl;
      return AWQ_SUCCESS;
    }
    // Tile width and split count for a tile height: the wide tile (256 rows
    // only) does 1.5x a narrow tile's work at a little more speed per flop
    // (fewer LDS bytes per flop): take it when it needs no split and its
    // rounds of work-groups over the CUs cost less.  Split K when the tiles
    // alone leave CUs idle and K is long enough.
    const int64_t nkt = ceil_div(p.K, kPrefillBK);
    auto shape_for = [&](int bm, int* bn, int64_t* tiles, int64_t* splits) {
      const int64_t m_tiles = ceil_div(p.M, bm);
      const int64_t r_narrow = ceil_div(m_tiles * ceil_div(p.N, kPrefillBN), kPrefillTargetWGs);
      const int64_t wide_tiles = m_tiles * ceil_div(p.N, kPrefillWideBN);
      const int64_t r_wide = ceil_div(wide_tiles, kPrefillTargetWGs);
      *bn = (bm == kPrefillBM && wide_tiles >= kPrefillTargetWGs && r_wide * 6 < r_narrow * 5)
                ? kPrefillWideBN
                : kPrefillBN;
      if (const int o = override_or_zero(AWQ_OPT_PREFILL_BN); o == kPrefillBN || o == kPrefillWideBN)
        *bn = o;
      if (bm != kPrefillBM) *bn = kPrefillBN;   // 192 needs 256 rows
      *tiles = m_tiles * ceil_div(p.N, *bn);
      *splits = 1;
      if (*tiles > 0 && *tiles < kPrefillTargetWGs) {
        *splits = kPrefillTargetWGs / *tiles;
        if (*splits > kPrefillMaxSplits) *splits = kPrefillMaxSplits;
        if (*splits > nkt / kPrefillMinSplitSteps) *splits = nkt / kPrefillMinSplitSteps;
        if (*splits < 2) *splits = 1;
      }
    };
    int bm = p.M <= kPrefillMinBM ? kPrefillMinBM
                                  : (p.M <= 2 * kPrefillMinBM ? 2 * kPrefillMinBM : kPrefillBM);
    const int bm_opt = override_or_zero(AWQ_OPT_PREFILL_BM);
    if (bm_opt) bm = bm_opt;
    int bn;
    int64_t tiles, splits;
    shape_for(bm, &bn, &tiles, &splits);
    // Short K (at most kPrefillShortKSteps steps): a split's partials and
    // the second kernel cost more than lower tiles lose, so when the
    // 256-row plan splits, take the tallest lower tile (128, or 64 for at most 256 rows)
    // whose tiles fill three quarters of the CUs without a split, else the
    // lowest allowed one with its own split.  Same box (us, before -> after):
    // K=1792 N=4096 M=256 21.3 -> 16.9, M=1024 30.1 -> 20.8; K=4096 N=4096
    // M=256 28.5 -> 22.1, M=512 30.6 -> 28.7; K=2048 N=8192 M=256 29.0 ->
    // 18.5, M=512 31.6 -> 24.0; K=4096 N=1536 M=2048 36.3 -> 35.2; K=4096
    // N=12288 M=256 37.2 -> 36.8.  Longer K keeps the tall split tile
    // (K=14336 N=4096 M=1024: 114 us split against 134 us at 128 rows).
    if (!bm_opt && override_or_zero(AWQ_OPT_PREFILL_SPLITS) == 0 && bm == kPrefillBM &&
        nkt <= kPrefillShortKSteps && splits > 1) {
      int pick = 0;
      for (int c = bm / 2; c >= kPrefillMinBM; c /= 2) {
        if (c == kPrefillMinBM && p.M > kPrefillMinBM * 4) break;
        int cbn;
        int64_t ct, cs;
        shape_for(c, &cbn, &ct, &cs);
        pick = c;
        if (ct * 4 >= kPrefillTargetWGs * 3) break;
      }
      if (pick) {
        bm = pick;
        shape_for(bm, &bn, &tiles, &splits);
      }
    }
    pl.prefill_bm = bm;
    pl.prefill_bn = bn;
    pl.m_tiles = static_cast<int>(ceil_div(p.M, bm));
    pl.n_tiles = static_cast<int>(ceil_div(p.N, bn));
    pl.group_shift = p.G == 1 ? 31 : log2_exact(p.g);
    if (const int o = override_or_zero(AWQ_OPT_PREFILL_SPLITS)) splits = o < nkt ? o : nkt;
    const int64_t kps = ceil_div(nkt, splits);
    splits = ceil_div(nkt, kps);   // no empty split
    pl.splits = static_cast<int>(splits);
    pl.steps = static_cast<int>(kps);
    if (splits > 1)
      pl.ws_bytes = kAtomicRegionBytes +
                    static_cast<size_t>(splits) * p.M * p.N * sizeof(float);
  }
  *out = pl;
  return AWQ_SUCCESS;
}

size_t gemm_workspace_size(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  Problem p;
  if (validate_shape(M, K, N, group_size, &p) != AWQ_SUCCESS) return 0;
  const Alignment al{true, true, true};
  size_t need = 0;
  Plan pl;
  if (decode_supported(p, al) && make_plan(p, al, AWQ_PATH_DECODE, &pl) == AWQ_SUCCESS)
    need = pl.ws_bytes;
  if (prefill_supported(p, al) && make_plan(p, al, AWQ_PATH_PREFILL, &pl) == AWQ_SUCCESS &&
      pl.ws_bytes > need)
    need = pl.ws_bytes;
  return need;
}

int validate_gidx_shape(int64_t M, int64_t K, int64_t N, int64_t num_groups, Problem* out) {
  if (M < 0 || K <= 0 || N <= 0 || num_groups <= 0) return AWQ_ERROR_INVALID_VALUE;
  if (N % 8 != 0) return AWQ_ERROR_SHAPE;
  if (K > kMaxElems || N > kMaxElems || M > kMaxElems || num_groups > kMaxElems)
    return AWQ_ERROR_SHAPE;
  if (K * N > kMaxElems || M * K > kMaxElems || M * N > kMaxElems || num_groups * N > kMaxElems)
    return AWQ_ERROR_SHAPE;
  if (out) {
    out->M = M;
    out->K = K;
    out->N = N;
    out->g = 0;
    out->G = num_groups;
  }
  return AWQ_SUCCESS;
}

int gidx_layout(const int32_t* g_idx, int64_t K, int64_t num_groups, int32_t* perm,
                int64_t perm_capacity, int32_t* block_group, int64_t block_capacity,
                int64_t* rows, int64_t* block_rows, int64_t* blocks) {
  if (!g_idx || !rows || !block_rows || !blocks || K <= 0 || num_groups <= 0)
    return AWQ_ERROR_INVALID_VALUE;
  if (K > kMaxElems || num_groups > kMaxElems) return AWQ_ERROR_SHAPE;
  for (int64_t k = 0; k < K; ++k)
    if (g_idx[k] < 0 || g_idx[k] >= num_groups) return AWQ_ERROR_INVALID_VALUE;
  // Stable sort of the row indices by group (memory O(K), independent of
  // num_groups); host allocation failure is reported, never thrown across
  // the C ABI.
  try {
    std::vector<int32_t> order(static_cast<size_t>(K));
    for (int64_t k = 0; k < K; ++k) order[static_cast<size_t>(k)] = static_cast<int32_t>(k);
    std::stable_sort(order.begin(), order.end(),
                     [g_idx](int32_t a, int32_t b) { return g_idx[a] < g_idx[b]; });
    // Activation order: every group holds K / num_groups rows, i.e. the
    // sorted map is j / (K / num_groups) at every position j.
    bool whole = K % num_groups == 0;
    const int64_t per = whole ? K / num_groups : 0;
    whole = whole && per >= kGidxBlockRows && (per & (per - 1)) == 0;
    for (int64_t j = 0; j < K && whole; ++j)
      if (g_idx[order[static_cast<size_t>(j)]] != j / per) whole = false;
    if (whole) {
      *rows = K;
      *block_rows = per;
      *blocks = num_groups;
    } else {
      int64_t nb = 0;
      for (int64_t j = 0; j < K;) {
        int64_t e = j;
        while (e < K && g_idx[order[static_cast<size_t>(e)]] == g_idx[order[static_cast<size_t>(j)]]) ++e;
        nb += (e - j + kGidxBlockRows - 1) / kGidxBlockRows;
        j = e;
      }
      // An even block count keeps the row count a multiple of the prefill
      // kernel's 64-row K step (no masked tail step): one null block more.
      nb += nb & 1;
      *rows = nb * kGidxBlockRows;
      *block_rows = kGidxBlockRows;
      *blocks = nb;
    }
    if (*rows > kMaxElems) return AWQ_ERROR_SHAPE;
    if (!perm && !block_group) return AWQ_SUCCESS;   // size query
    if (!perm || !block_group || perm_capacity < *rows || block_capacity < *blocks)
      return AWQ_ERROR_SHAPE;
    if (whole) {
      for (int64_t j = 0; j < K; ++j) perm[j] = order[static_cast<size_t>(j)];
      for (int64_t b = 0; b < num_groups; ++b) block_group[b] = static_cast<int32_t>(b);
    } else {
      int64_t out = 0, b = 0;
      for (int64_t j = 0; j < K;) {
        const int32_t grp = g_idx[order[static_cast<size_t>(j)]];
        int64_t e = j;
        while (e < K && g_idx[order[static_cast<size_t>(e)]] == grp) ++e;
        const int64_t nblk = (e - j + kGidxBlockRows - 1) / kGidxBlockRows;
        for (int64_t t = 0; t < nblk * kGidxBlockRows; ++t)
          perm[out++] = j + t < e ? order[static_cast<size_t>(j + t)] : -1;
        for (int64_t t = 0; t < nblk; ++t) block_group[b++] = grp;
        j = e;
      }
      if (b < *blocks) {   // the trailing null block (any valid group)
        for (int64_t t = 0; t < kGidxBlockRows; ++t) perm[out++] = -1;
        block_group[b] = block_group[b - 1];
      }
    }
  } catch (...) {
    return AWQ_ERROR_INVALID_VALUE;
  }
  return AWQ_SUCCESS;
}

size_t sorted_x_offset(int64_t M, int64_t rows, int64_t N, int64_t block_rows) {
  // Never inside the regions that must stay zero between calls, whatever
  // this problem's own plan needs: the workspace may also serve awq_gemm
  // calls of other shapes.
  size_t base = gemm_workspace_size(M, rows, N, block_rows);
  const size_t fixed = kAtomicRegionBytes;
  if (base < fixed) base = fixed;
  return round_up(base, 256);
}

size_t sorted_workspace_size(int64_t M, int64_t rows, int64_t N, int64_t block_rows) {
  if (M <= 0 || validate_shape(M, rows, N, block_rows, nullptr) != AWQ_SUCCESS) return 0;
  return sorted_x_offset(M, rows, N, block_rows) +
         round_up(static_cast<size_t>(M) * static_cast<size_t>(rows) * 2, 256);
}

int decode_gather_max_m() {
  const int v = option(AWQ_OPT_DECODE_GATHER_MAX_M);
  return v >= 0 ? v : kDecodeGatherMaxM;
}

int forced_path() {
  const int v = option(AWQ_OPT_FORCE_PATH);
  if (v == kOptInvalid) return -1;
  return v > 0 ? v : 0;
}

}  // namespace awq
