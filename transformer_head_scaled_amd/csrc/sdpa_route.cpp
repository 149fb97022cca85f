// Which attention kernel, and which workgroup shape, a problem runs on.
//
// One function decides for every mha_sdpa / mha_sdpa_window call; the
// launchers (sdpa_fwd.hip, sdpa_window.hip, sdpa_wide.hip, sdpa_decode.hip)
// instantiate exactly what it returns, the MHA_TRACE log prints it, and
// mha_sdpa_route() hands it to callers and tests.  Host code only.
//
// The rules and the measurements behind them (MI355X, interleaved runs of
// the alternatives on one box, identical results):
//
// * fp32: one kernel, 64 rows a workgroup (16, four lanes a row, where
//   64-row workgroups would number fewer than the 1024 SIMDs).
// * d = 256, 512: the wide-head kernel, 4 waves that split d per 32-row
//   block: unmasked, two blocks (8 waves) a workgroup sharing the staged
//   K/V tiles; causal, one block (at d = 512 8 waves, the key tiles split
//   between two groups of 4).
// * A window: the flash kernel's window form, rows as in the unmasked
//   two-block layout, at most 2 waves a workgroup while the window spans
//   fewer than 2048 keys besides the row itself (a workgroup walks the key
//   tiles of all its rows' windows; [4,8,4096,64], reach w both sides, four
//   waves against two: w 0 36.7 / 25.3 µs, 64 41.2 / 31.6, 256 55.4 / 41.8,
//   1024 97.9 / 88.9, 2048 141.8 / 145.3).
// * One query row, unmasked, d = 64 or 128, at least 512 keys: the decoding
//   kernel (registers only, 8 waves per (batch, head)).
// * Causal, d >= 64: the pair layout (one 32-row block a wave, two key
//   tiles a step); d = 16, 32: two blocks u and nb - 1 - u a wave (bound by
//   the exponentials, where the pair layout measured 5-10 % slower).
// * Unmasked, at most 64 query rows, at least 512 keys and fewer than 1024
//   (batch, head) pairs: the key split (the waves of a workgroup share one
//   32-row block and split the keys; with 2048 pairs at 512 keys the plain
//   layout, which fits several workgroups a CU, was faster).
// * Unmasked, d >= 64, fewer than two waves a SIMD with 64 rows a wave: the
//   pair layout (32 rows a wave doubles the waves).
// * Otherwise the two-block layout (64 rows a wave), 4 waves a workgroup
//   while that leaves two workgroups a CU, else 2; 1 for heads of at most 64
//   rows; 8 at d = 64 from 2048 rows where that leaves no ragged last round.

#include "kernels.h"
#include "mha.h"

namespace mha {

namespace {

constexpr int64_t kCUs = 256;
constexpr int64_t kSimds = kCUs * 4;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// two-block layout: waves per workgroup
int blocks_waves(int64_t n_q, int64_t heads) {
  if (n_q <= 64) return 1;
  return cdiv(n_q, 256) * heads >= 512 ? 4 : 2;
}

// Makespan of a grid in units of a tenth of a round of 256 CUs: eight-wave
// workgroups fill a CU (two waves a SIMD), so a partial last round costs a
// whole one; four-wave workgroups pair up two a CU, and a last round of at
// most one a CU (one wave a SIMD) measured about 0.6 of a round.
int64_t rounds8(int64_t wg8) { return cdiv(wg8, kCUs) * 10; }
int64_t rounds4(int64_t wg4) {
  const int64_t rem = wg4 % (2 * kCUs);
  return wg4 / (2 * kCUs) * 10 + (rem == 0 ? 0 : rem > kCUs ? 10 : 6);
}

// Pair layout: waves per workgroup.  Eight (each loaded tile serves 256 rows)
// where there are enough of them; four at d = 128 (one wave a SIMD), for short
// heads, for causal heads of at most 2048 rows ([16,8,512,64] +13 %,
// [16,8,1024,64] +10 % against eight: the waves of a workgroup wait for its
// longest block at every barrier) and for causal grids with fewer than two
// eight-wave workgroups a CU ([1,8,4096,64] 362 against 267 TFLOP/s: unequal
// work needs a second round to even out); unmasked by the makespan
// ([1,8,2048,64] 332 against 247, [4,8,1024,64] 529 against 409,
// [24,8,640,64] 608 against 435; [2,8,4096,64] and [8,16,384,64] keep eight).
int pairs_waves(int64_t n_q, int64_t heads, int d, bool causal) {
  if (n_q <= 32) return 1;
  if (n_q <= 64) return 2;
  if (d > 64 || n_q <= 128 || (causal && n_q <= 2048)) return 4;
  if (causal) return cdiv(n_q, 256) * heads < 2 * kCUs ? 4 : 8;
  return rounds4(cdiv(n_q, 128) * heads) < rounds8(cdiv(n_q, 256) * heads) ? 4 : 8;
}

bool use_split(int64_t n_q, int64_t n_k, int64_t heads, bool causal) {
  return !causal && n_q <= 64 && n_k >= 512 && heads < 1024;
}

// the key split's waves: a ring of 2 stages of 64 keys × (K + V) per wave
// within 128 KB of LDS, at most 4
int split_waves(int d) { return 512 / d / 2 < 4 ? 512 / d / 2 : 4; }

bool noncausal_pairs(int64_t n_q, int64_t heads, int d) {
  return d >= 64 && heads * cdiv(n_q, 64) < 2 * kSimds;
}

// Unmasked, d = 64, at least 2048 rows, where four waves would be chosen:
// eight-wave workgroups (512 rows: each staged tile serves twice the rows;
// [4,8,4096,64] +3.0 %, [2,8,8192,64] +3.6 %) unless they leave a ragged
// last round ([8,8,2560,64]: four waves 835 against 667 TFLOP/s).
bool noncausal_eight_waves(int64_t n_q, int64_t heads, int d) {
  if (!(d == 64 && n_q >= 2048 && blocks_waves(n_q, heads) == 4)) return false;
  return rounds8(cdiv(n_q, 512) * heads) <= rounds4(cdiv(n_q, 256) * heads);
}

}  // namespace

SdpaRoute sdpa_route(int dtype, bool causal, bool window, int64_t B, int64_t H, int64_t n_q,
                     int64_t n_k, int d, int64_t win_left, int64_t win_right) {
  const int64_t heads = B * H;
  SdpaRoute r{};
  if (dtype == MHA_F32) {
    // four lanes a row (16 rows a workgroup) where one lane a row would
    // leave SIMDs without a workgroup
    r.kernel = SDPA_K_F32, r.waves = 1, r.rows = heads * cdiv(n_q, 64) < kSimds ? 16 : 64;
  } else if (d > 128) {
    // causal, wide enough: the key tiles split between two groups (the
    // merge costs more than the split gains at d = 256)
    // causal at d = 512: the key tiles split between two groups; unmasked:
    // two 32-row blocks a workgroup sharing each staged tile (d 256 +22 %,
    // 512 +8 %; causal d 256 lost 11 %, its longest row block growing)
    const bool ksplit = causal && d >= SDPA_WIDE_SPLIT_MIN_D;
    const int rs = causal ? 1 : 2;
    r.kernel = SDPA_K_WIDE, r.waves = ksplit ? 8 : 4 * rs, r.rows = 32 * rs;
  } else if (window) {
    int w = blocks_waves(n_q, heads);
    if (w > 2 && win_left + win_right < 2048) w = 2;
    r.kernel = SDPA_K_WINDOW, r.waves = w, r.rows = 64 * w;
  } else if (!causal && n_q == 1 && (d == 64 || d == 128) && n_k >= 512) {
    r.kernel = SDPA_K_DECODE, r.waves = 8, r.rows = 1;
  } else if (causal && d >= 64) {
    const int w = pairs_waves(n_q, heads, d, true);
    r.kernel = SDPA_K_PAIRS, r.waves = w, r.rows = 32 * w;
  } else if (use_split(n_q, n_k, heads, causal)) {
    r.kernel = SDPA_K_SPLIT, r.waves = split_waves(d), r.rows = 32;
  } else if (!causal && noncausal_pairs(n_q, heads, d)) {
    const int w = pairs_waves(n_q, heads, d, false);
    r.kernel = SDPA_K_PAIRS, r.waves = w, r.rows = 32 * w;
  } else {
    const int w = (!causal && noncausal_eight_waves(n_q, heads, d)) ? 8 : blocks_waves(n_q, heads);
    r.kernel = SDPA_K_BLOCKS, r.waves = w, r.rows = 64 * w;
  }
  // workgroups in the grid
  switch (r.kernel) {
    case SDPA_K_DECODE: r.workgroups = heads; break;
    case SDPA_K_BLOCKS:
      if (causal) {  // a wave takes two 32-row blocks u and nb - 1 - u
        const int64_t units = (cdiv(n_q, 32) + 1) / 2;
        r.workgroups = cdiv(units, r.waves) * heads;
        break;
      }
      [[fallthrough]];
    default: r.workgroups = cdiv(n_q, r.rows) * heads;
  }
  return r;
}

}  // namespace mha
