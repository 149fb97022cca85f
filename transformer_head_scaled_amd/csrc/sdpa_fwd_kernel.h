// Fused scaled dot-product attention forward for gfx950 (bf16 / fp16): the
// flash kernel template (instantiated by sdpa_fwd.hip and sdpa_window.hip).
//
// Computes, per (batch, head), O = softmax(scale · Q·Kᵀ) · V with the
// causal mask (key c visible to query r iff c <= r), a restricted window
// (r − left <= c <= r + right), and/or a per-batch valid key length -- eq.
// (1) of "Lire « Attention Is All You Need »" (nickwang.xyz), §3.2.1, with
// the decoder mask of "Trois usages de l'attention dans le modèle"
// (forbidden scores set to -inf before the softmax) and the restricted
// self-attention of §4.  The n_q × n_k score matrix is never formed: key/value tiles
// stream through LDS and an online softmax (running max m and sum l per
// query row, fp32) rescales the fp32 output accumulator.
//
// Work decomposition.  A workgroup is 1, 2, 4 or 8 waves of one (batch,
// head); each wave owns 64 query rows as two blocks of 32 (the forms below
// -- causal, key split, pair layout, window -- change which rows and keys a
// wave takes).  64-key K and V tiles pass through a 2-stage LDS ring.  Scores are formed
// transposed, Sᵀ = K·Qᵀ, with the 32x32x16 MFMA: K is the A operand (rows
// = keys, read from LDS), Q the B operand (columns = queries, kept in
// registers for the whole kernel).  In the MFMA result layout every lane
// then holds 16 scores of ONE query row (its column), the other 16 of that
// row sitting in lane l^32 -- so a row max needs a single cross-lane
// exchange (v_permlane32_swap).
//
// The output is formed transposed too, Oᵀ = Vᵀ·Pᵀ: P (rounded to the
// input dtype) is the B operand and comes straight out of the Sᵀ result
// registers.  Those registers hold, for lane half h, the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key step rather than 8 consecutive
// keys; the contraction order is free, so the Vᵀ fragments are read in the
// same key order.  V stays row-major in LDS and the fragments come from
// transposing LDS reads (ds_read_b64_tr_b16, 4 keys x 4 d per 16-lane
// group).  In the Oᵀ result each lane again holds its own query row, so a
// rescale of a row of O is a plain per-lane multiply.
//
// Schedule.  Per tile a wave computes S for block 0, then S for block 1
// interleaved with the exponentials of block 0, then P0·V interleaved with
// the exponentials of block 1, then P1·V, so that the matrix cores and the
// vector ALU of a SIMD work at the same time.
//
// Softmax without a per-tile max.  The reference value m of a row only has
// to keep the weights finite: with weights p = exp2(s·c − m·c) the softmax
// is the same for every m.  A tile is first exponentiated against the
// current m; as long as each lane's partial row sum stays ≤ 2^8 (so every
// weight is ≤ 2^8) the tile is accepted as is.  Otherwise the wave takes
// the exact path: row max, new m, rescale of O and l by
// exp2((m_old − m_new)·c), and the weights again.  A block's first tile
// with a visible key sets m to that tile's row max before its weights are
// formed (nothing to rescale yet), so it does not take the exact path.
// The row sums add the fp32 weights (P·V uses them rounded to the input
// dtype; the two differ by at most 2^-9 relative per weight).
//
// Loads.  K and V tiles go from memory straight into LDS (buffer loads with
// an LDS destination), with the 16-byte chunks of each row permuted (XOR
// with a few bits of the key, per head dimension) so that the fragment
// reads of a phase hit all 64 banks once.  The buffer range ends at the valid key
// length, so rows past it read as 0 without per-lane branches: whatever
// the memory there holds -- NaN included -- has no effect, matching the
// reading that a masked key has weight exactly 0.  Masked causal and window
// tiles check their value fragments for NaN/inf, whose product with a zero
// weight would still be NaN, and if there is one, clear them for the matrix
// product and add them back to the rows that see their keys.  Causal tiles
// entirely above the diagonal are never loaded, tiles a whole wave cannot
// see are skipped by that wave, and only the diagonal, window-edge and
// key-length boundary tiles evaluate the per-element mask.

#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

// K-row chunk permutation for head dimension D (16-byte chunks, D / 8 of
// them per row): chunk c of key k is stored at c ^ kswz<D>(k).  A fragment
// read of 16 lanes covers 16 consecutive keys at one chunk index; 256 bytes
// of LDS span all 64 banks, i.e. 256 / (2·D) rows, and the permutation
// spreads the 16 keys over the 16 different 16-byte bank groups.
template <int D>
__host__ __device__ constexpr int kswz(int key) {
  return (key / (128 / D)) & (D / 8 - 1);
}
// V-row chunk permutation: a transposing read phase of 32 lanes covers 4
// consecutive keys (aligned to 4) × 32 columns = 4 × 64 bytes, which must
// land in different quarters of the 256-byte bank cycle.
template <int D>
__host__ __device__ constexpr int vswz(int key) {
  return D == 128 ? 4 * (key & 3) : D == 64 ? 4 * ((key >> 1) & 1) : 0;
}

// NW waves per workgroup, each owning 64 query rows (two blocks of 32), for
// head dimension DH = d_k = d_v in {16, 32, 64, 128}.  With DH = 128 the
// accumulators need more than 256 registers, so one wave per SIMD.
//
// SPLIT (few query rows, long key range, no causal mask -- a decoding step
// against a key/value cache): the NW waves of a workgroup share ONE 32-row
// query block and split the key range instead, wave w taking tiles w, w + NW,
// w + 2·NW, ... through a ring of its own in LDS, with no workgroup barrier
// in the key loop; at the end the NW partial results (reference value, row
// sum, unnormalised O) are merged through LDS with the rescale of the online
// softmax.  NW times the loads in flight per (batch, head); the ring of a
// wave has SPLIT_STAGES stages, so that many − 1 tiles are in flight.
#ifndef SDPA_SPLIT_STAGES
#define SDPA_SPLIT_STAGES 2
#endif
#ifndef SDPA_SPLIT_NW
#define SDPA_SPLIT_NW 4
#endif
// Ring stages of the key split for head dimension d: a wave's wait leaves
// (stages − 2) tiles of 2·(d / 8) load instructions outstanding, below the
// counter's 64.
constexpr int split_stages(int d) {
  return SDPA_SPLIT_STAGES < 2 + 63 / (2 * (d / 8)) ? SDPA_SPLIT_STAGES : 2 + 63 / (2 * (d / 8));
}
// Waves of the key split: a ring per wave, waves × stages × 64 keys × (K + V)
// rows of 2·d bytes within 128 KB of LDS.
constexpr int split_waves(int d) {
  return SDPA_SPLIT_NW < 512 / d / split_stages(d) ? SDPA_SPLIT_NW : 512 / d / split_stages(d);
}
//
// WINDOW (restricted attention): key c is visible to query r iff
// r − win_left <= c <= r + win_right (and c below the key length).  The
// rows are laid out as in the unmasked case; a workgroup walks only the key
// tiles some of its rows can see, and each wave computes, per tile, nothing
// (no row of its own sees a key there), the masked tile code (a window edge
// crosses the tile) or the plain one (all its rows see the whole tile).
//
// PAIRS (the causal layout for d >= 64): one 32-row block per wave,
// consecutive blocks per workgroup, and two consecutive key tiles per step,
// which take the places of the two blocks of the default layout in the tile
// code (S of one tile computed while the other's exponentials run).
// Workgroups are launched longest first (the work of a block grows with its
// rows).  Without the mask it runs too; at full occupancy it measured slower
// than the default layout (d 64: 873 against 948 TFLOP/s), so unmasked
// heads take it only where 64 rows a wave would leave SIMDs without a
// second wave (sdpa_fwd.hip).
template <int DT, int DH, bool CAUSAL, int NW, bool SPLIT = false, bool WINDOW = false,
          bool PAIRS = false>
// (Two waves per SIMD as the register target, except where one is all there
// can be: one-wave workgroups, d = 128, the key split, and two-wave pair
// workgroups, whose 64 KB of LDS leaves room for two per compute unit.)
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(
    (NW == 1 || DH > 64 || SPLIT || (PAIRS && NW <= 2)) ? 1 : 2, 2))) void sdpa_fwd_kernel(SdpaArgs p) {
  static_assert(!(SPLIT && CAUSAL), "the key split is for the unmasked case");
  static_assert(!(WINDOW && (CAUSAL || SPLIT)), "the window has its own mask");
  static_assert(!PAIRS || (!SPLIT && !WINDOW), "the pair layout has no key split or window");
  constexpr int D = DH;
  constexpr int QB = 2, BN = 64, NSTAGE = SPLIT ? split_stages(DH) : 2;
  constexpr int BM = NW * 32 * QB;  // query rows per workgroup
  constexpr int NST = D / 16;       // 16-deep MFMA steps of a score block
  constexpr int NDB = D >= 32 ? D / 32 : 1;  // 32-row blocks of Oᵀ (d = 16: one, half used)
  constexpr int CR = D / 8;         // 16-byte chunks per K/V row
  constexpr int KPP = 64 / CR;      // keys per 1 KB piece of a tile
  constexpr int PIECES = BN / KPP;  // 1 KB pieces per K (or V) tile
  constexpr int CPW = PIECES >= NW ? PIECES / NW : 1;  // pieces loaded per (loading) wave
  constexpr int NKL = CR >= 8 ? CR / 4 : 1;  // distinct per-lane K offsets (by piece)
  static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head dimension");
  constexpr float kAccept = 256.f;  // accept a tile while partial row sums are <= 2^8
  constexpr int NBUF = SPLIT ? NW : 1;  // LDS rings: one per wave with the key split
  constexpr int NSLOT = PAIRS ? 2 : 1;  // tiles per ring stage

  // K tile: [key][D], rows of D / 8 16-byte chunks permuted by kswz
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NBUF][NSTAGE * NSLOT][BN * D];
  // V tile: [key][D], chunks permuted by vswz, which keeps the transposing
  // fragment reads conflict-free
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NBUF][NSTAGE * NSLOT][BN * D];

  // Rows.  Unmasked: workgroup qb of a head takes rows [qb·BM, qb·BM + BM),
  // each wave 64 consecutive rows.  Causal: the work of a row grows with its
  // index, so a wave takes the 32-row blocks u and nb − 1 − u of its head
  // (u = its unit, nb the number of 32-row blocks rounded up to even): every
  // wave then has about the same work and the two waves that share a SIMD
  // run side by side until the end, instead of a long wave finishing alone.
  const int nb32e = ((p.n_q + 31) / 32 + 1) & ~1;
  const int units = nb32e / 2;  // causal: waves of work per head
  const int nqb = PAIRS ? (p.n_q + NW * 32 - 1) / (NW * 32)
                  : SPLIT ? (p.n_q + 31) / 32 : CAUSAL ? (units + NW - 1) / NW : (p.n_q + BM - 1) / BM;
  const uint32_t total = (uint32_t)nqb * p.B * p.H;
  // pairs: highest rows (most work) first.  Workgroup x runs on XCD x % 8;
  // when the heads divide evenly, each XCD takes its own heads and walks
  // them row group by row group from the top, so a head's K/V is read from
  // memory by one XCD (round-robin heads measured as fast but re-read them:
  // 79 MB against 67 MB per launch); otherwise consecutive workgroups are
  // different heads at the same rows.  When the whole grid is resident at
  // once (pair_split != 0: two workgroups a CU, x and x + 8·pair_split on
  // one CU), the second round's slots of each XCD take the row groups in
  // the opposite order, shortest first, so that a CU holds a long and a
  // short row group instead of two of the same rank.
  const uint32_t hw = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
  const uint32_t t = PAIRS ? hw : xcd_remap(hw, total);
  const uint32_t nbh = (uint32_t)p.B * p.H;
  const bool xcd_heads = PAIRS && nbh % 8 == 0;
  const uint32_t hpx = nbh / 8, ps = (uint32_t)p.pair_split;
  const uint32_t xk = (PAIRS && ps != 0 && t / 8 >= ps) ? ps + (total / 8 - 1 - t / 8) : t / 8;
  const int bh = !PAIRS ? (int)(t / nqb)
                 : xcd_heads ? (int)((t % 8) * hpx + xk % hpx) : (int)(t % nbh);
  const int qb = !PAIRS ? (int)(t % nqb)
                 : xcd_heads ? nqb - 1 - (int)(xk / hpx) : nqb - 1 - (int)(t / nbh);
  const int b = bh / p.H, hh = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is the same for all lanes of a wave: readfirstlane makes
  // that visible to the compiler, so per-wave bounds are scalars
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  const int unit = qb * NW + wave;
  const bool wave_active =
      !CAUSAL || (PAIRS ? qb * NW * 32 + wave * 32 < p.n_q : unit < units);
  int row0[QB];  // first row of each of this wave's two 32-row blocks
  if (PAIRS) {
    // one block per wave; the tile code of the upper block does the work
    row0[0] = row0[1] = qb * NW * 32 + wave * 32;
  } else if (CAUSAL) {
    row0[0] = 32 * unit;
    row0[1] = 32 * (nb32e - 1 - unit);
  } else if (SPLIT) {
    // one block per workgroup; the tile code of the upper block does the work
    row0[0] = row0[1] = 32 * qb;
  } else {
    row0[0] = qb * BM + wave * 64;
    row0[1] = row0[0] + 32;
  }
  int kend = n_eff;
  // causal: keys up to the last row of the workgroup's first wave (its
  // upper block is the highest of the workgroup)
  if (CAUSAL) kend = min(kend, PAIRS ? qb * NW * 32 + NW * 32 : 32 * (nb32e - qb * NW));
  // window: the keys the workgroup's first row reaches back to, up to those
  // its last row reaches forward to
  int jlo = 0;  // first key tile of the workgroup
  if (WINDOW) {
    const int r_last = min(p.n_q, qb * BM + BM) - 1;
    kend = min(kend, r_last + p.win_right + 1);
    jlo = max(0, qb * BM - p.win_left) / BN;
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;  // one past the last tile

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;
  // buffer resources covering exactly the valid keys of this (batch, head)
  // (raw descriptor words: base, stride 0, byte range, format word)
  // (readfirstlane: the words are the same for every lane; saying so keeps
  // them in scalar registers, which the load instruction requires)
  const uint64_t kaddr = (uint64_t)(uintptr_t)Kg;
  const u32x4 krs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)kaddr),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(kaddr >> 32) & 0xffffu),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((int64_t)n_eff * p.k_sr * 2)),
                     0x00020000u};
  const uint64_t vaddr = (uint64_t)(uintptr_t)Vg;
  const u32x4 vrs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)vaddr),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(vaddr >> 32) & 0xffffu),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((int64_t)n_eff * p.v_sr * 2)),
                     0x00020000u};

  // ---- Q fragments (B operand), resident for the whole kernel
  u32x4 qf[QB][NST];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int row = row0[qi] + l32;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < p.n_q) v = *(const u32x4*)(Qg + (int64_t)row * p.q_sr + s * 16 + hi * 8);
      qf[qi][s] = p.neg ? flip_signs(v) : v;
    }
  }

  f32x16 o[QB][NDB];
  float m[QB], l[QB], mc[QB];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[qi][db] = f32x16{};
    m[qi] = -INFINITY;
    l[qi] = 0.f;
    mc[qi] = 0.f;
  }
  const float c = p.c;

  // ---- staging.  K and V go straight from memory into LDS (buffer loads
  // with an LDS destination: each wave instruction fills 1 KB = KPP keys,
  // lane i writing bytes [16i, 16i + 16)); every lane fetches the 16-byte
  // chunk that the permuted layout puts at its position.
  // Piece r (= wave·CPW + i) of a tile: lane -> key KPP·r + lane / CR, LDS
  // chunk lane % CR.  The K permutation of that key is (4r + lane / 16) &
  // (CR − 1), so it depends on r only through r mod NKL (and CPW is a
  // multiple of NKL); the V one depends on lane / 16 only.
  uint32_t k_lane[NKL];
#pragma unroll
  for (int v = 0; v < NKL; ++v) {
    const int key = KPP * v + lane / CR;  // a key of a piece r ≡ v (mod NKL)
    k_lane[v] = (uint32_t)(((lane / CR) * p.k_sr + ((lane % CR) ^ kswz<D>(key)) * 8) * 2);
  }
  const uint32_t v_lane =
      (uint32_t)(((lane / CR) * p.v_sr + ((lane % CR) ^ vswz<D>(lane / CR)) * 8) * 2);
  const uint32_t k_tile = (uint32_t)(BN * p.k_sr * 2), v_tile = (uint32_t)(BN * p.v_sr * 2);
  // the K offset of piece r for this lane: from the table when a wave's
  // pieces start a cycle of NKL (CPW a multiple of NKL), else computed
  auto k_lane_of = [&](int r, int i) __attribute__((always_inline)) {
    if constexpr (SPLIT || CPW % NKL == 0) {
      return k_lane[i % NKL];
    } else {
      const int key = KPP * r + lane / CR;  // this lane's key in the tile
      return (uint32_t)(((lane / CR) * p.k_sr + ((lane % CR) ^ kswz<D>(key)) * 8) * 2);
    }
  };
  // with fewer pieces than waves (D = 16, four waves) the last waves load none
  const bool loader = SPLIT || PIECES >= NW || wave < PIECES;
  constexpr int LPW = SPLIT ? PIECES : CPW;  // pieces this wave loads per tile
  const int kvw = SPLIT ? wave : 0;          // this wave's LDS ring

  // issue this wave's LDS-destination loads of K (or V) for one tile
  auto gload_k = [&](int tile, int stage) __attribute__((always_inline)) {
    if (!loader) return;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = (SPLIT ? 0 : wave * CPW) + i;
      // (the destinations are per wave: readfirstlane makes them scalars)
      load_lds_b128(krs,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&Ks[kvw][stage][r * 512]),
                    k_lane_of(r, i) + (uint32_t)(r * KPP * p.k_sr * 2) + tile * k_tile);
    }
  };
  auto gload_v = [&](int tile, int stage) __attribute__((always_inline)) {
    if (!loader) return;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = (SPLIT ? 0 : wave * CPW) + i;
      load_lds_b128(vrs,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&Vs[kvw][stage][r * 512]),
                    v_lane + (uint32_t)(r * KPP * p.v_sr * 2) + tile * v_tile);
    }
  };
  // K fragment (kb, st) of this lane: key kb·32 + l32, chunk 2·st + hi
  // (kb·32 is a multiple of 128 / D, so the permutation is that of l32)
  const int kx = kswz<D>(l32);
  auto kfrag = [&](int buf, int kb, int st) __attribute__((always_inline)) {
    return *(const u32x4*)&Ks[kvw][buf][(kb * 32 + l32) * D + (((2 * st + hi) ^ kx) * 8)];
  };
  // Vᵀ fragment (kb, t2, db): d = db·32 + l32 and the 8 keys that the score
  // registers hold for this lane half, {4·hi .. 4·hi+3, 8+4·hi .. 8+4·hi+3}
  // of 16-key step kb·32 + t2·16.  Two transposing reads, 4 keys each: lane
  // i of a 16-lane group points at key (i / 4) of the 4 and at d columns
  // 4·(i % 4) .. +3 of its 16; the read hands lane r element r % 4 of lane
  // 4j + r / 4, i.e. key j at column r.  With D = 16 the lanes of columns
  // 16..31 (which do not exist) read the other four keys of the 8-key group
  // instead, so their phase still covers distinct banks; the Oᵀ rows they
  // produce are never stored.
  const int i16 = lane & 15;
  const bool v_pad = D < 32 && ((lane >> 4) & 1);
  const int v_key_l = (4 * hi + (i16 >> 2)) ^ (v_pad ? 4 : 0);  // key offset within a 16-key step (+ 8·e)
  const int v_x = vswz<D>(v_key_l);  // the row permutation (the step starts at a multiple of 8)
  const int v_col = (D < 32 ? 0 : 16 * ((lane >> 4) & 1)) + 4 * (i16 & 3);  // d within the 32-column block
  auto vfrag = [&](int buf, int kb, int t2, int db) __attribute__((always_inline)) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = kb * 32 + t2 * 16 + 8 * e + v_key_l;
      const int d = db * 32 + v_col;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)&Vs[kvw][buf][key * D + (((d >> 3) ^ v_x) * 8) + (d & 7)]);
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * e] = w[0];
      r[2 * e + 1] = w[1];
    }
    return r;
  };

  // tiles this wave takes with the key split (j = wave + t·NW)
  const int myn = SPLIT ? (ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0) : 0;
  // vmcnt that leaves the loads of KEEP later tiles outstanding (each tile is
  // 2·LPW load instructions of this wave)
  constexpr int kSplitKeep = SPLIT ? (NSTAGE - 2) * 2 * LPW : 0;
  static_assert(kSplitKeep < 64, "vmcnt range");
  constexpr int kSplitWait = (kSplitKeep & 15) | ((kSplitKeep >> 4) << 14) | 0x0070;
  if (PAIRS) {  // the first pair of tiles into the two slots of stage 0
    if (ntiles > 0) {
      gload_k(0, 0);
      gload_v(0, 0);
    }
    if (ntiles > 1) {
      gload_k(1, 1);
      gload_v(1, 1);
    }
  } else if (SPLIT) {
#pragma unroll
    for (int t0 = 0; t0 < NSTAGE - 1; ++t0)  // this wave's first tiles
      if (t0 < myn) {
        gload_k(wave + t0 * NW, t0);
        gload_v(wave + t0 * NW, t0);
      }
  } else {
#pragma unroll
    for (int t0 = 0; t0 < NSTAGE - 1; ++t0)
      if (jlo + t0 < ntiles) {
        gload_k(jlo + t0, (jlo + t0) % NSTAGE);
        gload_v(jlo + t0, (jlo + t0) % NSTAGE);
      }
  }
  // tile 0 has landed (at most the four loads of tile 1 are outstanding),
  // then the workgroup barrier; the "memory" clobber keeps LDS accesses on
  // their side of it
  if (SPLIT && myn >= NSTAGE - 1)
    __builtin_amdgcn_s_waitcnt(kSplitWait);  // tile 0 landed, the later ones may be out
  else if (!SPLIT && NSTAGE > 2 && ntiles > jlo + 1)
    __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");

  // Non-finite values in masked causal and window tiles.  A masked score has
  // weight exactly 0, but inside the matrix product 0·NaN and 0·inf are NaN,
  // so a NaN or ±inf value row would reach every row of the 32-row block
  // that loads it, also rows that do not see its key.  The masked tiles
  // therefore check their Vᵀ fragments (wave-uniform; no such value: the
  // common path, unchanged); when one is there, the fragments go into P·V
  // with their non-finite elements cleared, and afterwards each row adds
  // those elements of the keys it does see (a visible key's weight is
  // positive, so p·x and x are the same NaN or infinity).
  auto v_has_nonfinite = [&](const u32x4 (&vf)[2][2][NDB]) __attribute__((always_inline)) {
    u16x2 acc = {0, 0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int w = 0; w < 4; ++w) acc = magnitude_max(acc, vf[kb][t2][db][w]);
    constexpr unsigned short lim = nonfinite_from<DT>();
    return __builtin_amdgcn_ballot_w64(acc[0] >= lim || acc[1] >= lim) != 0;
  };
  auto v_clear_nonfinite = [&](u32x4 (&vf)[2][2][NDB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int w = 0; w < 4; ++w) vf[kb][t2][db][w] = zero_nonfinite<DT>(vf[kb][t2][db][w]);
  };
  // O of query block qi += the non-finite elements of the values of the keys
  // of LDS stage buf (keys kbase ..) that the lane's row sees.  This lane's
  // accumulator element i of 32-row block db holds column
  // d = db·32 + 8·(i / 4) + 4·hi + i % 4: four consecutive columns per group
  // of four, read from the value row as one 8-byte word.
  auto add_nonfinite_v = [&](int qi, int buf, int kbase) __attribute__((always_inline)) {
    const int row = row0[qi] + l32;
    for (int k = 0; k < BN; ++k) {
      const int key = kbase + k;
      bool vis = key < n_eff;
      if constexpr (CAUSAL) vis = vis && key <= row;
      if constexpr (WINDOW) vis = vis && key >= row - p.win_left && key <= row + p.win_right;
      if (!vis) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hi;
          if (d >= D) continue;  // D = 16: the padding rows of Oᵀ
          const u32x2 w = *(const u32x2*)&Vs[kvw][buf][k * D + (((d >> 3) ^ vswz<D>(k)) * 8) + (d & 7)];
          const f32x4 x = unpack4<DT>(w);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!__builtin_isfinite(x[e])) o[qi][db][4 * g + e] += x[e];
        }
    }
  };

  // weights of key block kb of query block qi against the current reference
  // value; returns their partial row sum
  // The row sum adds the fp32 weights with plain adds: a packed dot2 would
  // be exact to the rounded P, but on gfx950 it does not issue alongside
  // the matrix cores, while adds do.
  auto weights = [&](int qi, int kb, const f32x16& sv, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -mc[qi]));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -mc[qi]));
      pw[i] = pack2<DT>(e0, e1);
      rs0 += e0;
      rs1 += e1;
    }
    return rs0 + rs1;
  };
  // A row block's first tile with a visible key: the accept test cannot
  // pass against a reference value of −∞, so the reference becomes the
  // tile's row max, taken from the scores in registers before the weights
  // are formed -- what the exact path below would set, without recomputing
  // the scores twice from LDS (o and l are still 0, so nothing is
  // rescaled; the results are bit-identical).  Rows that see no key here
  // keep −∞ and still take the exact path.  Only where a row block sees
  // few tiles, so that its first one weighs: the window (reach 0 +27 %,
  // 256 +13 %), the key split (+4 %) and d <= 32 (causal d 32 +3 %).  In the
  // d 64 and 128 kernels the test in the loop cost more than it saved
  // (unmasked [4,8,4096,64] −1.7 %, d 128 −7.5 %).
  constexpr bool kFirstRef = WINDOW || SPLIT || DH <= 32;
  auto set_ref = [&](int qi, const f32x16 (&sv)[2]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
    mx = pair_max(mx);
    if (m[qi] == -INFINITY) {
      m[qi] = mx;
      mc[qi] = (mx == -INFINITY ? 0.f : mx) * c;
    }
  };
  auto first_ref = [&](int qi, const f32x16 (&sv)[2]) __attribute__((always_inline)) {
    if (!kFirstRef) return;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(m[qi] == -INFINITY) != 0, 0)) set_ref(qi, sv);
  };
  // per-element mask of query block qi (diagonal and key-length boundary
  // tiles only)
  auto apply_mask = [&](int qi, int kbase, int kb, f32x16& sv) __attribute__((always_inline)) {
    const int row = row0[qi] + l32;
    if constexpr (WINDOW) {
      // visible iff lo <= the register's key offset in the tile < lim
      int lo = row - p.win_left - kbase - 4 * hi;
      int lim = min(n_eff, row + p.win_right + 1) - kbase - 4 * hi;
      asm volatile("" : "+v"(lo), "+v"(lim));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
        sv[i] = (off >= lo && off < lim) ? sv[i] : -INFINITY;
      }
      return;
    }
    // visible iff the register's key offset in the tile (a constant) < lim
    int lim = (CAUSAL ? min(n_eff, row + 1) : n_eff) - kbase - 4 * hi;
    // opaque to the optimiser: otherwise it hoists one loop-invariant
    // threshold per register out of the key loop (32 extra registers)
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
      sv[i] = off < lim ? sv[i] : -INFINITY;
    }
  };
  // Sᵀ of query block qi, key block kb, for the keys of LDS stage buf,
  // masked like the tile
  auto scores = [&](auto masked, int qi, int buf, int kbase, int kb) __attribute__((always_inline)) {
    f32x16 sv = {};
#pragma unroll
    for (int st = 0; st < NST; ++st) sv = mfma_32x32x16<DT>(kfrag(buf, kb, st), qf[qi][st], sv);
    if constexpr (decltype(masked)::value) apply_mask(qi, kbase, kb, sv);
    return sv;
  };
  // accept the tile's weights of query block qi, or take the exact path:
  // row max, new reference value, rescale of O and l, weights again.  The
  // exact path recomputes the scores from LDS (twice, one key block at a
  // time) instead of keeping them, which keeps the common path's register
  // footprint small.
  auto settle = [&](auto masked, int qi, int buf, int kbase, uint32_t (&pw)[2][8], float rs) __attribute__((always_inline)) {
    // `!(rs <= kAccept)` is also true for NaN
    const bool reject = (m[qi] == -INFINITY) || !(rs <= kAccept);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(reject) != 0, 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x16 sv = scores(masked, qi, buf, kbase, kb);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[i]);
      }
      mx = pair_max(mx);
      const float m_new = fmaxf(m[qi], mx);
      const float alpha = (m[qi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m[qi] - m_new) * c);
      m[qi] = m_new;
      mc[qi] = (m_new == -INFINITY ? 0.f : m_new) * c;
      l[qi] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qi][db][i] *= alpha;
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) rs += weights(qi, kb, scores(masked, qi, buf, kbase, kb), pw[kb]);
    }
    l[qi] += rs;
  };

  // One 64-key tile for this wave's two query blocks.  The instruction
  // order lets one block's exponentials issue between the matrix
  // instructions of the other:
  //   S0 (MFMA), then S1 (MFMA) interleaved with the weights of block 0,
  //   P0·V (MFMA) interleaved with the weights of block 1, then P1·V.
  auto tile = [&](auto masked, int buf, int kbase, auto&& mid) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    u32x4 kf[2][NST];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st) kf[kb][st] = kfrag(buf, kb, st);
    f32x16 s0[2], s1[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        s0[kb] = mfma_32x32x16<DT>(kf[kb][st], qf[0][st], st == 0 ? f32x16{} : s0[kb]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        s1[kb] = mfma_32x32x16<DT>(kf[kb][st], qf[1][st], st == 0 ? f32x16{} : s1[kb]);
    if constexpr (MASKED) {
      apply_mask(0, kbase, 0, s0[0]);
      apply_mask(0, kbase, 1, s0[1]);
    }
    uint32_t p0[2][8], p1[2][8];
    first_ref(0, s0);
    const float rs0 = weights(0, 0, s0[0], p0[0]) + weights(0, 1, s0[1], p0[1]);
    // (vector work first, then one MFMA: measured 0.6-1 % faster at d 64
    // and 3 % at d 128 than MFMA first; in the pair tile code below the
    // other order is 2.5-3 % faster)
#pragma unroll
    for (int g = 0; g < 2 * NST; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x402, 112 / (2 * NST), 0);  // VALU / transcendental
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // then one MFMA of S1
    }
    u32x4 vf[2][2][NDB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vf[kb][t2][db] = vfrag(buf, kb, t2, db);
    settle(masked, 0, buf, kbase, p0, rs0);
    mid();
    // (the check right before the products: earlier, the fragments would be
    // live across the exact path of `settle`)
    constexpr bool CHECK_V = MASKED && (CAUSAL || WINDOW);
    bool vbad = false;
    if constexpr (CHECK_V) {
      vbad = v_has_nonfinite(vf);
      if (vbad) v_clear_nonfinite(vf);
    }


#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 bv = {p0[kb][4 * t2], p0[kb][4 * t2 + 1], p0[kb][4 * t2 + 2], p0[kb][4 * t2 + 3]};
          o[0][db] = mfma_32x32x16<DT>(vf[kb][t2][db], bv, o[0][db]);
        }
    if constexpr (CHECK_V)
      if (vbad) add_nonfinite_v(0, buf, kbase);
    if constexpr (MASKED) {
      apply_mask(1, kbase, 0, s1[0]);
      apply_mask(1, kbase, 1, s1[1]);
    }
    first_ref(1, s1);
    const float rs1 = weights(1, 0, s1[0], p1[0]) + weights(1, 1, s1[1], p1[1]);
#pragma unroll
    for (int g = 0; g < 4 * NDB; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x402, 112 / (4 * NDB), 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA of P0·V
    }
    settle(masked, 1, buf, kbase, p1, rs1);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 bv = {p1[kb][4 * t2], p1[kb][4 * t2 + 1], p1[kb][4 * t2 + 2], p1[kb][4 * t2 + 3]};
          o[1][db] = mfma_32x32x16<DT>(vf[kb][t2][db], bv, o[1][db]);
        }
    if constexpr (CHECK_V)
      if (vbad) add_nonfinite_v(1, buf, kbase);
  };

  // One 64-key tile for block 1 only (causal: block 0 has no visible key
  // left).
  auto tile_hi = [&](auto masked, int buf, int kbase, auto&& mid) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 s1[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s1[kb] = scores(std::false_type{}, 1, buf, kbase, kb);
    mid();
    u32x4 vf[2][2][NDB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vf[kb][t2][db] = vfrag(buf, kb, t2, db);
    if constexpr (MASKED) {
      apply_mask(1, kbase, 0, s1[0]);
      apply_mask(1, kbase, 1, s1[1]);
    }
    uint32_t p1[2][8];
    first_ref(1, s1);
    const float rs1 = weights(1, 0, s1[0], p1[0]) + weights(1, 1, s1[1], p1[1]);
    settle(masked, 1, buf, kbase, p1, rs1);
    constexpr bool CHECK_V = MASKED && (CAUSAL || WINDOW);
    bool vbad = false;
    if constexpr (CHECK_V) {
      vbad = v_has_nonfinite(vf);
      if (vbad) v_clear_nonfinite(vf);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 bv = {p1[kb][4 * t2], p1[kb][4 * t2 + 1], p1[kb][4 * t2 + 2], p1[kb][4 * t2 + 3]};
          o[1][db] = mfma_32x32x16<DT>(vf[kb][t2][db], bv, o[1][db]);
        }
    if constexpr (CHECK_V)
      if (vbad) add_nonfinite_v(1, buf, kbase);
  };

  // Two consecutive 64-key tiles (LDS buffers bufA and bufA + 1) for block 1
  // alone, the pair layout.  The instruction order is that of `tile`, the
  // tiles in the places of the blocks: S_A, then S_B interleaved with the
  // weights of A; A is settled before B's weights are formed (both update
  // the block's one softmax state); P_A·V interleaved with the weights of B,
  // then P_B·V.
  auto tile_pair = [&](auto masked, int bufA, int kbaseA, auto&& mid) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // vector instructions per MFMA in the two interleaved phases (d = 64:
    // 16; against 14 = 112 / 8 it measured between −0.3 % and +1.6 %
    // causal over two boxes, i.e. the same within noise)
    constexpr int kPairValu = DH == 64 ? 16 : 112 / (2 * NST);
    constexpr int kPairValuPV = DH == 64 ? 16 : 112 / (4 * NDB);
    const int bufB = bufA + 1, kbaseB = kbaseA + BN;
    u32x4 kf[2][NST];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st) kf[kb][st] = kfrag(bufA, kb, st);
    f32x16 sa[2], sb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        sa[kb] = mfma_32x32x16<DT>(kf[kb][st], qf[1][st], st == 0 ? f32x16{} : sa[kb]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st) kf[kb][st] = kfrag(bufB, kb, st);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < NST; ++st)
        sb[kb] = mfma_32x32x16<DT>(kf[kb][st], qf[1][st], st == 0 ? f32x16{} : sb[kb]);
    // Tile A needs no mask: a masked pair runs only when some row of the
    // block sees a key of tile B, and then (keys below the block's first
    // row, below the key length) every row sees all of tile A.  So A takes
    // the unmasked path: no mask, no check of its values.
    uint32_t pa[2][8], pb[2][8];
    first_ref(1, sa);
    const float rsa = weights(1, 0, sa[0], pa[0]) + weights(1, 1, sa[1], pa[1]);
#pragma unroll
    for (int g = 0; g < 2 * NST; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, kPairValu, 0);
    }
    u32x4 vf[2][2][NDB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vf[kb][t2][db] = vfrag(bufA, kb, t2, db);
    settle(std::false_type{}, 1, bufA, kbaseA, pa, rsa);
    mid();
    constexpr bool CHECK_V = MASKED && CAUSAL;
    bool vbad = false;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 bv = {pa[kb][4 * t2], pa[kb][4 * t2 + 1], pa[kb][4 * t2 + 2], pa[kb][4 * t2 + 3]};
          o[1][db] = mfma_32x32x16<DT>(vf[kb][t2][db], bv, o[1][db]);
        }
    if constexpr (MASKED) {
      apply_mask(1, kbaseB, 0, sb[0]);
      apply_mask(1, kbaseB, 1, sb[1]);
    }
    first_ref(1, sb);
    const float rsb = weights(1, 0, sb[0], pb[0]) + weights(1, 1, sb[1], pb[1]);
#pragma unroll
    for (int g = 0; g < 4 * NDB; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, kPairValuPV, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vf[kb][t2][db] = vfrag(bufB, kb, t2, db);
    settle(masked, 1, bufB, kbaseB, pb, rsb);
    if constexpr (CHECK_V) {
      vbad = v_has_nonfinite(vf);
      if (vbad) v_clear_nonfinite(vf);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 bv = {pb[kb][4 * t2], pb[kb][4 * t2 + 1], pb[kb][4 * t2 + 2], pb[kb][4 * t2 + 3]};
          o[1][db] = mfma_32x32x16<DT>(vf[kb][t2][db], bv, o[1][db]);
        }
    if constexpr (CHECK_V)
      if (vbad) add_nonfinite_v(1, bufB, kbaseB);
  };

  // One step of the pair layout: start the loads of the next pair (tiles
  // 2s + 2, 2s + 3 into the other stage), compute this pair (both tiles,
  // the first only, or nothing), wait, barrier.
  auto pair_step = [&](int s, auto masked, auto what) __attribute__((always_inline)) {
    constexpr int WHAT = decltype(what)::value;
    const int nA = 2 * s + 2;
    const bool moreA = nA < ntiles, moreB = nA + 1 < ntiles;
    const int nbuf = 2 * ((s + 1) % NSTAGE);
    if (moreA) gload_k(nA, nbuf);
    if (moreB) gload_k(nA + 1, nbuf + 1);
    auto load_v = [&]() __attribute__((always_inline)) {
      if (moreA) gload_v(nA, nbuf);
      if (moreB) gload_v(nA + 1, nbuf + 1);
    };
    const int buf = 2 * (s % NSTAGE), kbase = 2 * s * BN;
    if constexpr (WHAT == 2)
      tile_pair(masked, buf, kbase, load_v);
    else if constexpr (WHAT == 1)
      tile_hi(masked, buf, kbase, load_v);
    else
      load_v();
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the next pair has landed
    asm volatile("s_barrier" ::: "memory");
  };

  // One step of the key loop: start the loads of tile j + NSTAGE - 1 (K and
  // V both at the top: V issued mid-tile, as the pair layout does, measured
  // 1.5-2.5 % slower here), compute tile j (both blocks, block 1 only, or
  // nothing), barrier.  WHAT: 0 = nothing, 1 = block 1 only, 2 = both blocks.
  auto step = [&](int j, auto masked, auto what) __attribute__((always_inline)) {
    constexpr int WHAT = decltype(what)::value;
    const int buf = j % NSTAGE;
    const bool more = j + NSTAGE - 1 < ntiles;
    if (more) {
      gload_k(j + NSTAGE - 1, (j + NSTAGE - 1) % NSTAGE);
      gload_v(j + NSTAGE - 1, (j + NSTAGE - 1) % NSTAGE);
    }
    auto nothing = []() __attribute__((always_inline)) {};
    const int kbase = j * BN;
    if constexpr (WHAT == 2)
      tile(masked, buf, kbase, nothing);
    else if constexpr (WHAT == 1)
      tile_hi(masked, buf, kbase, nothing);
    // Before the barrier, this wave's loads of tile j + 1 have landed: only
    // the four issued in this step may still be outstanding (none if it
    // issued none, or with two stages, where tile j + 1 is this step's).
    if (NSTAGE > 2 && more)
      __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };
  // The key loop in phases, one loop per variant of the tile code (a shared
  // loop makes the compiler keep copies of the accumulators).  Every wave
  // takes part in all ntiles barriers.
  using no = std::false_type;
  using yes = std::true_type;
  // The kernels without first_ref (d 64 and 128, no window, no key split)
  // take the first tile's row max once, before the key loop: its scores
  // (masked, which is exact for any tile) from LDS stage 0, where the
  // prologue has put the workgroup's first tile.  The loop's first tile then
  // passes the accept test with the same weights the exact path would form,
  // for 8 MFMAs a block instead of that path's 16 (bit-identical results),
  // and the loop itself is unchanged.
  if constexpr (!kFirstRef) {
    if (jlo < ntiles) {
#pragma unroll
      for (int qi = PAIRS ? 1 : 0; qi < QB; ++qi) {
        f32x16 sv[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sv[kb] = scores(yes{}, qi, 0, jlo * BN, kb);
        set_ref(qi, sv);
      }
    }
  }
  const int nfull = min(n_eff / BN, ntiles);  // tiles inside the valid keys
  int j = jlo;
  if (PAIRS) {
    // This wave's block [r0, r0 + 32): pairs with both tiles fully visible,
    // then the pairs its diagonal (or the key length) crosses, masked, then
    // nothing.  Every wave takes part in all S steps.
    static_assert(NSTAGE == 2, "pair loads and waits assume two stages");
    const int S = (ntiles + 1) / 2;
    int s_full = 0, s_vis = 0, vis_end = 0;
    if (wave_active) {
      const int r0 = row0[1];
      // past the last tile a row sees; tiles below unm_end: all rows see all keys
      vis_end = (n_eff + BN - 1) / BN;
      int unm_end = n_eff / BN;
      if (CAUSAL) {
        vis_end = min(vis_end, (r0 + 31) / BN + 1);
        unm_end = min(unm_end, (r0 + 1) / BN);
      }
      s_full = min(max(unm_end, 0) / 2, S);
      s_vis = min(max((vis_end + 1) / 2, s_full), S);
    }
    int s = 0;
    for (; s < s_full; ++s) pair_step(s, no{}, std::integral_constant<int, 2>{});
    for (; s < s_vis; ++s) {
      if (2 * s + 1 < vis_end)
        pair_step(s, yes{}, std::integral_constant<int, 2>{});
      else
        pair_step(s, yes{}, std::integral_constant<int, 1>{});
    }
    for (; s < S; ++s) pair_step(s, no{}, std::integral_constant<int, 0>{});
  } else if (WINDOW) {
    // This wave's phases over the workgroup's tiles [jlo, ntiles): nothing
    // up to a, masked up to ib, plain up to ie, masked up to z, nothing after.
    // Only its existing rows r0 .. rl count: rows past n_q are not stored.
    const int r0 = row0[0];
    int a = ntiles, ib = ntiles, ie = ntiles, z = ntiles;
    if (r0 < p.n_q) {
      const int rl = min(r0 + 63, p.n_q - 1);
      const int vis_lo = max(0, r0 - p.win_left);             // first key a row sees
      const int vis_hi = min(n_eff, rl + p.win_right + 1);    // one past the last
      if (vis_hi > vis_lo) {
        const int in_lo = max(0, rl - p.win_left);            // keys every row sees
        const int in_hi = min(n_eff, r0 + p.win_right + 1);
        a = min(max(vis_lo / BN, jlo), ntiles);
        z = min(max((vis_hi + BN - 1) / BN, a), ntiles);
        ib = min(max((in_lo + BN - 1) / BN, a), z);
        ie = min(max(in_hi / BN, ib), z);
      }
    }
    for (; j < a; ++j) step(j, no{}, std::integral_constant<int, 0>{});
    for (; j < ib; ++j) step(j, yes{}, std::integral_constant<int, 2>{});
    for (; j < ie; ++j) step(j, no{}, std::integral_constant<int, 2>{});
    for (; j < z; ++j) step(j, yes{}, std::integral_constant<int, 2>{});
    for (; j < ntiles; ++j) step(j, no{}, std::integral_constant<int, 0>{});
  } else if (SPLIT) {
    // this wave's tiles j = wave + t·NW through its own ring: the loads of
    // tile t + NSTAGE − 1 go out at the top of step t (K) and mid-tile (V)
    // into the stage that step t − 1 read; the step ends with this wave's
    // own wait for tile t + 1 (no barrier)
    auto split_step = [&](int t, auto masked) __attribute__((always_inline)) {
      const int jt = wave + t * NW;
      const int ta = t + NSTAGE - 1;
      const bool more = ta < myn;
      if (more) gload_k(wave + ta * NW, ta % NSTAGE);
      auto load_v = [&]() __attribute__((always_inline)) {
        if (more) gload_v(wave + ta * NW, ta % NSTAGE);
      };
      tile_hi(masked, t % NSTAGE, jt * BN, load_v);
      if (more)
        __builtin_amdgcn_s_waitcnt(kSplitWait);  // tiles t + 2 .. ta may be out
      else
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    };
    int t = 0;
    for (; wave + t * NW < nfull; ++t) split_step(t, no{});
    for (; wave + t * NW < ntiles; ++t) split_step(t, yes{});
  } else if (!CAUSAL) {
    for (; j < nfull; ++j) step(j, no{}, std::integral_constant<int, 2>{});
    for (; j < ntiles; ++j) step(j, yes{}, std::integral_constant<int, 2>{});
  } else {
    // per block: the first tile that needs the mask, the last with a
    // visible key (an upper block past the last query row has none)
    int fm[QB], lt[QB];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
      fm[qi] = min((row0[qi] + 1) / BN, nfull);
      lt[qi] = min((row0[qi] + 31) / BN, ntiles - 1);
    }
    if (row0[1] >= p.n_q) lt[1] = -1;
    int end_a = 0, end_b = 0, end_c = 0, end_d = 0;
    if (wave_active) {
      end_a = min(fm[0], fm[1]);            // both blocks, no mask
      end_b = max(end_a, lt[0] + 1);        // both, masked: up to block 0's diagonal
      end_c = max(end_b, fm[1]);            // block 1 only, no mask
      end_d = max(end_c, lt[1] + 1);        // block 1 only, masked
    }
    for (; j < end_a; ++j) step(j, no{}, std::integral_constant<int, 2>{});
    for (; j < end_b; ++j) step(j, yes{}, std::integral_constant<int, 2>{});
    for (; j < end_c; ++j) step(j, no{}, std::integral_constant<int, 1>{});
    for (; j < end_d; ++j) step(j, yes{}, std::integral_constant<int, 1>{});
    for (; j < ntiles; ++j) step(j, no{}, std::integral_constant<int, 0>{});
  }

  if constexpr (SPLIT) {
    // Merge the NW partial results of the block.  Every wave is past its last
    // LDS access (its own wait) once the barrier passes, so the rings hold the
    // exchange, lane-contiguous: per wave 16·NDB output values in the V
    // rings, reference value and row sum in the K rings.
    constexpr int NO = 16 * NDB;
    static_assert(NW * NO * 64 * 4 <= (int)sizeof(Vs) && NW * 2 * 64 * 4 <= (int)sizeof(Ks),
                  "exchange area");
    float* xo = (float*)&Vs[0][0][0];
    float* xm = (float*)&Ks[0][0][0];
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xo[((wave * NO) + 16 * db + i) * 64 + lane] = o[1][db][i];
    // a wave that had no tile has no reference value
    xm[(wave * 2) * 64 + lane] = m[1] == -INFINITY ? -INFINITY : mc[1];
    xm[(wave * 2 + 1) * 64 + lane] = l[1];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, xm[(w * 2) * 64 + lane]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[1][db] = f32x16{};
    l[1] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = xm[(w * 2) * 64 + lane];
      const float sw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      l[1] += sw * xm[(w * 2 + 1) * 64 + lane];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[1][db][i] += sw * xo[((w * NO) + 16 * db + i) * 64 + lane];
    }
  }

  // ---- normalise and store this lane's query row (4 consecutive d per store)
#pragma unroll
  for (int qi = (SPLIT || PAIRS) ? 1 : 0; qi < QB; ++qi) {
    const float L = pair_sum(l[qi]);
    const int row = row0[qi] + l32;
    bool visible = n_eff > 0;  // (causal: key 0 is visible to every row)
    if constexpr (WINDOW) visible = min(n_eff, row + p.win_right + 1) > max(0, row - p.win_left);
    const float inv = row_sum_inverse(L, visible);
    if (wave_active && row < p.n_q) {
      uint16_t* orow = Og + (int64_t)row * p.o_sr;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          if (db * 32 + gp * 16 >= D) continue;  // D = 16: the padding rows of Oᵀ
          u32x2 w[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int g = 2 * gp + e;
            w[e] = u32x2{pack2<DT>(o[qi][db][4 * g] * inv, o[qi][db][4 * g + 1] * inv),
                         pack2<DT>(o[qi][db][4 * g + 2] * inv, o[qi][db][4 * g + 3] * inv)};
          }
          *(u32x4*)(orow + db * 32 + gp * 16 + 8 * hi) = row_pair_pieces(w[0], w[1], hi);
        }
    }
  }
}

}  // namespace

}  // namespace mha
