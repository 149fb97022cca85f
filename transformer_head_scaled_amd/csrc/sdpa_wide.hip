// Scaled dot-product attention for wide heads, d = 256 and 512 (bf16 /
// fp16): eq. (1) of "Lire « Attention Is All You Need »" (nickwang.xyz),
// §3.2.1, for the head sizes of its Table 3 row (A) with few heads
// (d_model 512 with h = 1 gives d_k = d_v = 512).
//
// One 32-row query block per group of 4 waves, the head dimension split
// across the waves: wave w owns columns [w·D/4, (w+1)·D/4) of Q, K, V and O.
// Unmasked, a workgroup holds two such groups on consecutive blocks, which
// share every staged K/V tile (RS = 2); causal at d = 512, two groups
// share one block and split its key tiles (KS = 2).
// The output accumulator of a block at d = 512 would need 256 registers
// per lane in one wave; split four ways it needs 64.  The scores need the
// whole contraction over d, so per 32-key tile each wave forms the partial
// Sᵀ over its columns (MFMA, as in the d <= 128 kernel: Sᵀ = K·Qᵀ, one
// query row per lane), the four partials are added through LDS (each wave
// adds them in the same order, so all four hold the same scores), every
// wave runs the same softmax step on them, and each wave accumulates its own
// columns of Oᵀ = Vᵀ·Pᵀ.  K and V tiles of 32 keys go straight from memory
// into one LDS buffer each (buffer loads with an LDS destination, one 1 KB
// row piece per instruction at d = 512), K and V loads staggered so that
// each lands while the other half of the tile is computed; their 16-byte chunks are permuted
// by key bits as in the d = 128 layout, so the fragment reads spread over
// all banks.  Causal tiles past the block's diagonal are not computed and
// rows past the key length read as zero; only the tiles that hold a masked
// key for some row of the block evaluate the per-element mask (and check
// their values for NaN/inf, which a zero weight would not cancel inside
// the matrix product).  The softmax
// has no per-tile max, as in the d <= 128 kernel: a tile's weights are
// formed against the row's current reference value and accepted while each
// lane's partial row sum stays <= 2^8; otherwise (and on the first tile)
// the tile's row max sets a new reference and O and l are rescaled.  The
// four waves hold the same scores, so they take the same path.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

// KS key groups of NW waves: KS = 2 splits a block's key tiles between two
// groups (even and odd tiles), each with its own LDS buffers, and merges the
// two partial results at the end.  RS row groups: RS = 2 gives the
// workgroup two consecutive 32-row blocks, one per group of NW waves, which
// share every staged K and V tile (half the tile bytes per flop) and keep
// their own score exchange; both groups walk the same tiles and barriers.
template <int DT, int D, bool CAUSAL, int KS = 1, int RS = 1>
__global__ __launch_bounds__(256 * KS * RS) void sdpa_wide_kernel(SdpaArgs p) {
  static_assert(KS == 1 || RS == 1, "a key split or a row split, not both");
  constexpr int NW = 4, BN = 32;
  constexpr int DS = D / NW;         // columns per wave
  constexpr int NST = DS / 16;       // 16-deep MFMA steps of a partial score block
  constexpr int NDB = DS / 32;       // 32-row blocks of this wave's Oᵀ
  constexpr int CR = D / 8;          // 16-byte chunks per K/V row
  constexpr int PPR = CR / 64;       // 1 KB pieces per row (d = 512: 1; d = 256: 0 -> 2 rows per piece)
  static_assert(D == 256 || D == 512, "wide head dimension");

  // one K and one V tile: 80 KB in all at d = 512 (48 KB at d = 256), so
  // that two (three) workgroups share a compute unit
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KS][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KS][BN * D];
  // partial scores: lane l's 16 values as four 16-byte chunks, chunk c
  // stored at c ^ ((l >> 2) & 3) (the 16 lanes of a 16-byte access phase
  // then cover all 64 banks)
  __shared__ __attribute__((aligned(16))) float Sx[KS * RS][NW][64 * 16];
  constexpr float kAccept = 256.f;

  const int nqb = (p.n_q + 32 * RS - 1) / (32 * RS);
  const uint32_t nbh = (uint32_t)p.B * p.H;
  // causal: the highest blocks (most keys) first
  const int qb = CAUSAL ? nqb - 1 - (int)(blockIdx.x / nbh) : (int)(blockIdx.x / nbh);
  const int bh = (int)(blockIdx.x % nbh);
  const int b = bh / p.H, hh = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  // (the wave index within its key group: it selects the columns)
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = (KS == 1 && RS == 1) ? 0 : wave_all / NW;
  const int wave = (KS == 1 && RS == 1) ? wave_all : wave_all % NW;
  const int kvg = KS == 1 ? 0 : grp;  // this wave's K and V buffers
  const int l32 = lane & 31, hi = lane >> 5;
  const int row0 = qb * 32 * RS + (RS == 1 ? 0 : 32 * grp);

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  int kend = n_eff;
  if (CAUSAL) kend = min(kend, row0 + 32);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;  // this block's tiles
  // the workgroup's tiles (its highest block's, with the row split)
  int kend_wg = n_eff;
  if (CAUSAL) kend_wg = min(kend_wg, qb * 32 * RS + 32 * RS);
  const int ntiles_wg = RS == 1 ? ntiles : (kend_wg > 0 ? (kend_wg + BN - 1) / BN : 0);

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;
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

  // this wave's Q columns (B operand), resident
  u32x4 qf[NST];
  {
    const int row = row0 + l32;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < p.n_q) v = *(const u32x4*)(Qg + (int64_t)row * p.q_sr + wave * DS + st * 16 + hi * 8);
      qf[st] = p.neg ? flip_signs(v) : v;
    }
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f, mc = 0.f;
  const float c = p.c;
  // first key masked for some row of the block (the block's first row sees
  // keys up to itself)
  const int mask_from = CAUSAL ? min(n_eff, row0 + 1) : n_eff;
  const int sx_sw = (lane >> 2) & 3;

  // ---- staging: a tile is BN rows of D/8 16-byte chunks, chunk c of key k
  // stored at c ^ (k & 15) (K; the 16 keys of a fragment read phase then
  // cover the 16 bank groups of a 256-byte segment) and c ^ 4·(k & 3) (V;
  // a transposing read phase of 4 keys covers the four quarters).  Each
  // wave instruction fills 1 KB: lane i writes chunk position i of a row
  // (d = 512) or of one of two rows (d = 256).
  constexpr int PIECES = BN * D * 2 / 1024;  // 1 KB pieces per tile
  constexpr int CPW = PIECES / (NW * RS);  // pieces per wave and tile
  static_assert(PIECES % (NW * RS) == 0, "tile pieces per wave");
  const int lw = RS == 1 ? wave : wave_all;  // this wave's share of the loads
  auto piece_src = [&](int r, bool is_v) __attribute__((always_inline)) {
    const int key = (PPR >= 1) ? r : 2 * r + lane / CR;  // PPR >= 1: one row per piece
    const int pos = lane % CR;
    const int ch = is_v ? (pos ^ (4 * (key & 3))) : (pos ^ (key & 15));
    return (uint32_t)(((int64_t)key * (is_v ? p.v_sr : p.k_sr) + ch * 8) * 2);
  };
  auto gload_k = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int r = lw * CPW + i;
      load_lds_b128(krs,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&Ks[kvg][r * 512]),
                    piece_src(r, false) + (uint32_t)(tile * BN * p.k_sr * 2));
    }
  };
  auto gload_v = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int r = lw * CPW + i;
      load_lds_b128(vrs,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&Vs[kvg][r * 512]),
                    piece_src(r, true) + (uint32_t)(tile * BN * p.v_sr * 2));
    }
  };
  // K fragment st of this wave: key l32, chunk (wave·DS)/8 + 2·st + hi
  auto kfrag = [&](int st) __attribute__((always_inline)) {
    const int ch = (wave * DS) / 8 + 2 * st + hi;
    return *(const u32x4*)&Ks[kvg][l32 * D + ((ch ^ (l32 & 15)) * 8)];
  };
  // Vᵀ fragment (t2, db): d = wave·DS + db·32 + l32, keys of the 16-key step
  // t2 in the score-register order, two transposing reads of 4 keys
  const int i16 = lane & 15;
  const int v_key_l = 4 * hi + (i16 >> 2);
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
  auto vfrag = [&](int t2, int db) __attribute__((always_inline)) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = t2 * 16 + 8 * e + v_key_l;
      const int d = wave * DS + db * 32 + v_col;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)&Vs[kvg][key * D + (((d >> 3) ^ (4 * (key & 3))) * 8) + (d & 7)]);
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * e] = w[0];
      r[2 * e + 1] = w[1];
    }
    return r;
  };

  // partial Sᵀ over this wave's columns for the keys in LDS
  auto spart = [&]() __attribute__((always_inline)) {
    f32x16 sp = {};
#pragma unroll
    for (int st = 0; st < NST; ++st) sp = mfma_32x32x16<DT>(kfrag(st), qf[st], sp);
    return sp;
  };
  auto put_sx = [&](const f32x16& sp) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4*)&Sx[grp][wave][lane * 16 + 4 * (q ^ sx_sw)] =
          f32x4{sp[4 * q], sp[4 * q + 1], sp[4 * q + 2], sp[4 * q + 3]};
  };
  // the full scores: the four partials, added in wave order
  auto get_sx = [&]() __attribute__((always_inline)) {
    f32x16 s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int at = lane * 16 + 4 * (q ^ sx_sw);
      const f32x4 v = ((*(const f32x4*)&Sx[grp][0][at] + *(const f32x4*)&Sx[grp][1][at]) +
                       *(const f32x4*)&Sx[grp][2][at]) + *(const f32x4*)&Sx[grp][3][at];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * q + e] = v[e];
    }
    return s;
  };
  // mask, weights and softmax state of tile j; P (packed) into pw
  auto softmax = [&](f32x16& s, int j, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    if (j * BN + BN > mask_from) {
      // mask: key offset in the tile of register i is 8·(i / 4) + 4·hi + i % 4
      const int row = row0 + l32;
      const int lim = (CAUSAL ? min(n_eff, row + 1) : n_eff) - j * BN - 4 * hi;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 8 * (i >> 2) + (i & 3);
        if (off >= lim) s[i] = -INFINITY;
      }
    }
    auto weights = [&]() __attribute__((always_inline)) {
      float r0 = 0.f, r1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], c, -mc));
        pw[i] = pack2<DT>(e0, e1);
        r0 += e0;
        r1 += e1;
      }
      return r0 + r1;
    };
    float rs = weights();
    // `!(rs <= kAccept)` is also true for NaN
    const bool reject = (m == -INFINITY) || !(rs <= kAccept);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(reject) != 0, 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
      mc = (m_new == -INFINITY ? 0.f : m_new) * c;
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      rs = weights();
    }
    l += rs;
  };
  // this wave's columns of Oᵀ += Vᵀ·Pᵀ for the values in LDS.  In a masked
  // causal tile a NaN or ±inf value row would reach, through 0·x in the
  // matrix product, the rows of the block that do not see its key; those
  // tiles check the fragments (wave-uniform), and when such a value is
  // there they clear it for the product and add it afterwards to the rows
  // that see the key (a visible key's weight is positive).
  auto add_nonfinite_v = [&](int j) __attribute__((always_inline)) {
    const int row = row0 + l32;
    for (int k = 0; k < BN; ++k) {
      const int key = j * BN + k;
      if (!(key < n_eff && key <= row)) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = wave * DS + db * 32 + 8 * g + 4 * hi;
          const u32x2 w = *(const u32x2*)&Vs[kvg][k * D + (((d >> 3) ^ (4 * (k & 3))) * 8) + (d & 7)];
          const f32x4 x = unpack4<DT>(w);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!__builtin_isfinite(x[e])) o[db][4 * g + e] += x[e];
        }
    }
  };
  auto pv = [&](int j, const uint32_t (&pw)[8]) __attribute__((always_inline)) {
    if (CAUSAL && j * BN + BN > mask_from) {
      u32x4 vf[2][NDB];
      u16x2 acc = {0, 0};
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          vf[t2][db] = vfrag(t2, db);
#pragma unroll
          for (int w = 0; w < 4; ++w) acc = magnitude_max(acc, vf[t2][db][w]);
        }
      constexpr unsigned short lim = nonfinite_from<DT>();
      const bool vbad = __builtin_amdgcn_ballot_w64(acc[0] >= lim || acc[1] >= lim) != 0;
      if (vbad) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int w = 0; w < 4; ++w) vf[t2][db][w] = zero_nonfinite<DT>(vf[t2][db][w]);
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 bv = {pw[4 * t2], pw[4 * t2 + 1], pw[4 * t2 + 2], pw[4 * t2 + 3]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mfma_32x32x16<DT>(vf[t2][db], bv, o[db]);
      }
      if (vbad) add_nonfinite_v(j);
      return;
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const u32x4 bv = {pw[4 * t2], pw[4 * t2 + 1], pw[4 * t2 + 2], pw[4 * t2 + 3]};
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = mfma_32x32x16<DT>(vfrag(t2, db), bv, o[db]);
    }
  };

  // One K and one V buffer: K of tile j + 1 is loaded once every wave has
  // formed its partials of tile j (it lands during the softmax and P·V), V
  // of tile j + 1 once every wave is past P·V of tile j (it lands during
  // the partials and the exchange).  The other workgroups of the compute
  // unit fill the waits.  (Two stages of K and V, with or without forming
  // the next tile's partials during the softmax, measured 4-43 % slower:
  // they leave room for one workgroup less.)
  // group grp takes the tiles grp, grp + KS, ...; both groups run the same
  // number of steps (two workgroup barriers each), a group past its last
  // tile only taking part in the barriers
  const int niter = (ntiles_wg + KS - 1) / KS;
  const int j0 = KS == 1 ? 0 : grp;  // the first tile of this wave's key group
  if (j0 < ntiles_wg) {
    gload_k(j0);
    gload_v(j0);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  for (int it = 0; it < niter; ++it) {
    const int j = j0 + KS * it;
    const bool mine = j < ntiles;
    if (mine) put_sx(spart());
    // exchange writes visible, V(j) landed, every wave past its K reads
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (j + KS < ntiles_wg) gload_k(j + KS);
    if (mine) {
      f32x16 s = get_sx();
      uint32_t pw[8];
      softmax(s, j, pw);
      pv(j, pw);
    }
    // K(j + KS) landed, every wave past its V and exchange reads
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (j + KS < ntiles_wg) gload_v(j + KS);
  }

  if constexpr (KS == 2) {
    // Merge: group 1 leaves its reference value (m·c, -inf without a tile),
    // per-lane row sums and unnormalised columns in its LDS buffers; group 0
    // rescales both parts to the larger reference value (the rescale of the
    // online softmax) and adds them.  Every wave is past its last LDS read
    // (the loop ends with a barrier).
    constexpr int NO = 16 * NDB;
    static_assert(NW * NO * 64 * 4 <= (int)(sizeof(Ks[0]) + sizeof(Vs[0])) &&
                  NW * 2 * 64 * 4 <= (int)sizeof(Sx[0]), "merge area");
    float* xo = (float*)&Ks[1][0];  // then Vs[1] where Ks[1] is too small
    float* xm = &Sx[1][0][0];
    if (grp == 1) {
      if constexpr (NW * NO * 64 * 4 <= (int)sizeof(Ks[0])) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) xo[((wave * NO) + 16 * db + i) * 64 + lane] = o[db][i];
      } else {
        float* xv = (float*)&Vs[1][0];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int at = ((wave * NO) + 16 * db + i) * 64 + lane;
            constexpr int HALF = (int)sizeof(Ks[0]) / 4;
            if (at < HALF) xo[at] = o[db][i]; else xv[at - HALF] = o[db][i];
          }
      }
      xm[(wave * 2) * 64 + lane] = m == -INFINITY ? -INFINITY : mc;
      xm[(wave * 2 + 1) * 64 + lane] = l;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (grp == 1) return;
    const float m1 = xm[(wave * 2) * 64 + lane];
    const float m0 = m == -INFINITY ? -INFINITY : mc;
    const float M = fmaxf(m0, m1);
    const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    l = w0 * l + w1 * xm[(wave * 2 + 1) * 64 + lane];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int at = ((wave * NO) + 16 * db + i) * 64 + lane;
        constexpr int HALF = (int)sizeof(Ks[0]) / 4;
        float x1;
        if constexpr (NW * NO * 64 * 4 <= (int)sizeof(Ks[0])) {
          x1 = xo[at];
        } else {
          x1 = at < HALF ? xo[at] : ((float*)&Vs[1][0])[at - HALF];
        }
        o[db][i] = w0 * o[db][i] + w1 * x1;
      }
  }

  // normalise and store this wave's columns of the lane's row
  const float L = pair_sum(l);
  const float inv = row_sum_inverse(L, n_eff > 0);
  const int row = row0 + l32;
  if (row < p.n_q) {
    uint16_t* orow = Og + (int64_t)row * p.o_sr + wave * DS;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x2 w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int g = 2 * gp + e;
          w[e] = u32x2{pack2<DT>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                       pack2<DT>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        }
        *(u32x4*)(orow + db * 32 + gp * 16 + 8 * hi) = row_pair_pieces(w[0], w[1], hi);
      }
  }
}

template <int DT, int D>
hipError_t launch_d(const SdpaArgs& a, int causal, int waves, int rows, hipStream_t st) {
  const int64_t grid = (a.n_q + rows - 1) / rows * (int64_t)a.B * a.H;
  if (rows == 64) {  // the row split, unmasked only (the route's choice)
    if (causal || waves != 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((sdpa_wide_kernel<DT, D, false, 1, 2>), dim3((unsigned)grid), dim3(512), 0, st, a);
    return hipGetLastError();
  }
  if (rows != 32) return hipErrorInvalidValue;
  if constexpr (D >= SDPA_WIDE_SPLIT_MIN_D) {
    if (causal && waves == 8) {
      hipLaunchKernelGGL((sdpa_wide_kernel<DT, D, true, 2>), dim3((unsigned)grid), dim3(512), 0, st, a);
      return hipGetLastError();
    }
  }
  if (waves != 4)
    return hipErrorInvalidValue;
  else if (causal)
    hipLaunchKernelGGL((sdpa_wide_kernel<DT, D, true>), dim3((unsigned)grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((sdpa_wide_kernel<DT, D, false>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_wide(const SdpaArgs& a, int dtype, int causal, int d, int waves, int rows,
                            hipStream_t st) {
  if (a.window) return hipErrorInvalidValue;  // not offered for wide heads
  if (dtype == DT_BF16) {
    if (d == 256) return launch_d<DT_BF16, 256>(a, causal, waves, rows, st);
    if (d == 512) return launch_d<DT_BF16, 512>(a, causal, waves, rows, st);
  } else if (dtype == DT_F16) {
    if (d == 256) return launch_d<DT_F16, 256>(a, causal, waves, rows, st);
    if (d == 512) return launch_d<DT_F16, 512>(a, causal, waves, rows, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mha
