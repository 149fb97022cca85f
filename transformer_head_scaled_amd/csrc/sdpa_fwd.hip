// Fused scaled dot-product attention forward for gfx950 (bf16 / fp16).
//
// Computes, per (batch, head), O = softmax(scale · Q·Kᵀ) · V with the
// causal mask (key c visible to query r iff c <= r) and/or a per-batch
// valid key length -- eq. (1) of "Lire « Attention Is All You Need »"
// (nickwang.xyz), §3.2.1, with the decoder mask of §3.2.3 ("Trois usages
// de l'attention dans le modèle": forbidden scores set to -inf before the
// softmax).  The n_q × n_k score matrix is never formed: key/value tiles
// stream through LDS and an online softmax (running max m and sum l per
// query row, fp32) rescales the fp32 output accumulator.
//
// Work decomposition.  One workgroup = 4 waves = BM = 4·32·QB query rows of
// one (batch, head).  Each wave owns QB blocks of 32 query rows.  Scores
// are formed transposed, Sᵀ = K·Qᵀ, with the 32x32x16 MFMA: K is the A
// operand (rows = keys, read from LDS), Q the B operand (columns = queries,
// kept in registers for the whole kernel).  In the MFMA result layout every
// lane then holds 16 scores of ONE query row (its column), the other 16 of
// that row sitting in lane l^32 -- so the row max and row sum need a single
// cross-lane exchange (v_permlane32_swap) instead of a 32-lane reduction.
//
// The output is formed transposed too, Oᵀ = Vᵀ·Pᵀ: P (rounded to the
// input dtype) is the B operand and comes straight out of the Sᵀ result
// registers.  Those registers hold, for lane half h, the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key step rather than 8 consecutive
// keys; the contraction order is free, so Vᵀ is stored in LDS with the
// keys of every 16-group permuted the same way (bits 2 and 3 of the key
// offset swapped) and each lane reads its 8 values with one 16-byte load.
// In the Oᵀ result each lane again holds its own query row, so the
// per-row rescale by exp(m_old - m_new) is a plain per-lane multiply.
//
// Masking.  Causal tiles entirely above the diagonal are never loaded;
// tiles that a whole wave cannot see are skipped by that wave; only the
// diagonal tile and the key-length boundary tile evaluate the per-element
// mask.  Key rows at or beyond the valid length are zero-filled in LDS
// (never read from memory), so whatever they hold -- NaN included -- has
// no effect, matching the reading that a masked key has weight exactly 0.

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int D = 64;  // head dimension d_k = d_v handled by this kernel

// Position of key offset k (0..15) inside a 16-key group of a transposed
// Vᵀ row: bits 2 and 3 swapped, the order in which the score registers hold
// the keys (see the top of this file).
__device__ __forceinline__ int swz16(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}


// One workgroup: NW waves, each owning QB blocks of 32 query rows (BM = 32·QB·NW
// rows of one (batch, head)); key/value tiles of BN keys, double-buffered in LDS.
template <int DT, bool CAUSAL, int BN, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_kernel(SdpaArgs p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32 * QB;
  constexpr int KST = D + 8;  // LDS row stride of K and V (elements): 144 B, see below
  constexpr int NKB = BN / 32;
  constexpr int KCH = BN * D / 8 / NT;  // 16-byte chunks of K (and of V) per thread
  static_assert(KCH >= 1 && KCH * 8 * NT == BN * D, "tile shape");

  constexpr int NSTAGE = kSdpaStages;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NSTAGE][BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NSTAGE][BN * KST];

  const int nqb = (p.n_q + BM - 1) / BM;
  const uint32_t total = (uint32_t)nqb * p.B * p.H;
  const uint32_t t = xcd_remap(blockIdx.x, total);
  const int bh = t / nqb;
  int qb = t % nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int b = bh / p.H, hh = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  const int q0 = qb * BM;
  int kend = n_eff;
  if (CAUSAL) kend = min(kend, q0 + BM);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;

  const int wave_q_first = q0 + wave * QB * 32;
  const int wave_q_last = wave_q_first + QB * 32 - 1;

  // ---- Q fragments (B operand), resident for the whole kernel
  u32x4 qf[QB][4];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int row = wave_q_first + qi * 32 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < p.n_q) v = *(const u32x4*)(Qg + (int64_t)row * p.q_sr + s * 16 + hi * 8);
      qf[qi][s] = p.neg ? flip_signs(v) : v;
    }
  }

  f32x16 o[QB][2];
  float m[QB], l[QB];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    o[qi][0] = f32x16{};
    o[qi][1] = f32x16{};
    m[qi] = -INFINITY;
    l[qi] = 0.f;
  }
  const float c = p.c;
  const float thr = p.thr;  // lazy-rescale slack in raw score units

  // ---- global -> register -> LDS staging of one K/V tile (rows as they are
  // in memory; a 16-byte pad per row keeps both the 16-byte K reads and the
  // transposing V reads free of bank conflicts)
  u32x4 kreg[KCH], vreg[KCH];
  auto gload = [&](int tile) {
    const int kb0 = tile * BN;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + r * NT;
      const int key = kb0 + (ch >> 3);
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < n_eff) {
        kv = *(const u32x4*)(Kg + (int64_t)key * p.k_sr + (ch & 7) * 8);
        vv = *(const u32x4*)(Vg + (int64_t)key * p.v_sr + (ch & 7) * 8);
      }
      kreg[r] = kv;
      vreg[r] = vv;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + r * NT;
      *(u32x4*)&Ks[buf][(ch >> 3) * KST + (ch & 7) * 8] = kreg[r];
      *(u32x4*)&Vs[buf][(ch >> 3) * KST + (ch & 7) * 8] = vreg[r];
    }
  };

  // tiles 0 .. NSTAGE-2 are staged before the loop; iteration j loads tile
  // j + NSTAGE - 1 into the stage that tile j - 1 used
#pragma unroll
  for (int t0 = 0; t0 < NSTAGE - 1; ++t0)
    if (t0 < ntiles) {
      gload(t0);
      swrite(t0);
    }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j % NSTAGE;
    if (j + NSTAGE - 1 < ntiles) gload(j + NSTAGE - 1);
    const int kbase = j * BN;
    const bool wave_live = !CAUSAL || kbase <= wave_q_last;
    if (wave_live) {
      // Only the diagonal tile (causal) and the key-length boundary tile
      // need the per-element mask; every other tile skips it.
      const bool need_mask = (kbase + BN > n_eff) || (CAUSAL && kbase + BN - 1 > wave_q_first);
      const uint16_t* Kb = &Ks[buf][l32 * KST + hi * 8];
      // Vᵀ operand via ds_read_b64_tr_b16: within each 16-lane group, lane r
      // addresses row (r >> 2) of a 4-row block at column 4·(r & 3) and gets
      // back one column: the 4 rows' values at column r.  Lane l therefore
      // receives V[base + 0..3][d = l % 32] for a block starting at key
      // base = 4·(l / 32) (+ 8 for the upper half of the 8 elements).
      const int r16 = lane & 15;
      const uint16_t* Vb =
          &Vs[buf][(4 * hi + (r16 >> 2)) * KST + 16 * ((lane >> 4) & 1) + 4 * (r16 & 3)];
      // ---- Sᵀ = K·Qᵀ for BN keys × 32·QB queries
      if (kSdpaPrio) __builtin_amdgcn_s_setprio(1);
      f32x16 s[QB][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const u32x4 a = *(const u32x4*)(Kb + kb * 32 * KST + st * 16);
#pragma unroll
          for (int qi = 0; qi < QB; ++qi)
            s[qi][kb] = mfma_32x32x16<DT>(a, qf[qi][st], st == 0 ? f32x16{} : s[qi][kb]);
        }
      }

      if (kSdpaPrio) __builtin_amdgcn_s_setprio(0);
      uint32_t pk[QB][NKB][8];  // P rounded to the input dtype, packed in pairs
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        if (need_mask) {
          // an opaque statement keeps the compiler from turning this
          // uniform branch into per-element selects on every tile
          asm volatile("");
          const int row = wave_q_first + qi * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
              const bool vis = key < n_eff && (!CAUSAL || key <= row);
              s[qi][kb][i] = vis ? s[qi][kb][i] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qi][kb][i]);
        mx = pair_max(mx);
        // Lazy rescaling: the running max only moves when a row's new max
        // exceeds it by more than thr (weights then stay <= 2^8), and then
        // for the whole wave at once.  Any reference value gives the same
        // softmax; the rescale keeps O and l consistent with it exactly.
        const bool need = (m[qi] == -INFINITY) ? (mx != -INFINITY) : (mx > m[qi] + thr);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
          const float m_new = fmaxf(m[qi], mx);
          const float alpha =
              (m[qi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m[qi] - m_new) * c);
          m[qi] = m_new;
          l[qi] *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            o[qi][0][i] *= alpha;
            o[qi][1][i] *= alpha;
          }
        }
        const float mc = (m[qi] == -INFINITY ? 0.f : m[qi]) * c;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float pv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // masked scores are -inf and c > 0, so exp2 gives exactly 0
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][kb][i], c, -mc));
            pv[i] = e;
            rs += e;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) pk[qi][kb][i] = pack2<DT>(pv[2 * i], pv[2 * i + 1]);
        }
        l[qi] += rs;
      }

      // ---- Oᵀ += Vᵀ·Pᵀ
      if (kSdpaPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const uint16_t* vp = Vb + (kb * 32 + t2 * 16) * KST + db * 32;
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * KST));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            const u32x4 a = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
            for (int qi = 0; qi < QB; ++qi) {
              const u32x4 bv = {pk[qi][kb][4 * t2 + 0], pk[qi][kb][4 * t2 + 1],
                                pk[qi][kb][4 * t2 + 2], pk[qi][kb][4 * t2 + 3]};
              o[qi][db] = mfma_32x32x16<DT>(a, bv, o[qi][db]);
            }
          }
        }
      }
      if (kSdpaPrio) __builtin_amdgcn_s_setprio(0);
    }
    if (j + NSTAGE - 1 < ntiles) swrite((j + NSTAGE - 1) % NSTAGE);
    __syncthreads();
  }

  // ---- normalise and store this lane's query row (4 consecutive d per store)
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const float L = pair_sum(l[qi]);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int row = wave_q_first + qi * 32 + l32;
    if (row < p.n_q) {
      uint16_t* orow = Og + (int64_t)row * p.o_sr;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + g * 8 + hi * 4;
          const u32x2 w = {pack2<DT>(o[qi][db][4 * g] * inv, o[qi][db][4 * g + 1] * inv),
                           pack2<DT>(o[qi][db][4 * g + 2] * inv, o[qi][db][4 * g + 3] * inv)};
          *(u32x2*)(orow + d) = w;
        }
    }
  }
}

// Ping-pong variant.  Workgroup = 8 waves x 64 query rows = 512 rows of one
// (batch, head), key tiles of 32.  Waves w and w+4 share a SIMD; waves 0-3
// form group A and 4-7 group B.  Each loop iteration has two halves
// separated by a workgroup barrier; in every half one group issues only
// MFMAs (P·V of tile j-1, then the scores of tile j) while the other runs
// only VALU work (mask, row max, lazy rescale, exp2, row sums and rounding
// of P for its latest scores).  The roles swap each half, so on every SIMD
// one wave keeps the matrix core busy while the other keeps the vector ALUs
// busy.
//
// The MFMA half is written as inline assembly: all operand reads of a block
// are issued first and each MFMA waits only for its own operand, so LDS
// latency overlaps the matrix work instead of sitting between MFMAs.  Vᵀ is
// staged into LDS already transposed (key order permuted as described at
// the top of this file), making every operand a single 16-byte read.

#define MHA_MFMA_BF16 "v_mfma_f32_32x32x16_bf16 "
#define MHA_MFMA_F16 "v_mfma_f32_32x32x16_f16 "
// after a block's last MFMA: wait states before any other instruction may
// read its results or overwrite its operands
#define MHA_MFMA_DRAIN "s_nop 7\n s_nop 7\n s_nop 7\n"

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // the low 32 bits of a generic pointer into LDS are the LDS byte offset
  return (uint32_t)(uintptr_t)p;
}

// Sᵀ for two 32-row blocks against one 32-key K tile: four 16-byte K
// fragments (d steps of 16 at byte offsets 0, 32, 64, 96), eight MFMAs.
template <int DT>
__device__ __forceinline__ void pp_scores(uint32_t ka, const u32x4 (&q)[2][4], f32x16 (&s)[2]) {
  u32x4 f0, f1, f2, f3;
#define MHA_S_BLOCK(MF)                                                                       \
  asm volatile("s_waitcnt lgkmcnt(0)\n"                                                       \
               "ds_read_b128 %[f0], %[ka] offset:0\n"                                         \
               "ds_read_b128 %[f1], %[ka] offset:32\n"                                        \
               "ds_read_b128 %[f2], %[ka] offset:64\n"                                        \
               "ds_read_b128 %[f3], %[ka] offset:96\n"                                        \
               "s_waitcnt lgkmcnt(3)\n" MF "%[s0], %[f0], %[q00], 0\n" MF                      \
               "%[s1], %[f0], %[q10], 0\n"                                                    \
               "s_waitcnt lgkmcnt(2)\n" MF "%[s0], %[f1], %[q01], %[s0]\n" MF                  \
               "%[s1], %[f1], %[q11], %[s1]\n"                                                \
               "s_waitcnt lgkmcnt(1)\n" MF "%[s0], %[f2], %[q02], %[s0]\n" MF                  \
               "%[s1], %[f2], %[q12], %[s1]\n"                                                \
               "s_waitcnt lgkmcnt(0)\n" MF "%[s0], %[f3], %[q03], %[s0]\n" MF                  \
               "%[s1], %[f3], %[q13], %[s1]\n" MHA_MFMA_DRAIN                                 \
               : [s0] "=&v"(s[0]), [s1] "=&v"(s[1]), [f0] "=&v"(f0), [f1] "=&v"(f1),          \
                 [f2] "=&v"(f2), [f3] "=&v"(f3)                                               \
               : [ka] "v"(ka), [q00] "v"(q[0][0]), [q01] "v"(q[0][1]), [q02] "v"(q[0][2]),    \
                 [q03] "v"(q[0][3]), [q10] "v"(q[1][0]), [q11] "v"(q[1][1]),                  \
                 [q12] "v"(q[1][2]), [q13] "v"(q[1][3])                                       \
               : "memory")
  if constexpr (DT == DT_BF16)
    MHA_S_BLOCK(MHA_MFMA_BF16);
  else
    MHA_S_BLOCK(MHA_MFMA_F16);
#undef MHA_S_BLOCK
}

// O[qi][db] += Vᵀ fragment (t2, db) · P[qi][t2] for one 32-key tile; the
// fragment of 16-key step t2 and d block db sits at byte offset
// db·(32 rows · 80 B) + t2·32.
template <int DT>
__device__ __forceinline__ void pp_pv(uint32_t va, const u32x4 (&pk)[2][2], f32x16 (&o)[2][2]) {
  u32x4 f0, f1, f2, f3;
#define MHA_PV_BLOCK(MF)                                                                      \
  asm volatile("s_waitcnt lgkmcnt(0)\n"                                                       \
               "ds_read_b128 %[f0], %[va] offset:0\n"                                         \
               "ds_read_b128 %[f1], %[va] offset:2560\n"                                      \
               "ds_read_b128 %[f2], %[va] offset:32\n"                                        \
               "ds_read_b128 %[f3], %[va] offset:2592\n"                                      \
               "s_waitcnt lgkmcnt(3)\n" MF "%[o00], %[f0], %[p00], %[o00]\n" MF               \
               "%[o10], %[f0], %[p10], %[o10]\n"                                              \
               "s_waitcnt lgkmcnt(2)\n" MF "%[o01], %[f1], %[p00], %[o01]\n" MF               \
               "%[o11], %[f1], %[p10], %[o11]\n"                                              \
               "s_waitcnt lgkmcnt(1)\n" MF "%[o00], %[f2], %[p01], %[o00]\n" MF               \
               "%[o10], %[f2], %[p11], %[o10]\n"                                              \
               "s_waitcnt lgkmcnt(0)\n" MF "%[o01], %[f3], %[p01], %[o01]\n" MF               \
               "%[o11], %[f3], %[p11], %[o11]\n" MHA_MFMA_DRAIN                               \
               : [o00] "+v"(o[0][0]), [o01] "+v"(o[0][1]), [o10] "+v"(o[1][0]),               \
                 [o11] "+v"(o[1][1]), [f0] "=&v"(f0), [f1] "=&v"(f1), [f2] "=&v"(f2),          \
                 [f3] "=&v"(f3)                                                               \
               : [va] "v"(va), [p00] "v"(pk[0][0]), [p01] "v"(pk[0][1]), [p10] "v"(pk[1][0]), \
                 [p11] "v"(pk[1][1])                                                          \
               : "memory")
  if constexpr (DT == DT_BF16)
    MHA_PV_BLOCK(MHA_MFMA_BF16);
  else
    MHA_PV_BLOCK(MHA_MFMA_F16);
#undef MHA_PV_BLOCK
}

template <int DT, bool CAUSAL>
__global__ __launch_bounds__(512) void sdpa_fwd_pp_kernel(SdpaArgs p) {
  constexpr int BN = 32;
  constexpr int BM = 512;
  constexpr int KST = D + 8;   // K: [key][KST], 144-byte rows
  constexpr int VST = BN + 8;  // Vᵀ: [d][VST], 80-byte rows, permuted key order
  static_assert(D * VST * 2 == 5120 && 32 * VST * 2 == 2560, "PV block offsets");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VST];

  const int nqb = (p.n_q + BM - 1) / BM;
  const uint32_t total = (uint32_t)nqb * p.B * p.H;
  const uint32_t t = xcd_remap(blockIdx.x, total);
  const int bh = t / nqb;
  int qb = t % nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int b = bh / p.H, hh = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int grp = wave >> 2;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  const int q0 = qb * BM;
  const int wave_q_first = q0 + wave * 64;
  const int wave_q_last = wave_q_first + 63;
  int kend = n_eff;
  if (CAUSAL) kend = min(kend, q0 + BM);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  int nt_w = ntiles;  // tiles this wave computes
  if (CAUSAL) nt_w = min(ntiles, wave_q_last / BN + 1);

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;

  u32x4 qf[2][4];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int row = wave_q_first + qi * 32 + l32;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < p.n_q) v = *(const u32x4*)(Qg + (int64_t)row * p.q_sr + st * 16 + hi * 8);
      qf[qi][st] = p.neg ? flip_signs(v) : v;
    }
  }
  f32x16 o[2][2];
  float m[2], l[2], mc[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    o[qi][0] = f32x16{};
    o[qi][1] = f32x16{};
    m[qi] = -INFINITY;
    l[qi] = 0.f;
    mc[qi] = 0.f;
  }
  const float c = p.c;
  const float thr = p.thr;

  // Staging.  Group A's 256 threads bring in the K tile (one 16-byte chunk
  // each), group B's the V tile (4 keys x 2 d each, written transposed).
  const int lt = tid & 255;
  u32x4 kreg;
  uint32_t vreg[4];
  const int v_dq = lt & 31, v_kg = lt >> 5;  // d pair 2·v_dq, keys 4·v_kg .. +3
  auto gload = [&](int tile) {
    if (grp == 0) {
      const int key = tile * BN + (lt >> 3);
      kreg = u32x4{0u, 0u, 0u, 0u};
      if (key < n_eff) kreg = *(const u32x4*)(Kg + (int64_t)key * p.k_sr + (lt & 7) * 8);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = tile * BN + v_kg * 4 + r;
        vreg[r] = key < n_eff ? *(const uint32_t*)(Vg + (int64_t)key * p.v_sr + v_dq * 2) : 0u;
      }
    }
  };
  auto swrite = [&](int stage) {
    if (grp == 0) {
      *(u32x4*)&Ks[stage][(lt >> 3) * KST + (lt & 7) * 8] = kreg;
    } else {
      const int pos = (v_kg * 4 & ~15) | swz16(v_kg * 4 & 15);
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        const int sh = dd * 16;
        const uint32_t e0 = (vreg[0] >> sh) & 0xFFFFu, e1 = (vreg[1] >> sh) & 0xFFFFu;
        const uint32_t e2 = (vreg[2] >> sh) & 0xFFFFu, e3 = (vreg[3] >> sh) & 0xFFFFu;
        *(u32x2*)&Vt[stage][(v_dq * 2 + dd) * VST + pos] = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
      }
    }
  };

  const uint32_t k_lane = lds_addr(&Ks[0][l32 * KST + hi * 8]);
  const uint32_t v_lane = lds_addr(&Vt[0][l32 * VST + hi * 8]);
  constexpr uint32_t K_STAGE = BN * KST * 2, V_STAGE = D * VST * 2;

  f32x16 s[2];     // [row block] scores of the latest tile
  u32x4 pk[2][2];  // [row block][16-key step] P of the latest softmaxed tile

  auto mfma_phase = [&](int j) {
    if (j >= 1 && j - 1 < nt_w) pp_pv<DT>(v_lane + ((j - 1) & 1) * V_STAGE, pk, o);
    if (j < nt_w) pp_scores<DT>(k_lane + (j & 1) * K_STAGE, qf, s);
  };

  // VALU half: softmax of tile j's scores into P
  auto valu_phase = [&](int j) {
    if (j < 0 || j >= nt_w) return;
    const int kbase = j * BN;
    const bool need_mask = (kbase + BN > n_eff) || (CAUSAL && kbase + BN - 1 > wave_q_first);
    if (need_mask) {
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        const int row = wave_q_first + qi * 32 + l32;
        // visible iff the register's key offset in the tile (a constant)
        // is below lim
        const int lim = (CAUSAL ? min(n_eff, row + 1) : n_eff) - kbase - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          s[qi][i] = off < lim ? s[qi][i] : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qi][i]);
      mx = pair_max(mx);
      const bool need = (m[qi] == -INFINITY) ? (mx != -INFINITY) : (mx > m[qi] + thr);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
        const float m_new = fmaxf(m[qi], mx);
        const float alpha =
            (m[qi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m[qi] - m_new) * c);
        m[qi] = m_new;
        mc[qi] = (m_new == -INFINITY ? 0.f : m_new) * c;
        l[qi] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o[qi][0][i] *= alpha;
          o[qi][1][i] *= alpha;
        }
      }
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][2 * i], c, -mc[qi]));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][2 * i + 1], c, -mc[qi]));
        rs += e0;
        rs += e1;
        pk[qi][i >> 2][i & 3] = pack2<DT>(e0, e1);
      }
      l[qi] += rs;
    }
  };

  // prologue: tile 0 of K
  if (grp == 0 && ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  // Each group runs its own copy of the loop (same number of barriers), so
  // the register allocator never has to keep both groups' live sets at once.
  if (grp == 0) {
    for (int j = 0; j <= ntiles; ++j) {
      const bool stage = j + 1 < ntiles;  // K of tile j+1
      if (stage) gload(j + 1);
      mfma_phase(j);
      __syncthreads();
      valu_phase(j);
      if (stage) swrite((j + 1) & 1);
      __syncthreads();
    }
  } else {
    for (int j = 0; j <= ntiles; ++j) {
      const bool stage = j < ntiles;  // V of tile j
      if (stage) gload(j);
      valu_phase(j - 1);
      __syncthreads();
      mfma_phase(j);
      if (stage) swrite(j & 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const float L = pair_sum(l[qi]);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int row = wave_q_first + qi * 32 + l32;
    if (row < p.n_q) {
      uint16_t* orow = Og + (int64_t)row * p.o_sr;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + g * 8 + hi * 4;
          const u32x2 w = {pack2<DT>(o[qi][db][4 * g] * inv, o[qi][db][4 * g + 1] * inv),
                           pack2<DT>(o[qi][db][4 * g + 2] * inv, o[qi][db][4 * g + 3] * inv)};
          *(u32x2*)(orow + d) = w;
        }
    }
  }
}

// ---------------------------------------------------------------- fp32 path
//
// Plain fp32 attention for small problems and the 1e-5 parity case: one
// thread per query row, K/V tiles of 32 keys broadcast from LDS, online
// softmax.  Any head dimension in {16, 32, 64, 128}.  Inputs, weights and
// the output accumulator are fp32; the dot products, the running max and
// the exponent argument are formed in fp64, so the scores carry no fp32
// summation error even when they are large (an unscaled softmax), and the
// only fp32 roundings left are expf and the weighted sum of V.
template <int DH>
__global__ __launch_bounds__(64) void sdpa_f32_kernel(SdpaArgs p, float scale, int causal) {
  constexpr int TK = 32;
  __shared__ __attribute__((aligned(16))) float Ks[TK * DH];
  __shared__ __attribute__((aligned(16))) float Vs[TK * DH];
  const int b = blockIdx.z, hh = blockIdx.y;
  const int row = blockIdx.x * 64 + threadIdx.x;
  const float* Qg = (const float*)p.Q + b * p.q_sb + hh * p.q_sh;
  const float* Kg = (const float*)p.K + b * p.k_sb + hh * p.k_sh;
  const float* Vg = (const float*)p.V + b * p.v_sb + hh * p.v_sh;
  float* Og = (float*)p.O + b * p.o_sb + hh * p.o_sh;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  int kend = n_eff;
  if (causal) kend = min(kend, (int)(blockIdx.x + 1) * 64);
  const int ntiles = kend > 0 ? (kend + TK - 1) / TK : 0;

  float q[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = row < p.n_q ? Qg[(int64_t)row * p.q_sr + d] : 0.f;
    o[d] = 0.f;
  }
  double m = -INFINITY;
  float l = 0.f;

  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();
    for (int e = threadIdx.x; e < TK * DH / 4; e += 64) {
      const int key = j * TK + (e * 4) / DH, d = (e * 4) % DH;
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < n_eff) {
        kv = *(const float4*)(Kg + (int64_t)key * p.k_sr + d);
        vv = *(const float4*)(Vg + (int64_t)key * p.v_sr + d);
      }
      *(float4*)&Ks[e * 4] = kv;
      *(float4*)&Vs[e * 4] = vv;
    }
    __syncthreads();
    double s[TK];
    double mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      double acc = 0.0;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc = __builtin_fma((double)q[d], (double)Ks[k * DH + d], acc);
      const int key = j * TK + k;
      const bool vis = key < n_eff && (!causal || key <= row);
      s[k] = vis ? acc * (double)scale : -INFINITY;
      mx = fmax(mx, s[k]);
    }
    const double m_new = fmax(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf((float)(m - m_new));
    const double mu = m_new == -INFINITY ? 0.0 : m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] *= alpha;
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      const float e = s[k] == -INFINITY ? 0.f : expf((float)(s[k] - mu));
      l += e;
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] = __builtin_fmaf(e, Vs[k * DH + d], o[d]);
    }
    m = m_new;
  }
  if (row < p.n_q) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) Og[(int64_t)row * p.o_sr + d] = o[d] * inv;
  }
}

template <int DT, bool CAUSAL, int BN, int QB, int NW>
hipError_t launch_mfma(const SdpaArgs& a, hipStream_t st) {
  constexpr int BM = NW * 32 * QB;
  const int64_t nqb = (a.n_q + BM - 1) / BM;
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, CAUSAL, BN, QB, NW>), dim3((unsigned)grid), dim3(NW * 64),
                     0, st, a);
  return hipGetLastError();
}

template <int DT, bool CAUSAL>
hipError_t launch_pp(const SdpaArgs& a, hipStream_t st) {
  const int64_t nqb = (a.n_q + 511) / 512;
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_pp_kernel<DT, CAUSAL>), dim3((unsigned)grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_f32(const SdpaArgs& a, float scale, int causal, hipStream_t st) {
  dim3 grid((unsigned)((a.n_q + 63) / 64), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((sdpa_f32_kernel<DH>), grid, dim3(64), 0, st, a, scale, causal);
  return hipGetLastError();
}

}  // namespace

int sdpa_rows_per_workgroup(int dtype) {
  return dtype == DT_F32 ? 64 : kSdpaPingPong ? 512 : kSdpaNW * 32 * kSdpaQB;
}

hipError_t launch_sdpa(const SdpaArgs& a, int dtype, int causal, int d, float scale, hipStream_t st) {
  if (dtype == DT_F32) {
    switch (d) {
      case 16: return launch_f32<16>(a, scale, causal, st);
      case 32: return launch_f32<32>(a, scale, causal, st);
      case 64: return launch_f32<64>(a, scale, causal, st);
      case 128: return launch_f32<128>(a, scale, causal, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (d != D) return hipErrorInvalidValue;
  if constexpr (kSdpaPingPong) {
    if (dtype == DT_BF16)
      return causal ? launch_pp<DT_BF16, true>(a, st) : launch_pp<DT_BF16, false>(a, st);
    return causal ? launch_pp<DT_F16, true>(a, st) : launch_pp<DT_F16, false>(a, st);
  } else {
    if (dtype == DT_BF16)
      return causal ? launch_mfma<DT_BF16, true, kSdpaBN, kSdpaQB, kSdpaNW>(a, st)
                    : launch_mfma<DT_BF16, false, kSdpaBN, kSdpaQB, kSdpaNW>(a, st);
    return causal ? launch_mfma<DT_F16, true, kSdpaBN, kSdpaQB, kSdpaNW>(a, st)
                  : launch_mfma<DT_F16, false, kSdpaBN, kSdpaQB, kSdpaNW>(a, st);
  }
}

}  // namespace mha
