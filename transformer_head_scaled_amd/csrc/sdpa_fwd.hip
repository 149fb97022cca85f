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

__device__ __forceinline__ int swz16(int k) {
  // position of key offset k inside the permuted Vᵀ row: swap bits 2 and 3
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int N>
struct RowVec;  // N 16-bit values as one global/LDS word
template <>
struct RowVec<2> {
  typedef uint32_t T;
  static __device__ __forceinline__ uint32_t get(T v, int dd) { return (v >> (16 * dd)) & 0xFFFFu; }
};
template <>
struct RowVec<4> {
  typedef u32x2 T;
  static __device__ __forceinline__ uint32_t get(T v, int dd) {
    return (v[dd >> 1] >> (16 * (dd & 1))) & 0xFFFFu;
  }
};
template <>
struct RowVec<8> {
  typedef u32x4 T;
  static __device__ __forceinline__ uint32_t get(T v, int dd) {
    return (v[dd >> 1] >> (16 * (dd & 1))) & 0xFFFFu;
  }
};

// One workgroup: NW waves, each owning QB blocks of 32 query rows (BM = 32·QB·NW
// rows of one (batch, head)); key/value tiles of BN keys, double-buffered in LDS.
template <int DT, bool CAUSAL, int BN, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_kernel(SdpaArgs p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32 * QB;
  constexpr int KST = D + 8;   // LDS row stride of K (elements): 144 B, conflict-free 16-B reads
  constexpr int VST = BN + 8;  // LDS row stride of Vᵀ
  constexpr int NKB = BN / 32;
  constexpr int KCH = BN * D / 8 / NT;  // 16-byte K chunks per thread
  constexpr int VD = BN / (4 * NW);     // d values per thread per key row (4 keys per thread)
  static_assert(KCH >= 1 && KCH * 8 * NT == BN * D, "K tile shape");
  static_assert((VD == 2 || VD == 4 || VD == 8) && VD * 4 * NT == BN * D, "V tile shape");
  typedef typename RowVec<VD>::T vrow_t;

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

  // ---- global -> register -> LDS staging of one K/V tile
  u32x4 kreg[KCH];
  vrow_t vreg[4];
  constexpr int DG = D / VD;  // threads per key group along d
  const int v_dq = tid % DG, v_kg = tid / DG;

  auto gload = [&](int tile) {
    const int kb0 = tile * BN;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + r * NT;
      const int key = kb0 + (ch >> 3);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < n_eff) v = *(const u32x4*)(Kg + (int64_t)key * p.k_sr + (ch & 7) * 8);
      kreg[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb0 + v_kg * 4 + r;
      vrow_t v = {};
      if (key < n_eff) v = *(const vrow_t*)(Vg + (int64_t)key * p.v_sr + v_dq * VD);
      vreg[r] = v;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + r * NT;
      *(u32x4*)&Ks[buf][(ch >> 3) * KST + (ch & 7) * 8] = kreg[r];
    }
    const int pos = (v_kg * 4 & ~15) | swz16(v_kg * 4 & 15);
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) {
      const uint32_t e0 = RowVec<VD>::get(vreg[0], dd), e1 = RowVec<VD>::get(vreg[1], dd);
      const uint32_t e2 = RowVec<VD>::get(vreg[2], dd), e3 = RowVec<VD>::get(vreg[3], dd);
      *(u32x2*)&Vt[buf][(v_dq * VD + dd) * VST + pos] = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
  };

  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const int kbase = j * BN;
    const bool wave_live = !CAUSAL || kbase <= wave_q_last;
    if (wave_live) {
      const uint16_t* Kb = &Ks[buf][l32 * KST + hi * 8];
      const uint16_t* Vb = &Vt[buf][l32 * VST + hi * 8];
      // ---- Sᵀ = K·Qᵀ for BN keys × 32·QB queries
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

      const bool need_mask = (kbase + BN > n_eff) || (CAUSAL && kbase + BN - 1 > wave_q_first);
      uint32_t pk[QB][NKB][8];  // P rounded to the input dtype, packed in pairs
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        const int row = wave_q_first + qi * 32 + l32;
        if (need_mask) {
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
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
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
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][kb][i], c, -mc));
            if (need_mask) e = (s[qi][kb][i] == -INFINITY) ? 0.f : e;
            pv[i] = e;
            rs += e;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) pk[qi][kb][i] = pack2<DT>(pv[2 * i], pv[2 * i + 1]);
        }
        l[qi] += rs;
      }

      // ---- Oᵀ += Vᵀ·Pᵀ
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const u32x4 a = *(const u32x4*)(Vb + db * 32 * VST + kb * 32 + t2 * 16);
#pragma unroll
            for (int qi = 0; qi < QB; ++qi) {
              const u32x4 bv = {pk[qi][kb][4 * t2 + 0], pk[qi][kb][4 * t2 + 1],
                                pk[qi][kb][4 * t2 + 2], pk[qi][kb][4 * t2 + 3]};
              o[qi][db] = mfma_32x32x16<DT>(a, bv, o[qi][db]);
            }
          }
        }
      }
    }
    if (j + 1 < ntiles) swrite(buf ^ 1);
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

template <int DH>
hipError_t launch_f32(const SdpaArgs& a, float scale, int causal, hipStream_t st) {
  dim3 grid((unsigned)((a.n_q + 63) / 64), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((sdpa_f32_kernel<DH>), grid, dim3(64), 0, st, a, scale, causal);
  return hipGetLastError();
}

}  // namespace

int sdpa_rows_per_workgroup(int dtype) { return dtype == DT_F32 ? 64 : kSdpaNW * 32 * kSdpaQB; }

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
  if (dtype == DT_BF16)
    return causal ? launch_mfma<DT_BF16, true, kSdpaBN, kSdpaQB, kSdpaNW>(a, st)
                  : launch_mfma<DT_BF16, false, kSdpaBN, kSdpaQB, kSdpaNW>(a, st);
  return causal ? launch_mfma<DT_F16, true, kSdpaBN, kSdpaQB, kSdpaNW>(a, st)
                : launch_mfma<DT_F16, false, kSdpaBN, kSdpaQB, kSdpaNW>(a, st);
}

}  // namespace mha
