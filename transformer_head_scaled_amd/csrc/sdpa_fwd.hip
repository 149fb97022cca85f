// Fused scaled dot-product attention forward for gfx950 (bf16 / fp16).
//
// Computes, per (batch, head), O = softmax(scale · Q·Kᵀ) · V with the
// causal mask (key c visible to query r iff c <= r) and/or a per-batch
// valid key length -- eq. (1) of "Lire « Attention Is All You Need »"
// (nickwang.xyz), §3.2.1, with the decoder mask of "Trois usages de
// l'attention dans le modèle" (forbidden scores set to -inf before the
// softmax).  The n_q × n_k score matrix is never formed: key/value tiles
// stream through LDS and an online softmax (running max m and sum l per
// query row, fp32) rescales the fp32 output accumulator.
//
// Work decomposition.  One workgroup = 4 waves x 64 query rows (two blocks
// of 32) of one (batch, head); 64-key K/V tiles pass through a 3-stage LDS
// ring.  Scores are formed transposed, Sᵀ = K·Qᵀ, with the 32x32x16 MFMA:
// K is the A operand (rows = keys, read from LDS), Q the B operand
// (columns = queries, kept in registers for the whole kernel).  In the
// MFMA result layout every lane then holds 16 scores of ONE query row (its
// column), the other 16 of that row sitting in lane l^32 -- so a row max
// needs a single cross-lane exchange (v_permlane32_swap).
//
// The output is formed transposed too, Oᵀ = Vᵀ·Pᵀ: P (rounded to the
// input dtype) is the B operand and comes straight out of the Sᵀ result
// registers.  Those registers hold, for lane half h, the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key step rather than 8 consecutive
// keys; the contraction order is free, so Vᵀ is staged into LDS transposed
// with the keys of every 16-group permuted the same way (bits 2 and 3 of
// the key offset swapped) and each lane reads its 8 values with one
// 16-byte load.  In the Oᵀ result each lane again holds its own query row,
// so a rescale of a row of O is a plain per-lane multiply.
//
// Softmax without a per-tile max.  The reference value m of a row only has
// to keep the weights finite: with weights p = exp2(s·c − m·c) the softmax
// is the same for every m.  A tile is first exponentiated against the
// current m; as long as each lane's partial row sum stays ≤ 2^8 (so every
// weight is ≤ 2^8) the tile is accepted as is.  Otherwise -- and on the
// first tile of a wave -- the wave takes the exact path: row max, new m,
// rescale of O and l by exp2((m_old − m_new)·c), and the weights again.
// The row sums are accumulated from the rounded weights (one dot2 per pair),
// the same values P·V uses.
//
// Loads.  K and V are read with buffer loads whose range ends at the valid
// key length, so rows past it read as 0 without per-lane branches: whatever
// the memory there holds -- NaN included -- has no effect, matching the
// reading that a masked key has weight exactly 0.  Causal tiles entirely
// above the diagonal are never loaded, tiles a whole wave cannot see are
// skipped by that wave, and only the diagonal and key-length boundary tiles
// evaluate the per-element mask.

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

// Sum of the two half-precision weights packed in `w` added to acc (fp32).
template <int DT>
__device__ __forceinline__ float dot2_sum(uint32_t w, float acc) {
  if constexpr (DT == DT_BF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  }
}

template <int DT, bool CAUSAL>
__global__ __launch_bounds__(256) void sdpa_fwd_kernel(SdpaArgs p) {
  constexpr int NW = 4, QB = 2, BN = 64, NSTAGE = 3;
  constexpr int BM = NW * 32 * QB;  // 256 query rows
  constexpr int KST = D + 8;        // K tile: [key][KST], 144-byte rows
  constexpr int VST = BN + 8;       // Vᵀ tile: [d][VST], 144-byte rows, permuted keys
  constexpr float kAccept = 256.f;  // accept a tile while partial row sums are <= 2^8

  __shared__ __attribute__((aligned(16))) uint16_t Ks[NSTAGE][BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[NSTAGE][D * VST];

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
  const int wave_q_first = q0 + wave * QB * 32;
  const int wave_q_last = wave_q_first + QB * 32 - 1;

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;
  // buffer resources covering exactly the valid keys of this (batch, head)
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, (int)((int64_t)n_eff * p.k_sr * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, (int)((int64_t)n_eff * p.v_sr * 2), 0x00020000);

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
  float m[QB], l[QB], mc[QB];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    o[qi][0] = f32x16{};
    o[qi][1] = f32x16{};
    m[qi] = -INFINITY;
    l[qi] = 0.f;
    mc[qi] = 0.f;
  }
  const float c = p.c;

  // ---- staging: K as is (two 16-byte chunks per thread), V transposed
  // (4 keys x 4 d per thread, written as four 8-byte runs along the keys)
  u32x4 kreg[2];
  u32x2 vreg[4];
  const int v_dq = tid & 15, v_kg = tid >> 4;
  const uint32_t k_off0 = (uint32_t)(((tid >> 3) * p.k_sr + (tid & 7) * 8) * 2);
  const uint32_t k_off1 = (uint32_t)((((tid + 256) >> 3) * p.k_sr + (tid & 7) * 8) * 2);
  const uint32_t v_off = (uint32_t)(((v_kg * 4) * p.v_sr + v_dq * 4) * 2);
  const uint32_t k_tile = (uint32_t)(BN * p.k_sr * 2), v_tile = (uint32_t)(BN * p.v_sr * 2);
  const uint32_t v_row = (uint32_t)(p.v_sr * 2);

  auto gload = [&](int tile) {
    kreg[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, k_off0 + tile * k_tile, 0, 0));
    kreg[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, k_off1 + tile * k_tile, 0, 0));
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vreg[r] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, v_off + tile * v_tile + r * v_row, 0, 0));
  };
  auto swrite = [&](int stage) {
    *(u32x4*)&Ks[stage][(tid >> 3) * KST + (tid & 7) * 8] = kreg[0];
    *(u32x4*)&Ks[stage][((tid + 256) >> 3) * KST + (tid & 7) * 8] = kreg[1];
    const int pos = (v_kg * 4 & ~15) | swz16(v_kg * 4 & 15);
    uint16_t* vt = &Vt[stage][(v_dq * 4) * VST + pos];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      // d = 4·v_dq + 2·h2 (low halves) and + 1 (high halves)
      const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][h2], vreg[0][h2], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][h2], vreg[2][h2], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][h2], vreg[0][h2], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][h2], vreg[2][h2], 0x07060302u);
      *(u32x2*)(vt + (2 * h2) * VST) = u32x2{lo01, lo23};
      *(u32x2*)(vt + (2 * h2 + 1) * VST) = u32x2{hi01, hi23};
    }
  };

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
      const uint16_t* Kb = &Ks[buf][l32 * KST + hi * 8];
      const uint16_t* Vb = &Vt[buf][l32 * VST + hi * 8];
      // ---- Sᵀ = K·Qᵀ for 64 keys × 64 queries
      __builtin_amdgcn_s_setprio(1);
      f32x16 s[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const u32x4 a = *(const u32x4*)(Kb + kb * 32 * KST + st * 16);
#pragma unroll
          for (int qi = 0; qi < QB; ++qi)
            s[qi][kb] = mfma_32x32x16<DT>(a, qf[qi][st], st == 0 ? f32x16{} : s[qi][kb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);

      // only the diagonal tile (causal) and the key-length boundary tile
      // need the per-element mask
      const bool need_mask = (kbase + BN > n_eff) || (CAUSAL && kbase + BN - 1 > wave_q_first);
      if (need_mask) {
        // an opaque statement keeps the compiler from turning this uniform
        // branch into per-element selects on every tile
        asm volatile("");
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
          const int row = wave_q_first + qi * 32 + l32;
          // visible iff the register's key offset in the tile (a constant) < lim
          const int lim = (CAUSAL ? min(n_eff, row + 1) : n_eff) - kbase - 4 * hi;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
              s[qi][kb][i] = off < lim ? s[qi][kb][i] : -INFINITY;
            }
        }
      }

      uint32_t pk[QB][2][8];  // P rounded to the input dtype, packed in pairs
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        // weights against the current reference value
        auto weights = [&]() {
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][kb][2 * i], c, -mc[qi]));
              const float e1 =
                  __builtin_amdgcn_exp2f(__builtin_fmaf(s[qi][kb][2 * i + 1], c, -mc[qi]));
              pk[qi][kb][i] = pack2<DT>(e0, e1);
              rs = dot2_sum<DT>(pk[qi][kb][i], rs);
            }
          return rs;
        };
        float rs = weights();
        // accept unless a weight may exceed 2^8 (or is not finite), or the
        // row has no reference value yet; `!(rs <= kAccept)` is also true
        // for NaN
        const bool reject = (m[qi] == -INFINITY) || !(rs <= kAccept);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(reject) != 0, 0)) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qi][kb][i]);
          mx = pair_max(mx);
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
          rs = weights();
        }
        l[qi] += rs;
      }

      // ---- Oᵀ += Vᵀ·Pᵀ
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
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
      __builtin_amdgcn_s_setprio(0);
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

template <int DT, bool CAUSAL>
hipError_t launch_mfma(const SdpaArgs& a, hipStream_t st) {
  const int64_t nqb = (a.n_q + 255) / 256;
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_f32(const SdpaArgs& a, float scale, int causal, hipStream_t st) {
  dim3 grid((unsigned)((a.n_q + 63) / 64), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((sdpa_f32_kernel<DH>), grid, dim3(64), 0, st, a, scale, causal);
  return hipGetLastError();
}

}  // namespace

int sdpa_rows_per_workgroup(int dtype) { return dtype == DT_F32 ? 64 : 256; }

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
    return causal ? launch_mfma<DT_BF16, true>(a, st) : launch_mfma<DT_BF16, false>(a, st);
  return causal ? launch_mfma<DT_F16, true>(a, st) : launch_mfma<DT_F16, false>(a, st);
}

}  // namespace mha
