// Scaled dot-product attention: the fp32 kernel, the launchers of the flash
// kernel (sdpa_fwd_kernel.h) for the unmasked, causal and key-split forms,
// and the dispatch.  The restricted-window launches are in sdpa_window.hip.

#include "sdpa_fwd_kernel.h"

namespace mha {

namespace {

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
  int jlo = 0;  // restricted window: the keys the block's rows can reach
  if (p.window) {
    kend = min(kend, min((int)(blockIdx.x + 1) * 64, p.n_q) - 1 + p.win_right + 1);
    jlo = max(0, (int)blockIdx.x * 64 - p.win_left) / TK;
  }
  const int ntiles = kend > 0 ? (kend + TK - 1) / TK : 0;

  float q[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = row < p.n_q ? Qg[(int64_t)row * p.q_sr + d] : 0.f;
    o[d] = 0.f;
  }
  double m = -INFINITY;
  float l = 0.f;

  for (int j = jlo; j < ntiles; ++j) {
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
      const bool vis = key < n_eff && (!causal || key <= row) &&
                       (!p.window || (key >= row - p.win_left && key <= row + p.win_right));
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
      // a masked key is skipped outright (not added with weight 0), so the
      // values it holds -- NaN included -- never reach this row
      if (s[k] == -INFINITY) continue;
      const float e = expf((float)(s[k] - mu));
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

template <int DT, int DH, int NW>
hipError_t launch_split(const SdpaArgs& a, hipStream_t st) {
  const int64_t grid = (a.n_q + 31) / 32 * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, false, NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// The key split: few query rows (one or two 32-row blocks) against a long
// key range (at least two key tiles per wave), unmasked, and too few
// (batch, head) pairs for one-wave workgroups to keep enough loads in
// flight (measured: with 2048 pairs and 512 keys the unsplit launch, which
// fits several workgroups per CU, is faster).
#ifndef SDPA_SPLIT_MIN_NK
#define SDPA_SPLIT_MIN_NK 512
#endif
#ifndef SDPA_SPLIT_MAX_HEADS
#define SDPA_SPLIT_MAX_HEADS 1024
#endif
bool use_split(int64_t n_q, int64_t n_k, int64_t heads, bool causal) {
  return !causal && n_q <= 64 && n_k >= SDPA_SPLIT_MIN_NK && heads < SDPA_SPLIT_MAX_HEADS;
}

template <int DT, int DH, bool CAUSAL, int NW>
hipError_t launch_nw(const SdpaArgs& a, hipStream_t st) {
  // causal: one wave per pair of 32-row blocks (see the kernel)
  const int64_t units = ((a.n_q + 31) / 32 + 1) / 2;
  const int64_t nqb = CAUSAL ? (units + NW - 1) / NW : (a.n_q + NW * 64 - 1) / (NW * 64);
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, CAUSAL, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// The causal pair layout (sdpa_fwd_kernel.h): a workgroup of NW waves takes
// NW consecutive 32-row blocks.  It is the causal layout for d >= 64
// (measured 0-3 % faster than two blocks u, nb − 1 − u per wave at d = 64,
// 28 % at d = 128); at d = 16, 32, where the exponentials bound the kernel,
// the other measured 5-10 % faster and is kept.  0 selects the other for all.
#ifndef SDPA_CAUSAL_PAIRS
#define SDPA_CAUSAL_PAIRS 1
#endif
template <int DT, int DH, bool CAUSAL, int NW>
hipError_t launch_pairs_nw(const SdpaArgs& a, hipStream_t st) {
  const int64_t grid = (a.n_q + NW * 32 - 1) / (NW * 32) * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, CAUSAL, NW, false, false, true>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// Waves per pair workgroup: eight (each loaded tile then serves 256 query
// rows, as in the other layouts), four for d = 128 (one wave per SIMD),
// short sequences, causal ones up to 2048 rows and long ones with too few
// heads for two eight-wave workgroups per CU, fewer below 64 rows.
// Causal, d = 64, four against eight (interleaved runs): [16,8,512,64]
// +13 %, [64,8,512,64] +18 %, [16,8,1024,64] +10 %, [8,8,2048,64] +4 %;
// [4,8,4096,64] −3.5 %, [2,8,8192,64] −4.5 %.  Smaller workgroups balance
// better where a head has few row blocks: the waves of one workgroup wait
// for its longest row block at every barrier.
int pairs_waves(int64_t n_q, int64_t heads, int d, bool causal) {
  if (n_q <= 32) return 1;
  if (n_q <= 64) return 2;
  if (d > 64 || n_q <= 128 || (causal && n_q <= 2048)) return 4;
  // Eight waves (one workgroup a CU) only while there are enough of those
  // workgroups.  Causal needs at least two per CU, since its workgroups
  // carry unequal work and the longest-first order needs a second round to
  // even it out ([1,8,4096,64]: 128 workgroups, four waves 362 against 267
  // TFLOP/s; [2,8,4096,64]: 256, 660 against 530).  Unmasked, by the
  // makespan below ([1,8,2048,64] 332 against 247, [4,8,1024,64] 529
  // against 409, [16,8,640,64] 525 against 453, [24,8,640,64] 608 against
  // 435; [2,8,4096,64] and [8,16,384,64] stay with eight).  (Fewer than four
  // waves measured slower.)
  if (causal) return (n_q + 255) / 256 * heads < 2 * 256 ? 4 : 8;
  // Unmasked: the shorter estimated makespan, in rounds of 256 CUs.  An
  // eight-wave workgroup fills a CU (two waves a SIMD), so a partial last
  // round costs a whole one; four-wave workgroups pair up two a CU, and a
  // last round of at most one a CU runs one wave a SIMD, measured ≈ 0.6 of a
  // round.  Ties go to eight waves (each staged tile serves twice the rows).
  const int64_t wg8 = (n_q + 255) / 256 * heads, wg4 = (n_q + 127) / 128 * heads;
  const int64_t t8 = (wg8 + 255) / 256 * 10;
  const int64_t rem4 = wg4 % 512;
  const int64_t t4 = wg4 / 512 * 10 + (rem4 == 0 ? 0 : rem4 > 256 ? 10 : 6);
  return t4 < t8 ? 4 : 8;
}

template <int DT, int DH, bool CAUSAL>
hipError_t launch_pairs(const SdpaArgs& a, hipStream_t st) {
  switch (pairs_waves(a.n_q, (int64_t)a.B * a.H, DH, CAUSAL)) {
    case 1: return launch_pairs_nw<DT, DH, CAUSAL, 1>(a, st);
    case 2: return launch_pairs_nw<DT, DH, CAUSAL, 2>(a, st);
    case 4: return launch_pairs_nw<DT, DH, CAUSAL, 4>(a, st);
    default: return launch_pairs_nw<DT, DH, CAUSAL, (DH <= 64 ? 8 : 4)>(a, st);
  }
}

// Unmasked, d >= 64: the pair layout (32 query rows a wave) when the
// two-block layout (64 a wave) would leave fewer than two waves on each
// SIMD: twice the waves, and one workgroup of eight then fills a compute
// unit.  0 selects two blocks for all.
#ifndef SDPA_NONCAUSAL_PAIRS
#define SDPA_NONCAUSAL_PAIRS 1
#endif
constexpr int64_t kSimds = 256 * 4;  // 256 compute units of 4 SIMDs
bool noncausal_pairs(int64_t n_q, int64_t heads, int d) {
  const int64_t waves2 = heads * ((n_q + 63) / 64);  // waves of the two-block layout
  return SDPA_NONCAUSAL_PAIRS && d >= 64 && waves2 < 2 * kSimds;
}

// Unmasked, d = 64, at least 2048 query rows: workgroups of 8 waves (512
// rows) where the rule below picks 4: each K/V tile that a workgroup loads
// into LDS then serves twice the rows.  Measured against 4 waves
// (interleaved runs, identical results): [4,8,4096,64] +3.0 %,
// [2,8,8192,64] +3.6 %, [8,8,2048,64] +2.2 %, [8,8,4096,64] +0.4 %.
// (d = 128 holds one wave per SIMD, so 8 waves do not fit a compute unit;
// at d = 16 and 32, bound by the exponentials, 8 waves measured 5-8 %
// slower.)
// Only where eight-wave workgroups (one a CU) do not leave a ragged last
// round: the same makespan estimate as for the pair layout, in rounds of
// 256 CUs, ties to eight ([8,8,2560,64]: 320 eight-wave workgroups, four
// waves 835 against 667 TFLOP/s; [12,8,2048,64] 939 against 773;
// [4,8,4608,64] 796 against 634; balanced grids unchanged).
bool noncausal_eight_waves(int64_t n_q, int64_t heads, int d) {
  if (!(d == 64 && n_q >= 2048 && waves_per_wg(n_q, heads, false) == 4)) return false;
  const int64_t wg8 = (n_q + 511) / 512 * heads, wg4 = (n_q + 255) / 256 * heads;
  const int64_t t8 = (wg8 + 255) / 256 * 10;
  const int64_t rem4 = wg4 % 512;
  const int64_t t4 = wg4 / 512 * 10 + (rem4 == 0 ? 0 : rem4 > 256 ? 10 : 6);
  return t8 <= t4;
}

template <int DT, int DH, bool CAUSAL>
hipError_t launch_mfma(const SdpaArgs& a, hipStream_t st) {
  const int64_t heads = (int64_t)a.B * a.H;
  if constexpr (CAUSAL && SDPA_CAUSAL_PAIRS && DH >= 64) {
    return launch_pairs<DT, DH, true>(a, st);
  } else {
    if (use_split(a.n_q, a.n_k, heads, CAUSAL))
      return launch_split<DT, DH, split_waves(DH)>(a, st);
    if constexpr (!CAUSAL && DH >= 64)
      if (noncausal_pairs(a.n_q, heads, DH)) return launch_pairs<DT, DH, false>(a, st);
    if constexpr (!CAUSAL && DH == 64)
      if (noncausal_eight_waves(a.n_q, heads, DH)) return launch_nw<DT, DH, false, 8>(a, st);
    switch (waves_per_wg(a.n_q, (int64_t)a.B * a.H, CAUSAL)) {
      case 1: return launch_nw<DT, DH, CAUSAL, 1>(a, st);
      case 2: return launch_nw<DT, DH, CAUSAL, 2>(a, st);
      default: return launch_nw<DT, DH, CAUSAL, 4>(a, st);
    }
  }
}

template <int DT, int DH>
hipError_t launch_mask(const SdpaArgs& a, int causal, hipStream_t st) {
  return causal ? launch_mfma<DT, DH, true>(a, st) : launch_mfma<DT, DH, false>(a, st);
}

template <int DT>
hipError_t launch_dim(const SdpaArgs& a, int causal, int d, hipStream_t st) {
  switch (d) {
    case 16: return launch_mask<DT, 16>(a, causal, st);
    case 32: return launch_mask<DT, 32>(a, causal, st);
    case 64: return launch_mask<DT, 64>(a, causal, st);
    case 128: return launch_mask<DT, 128>(a, causal, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DH>
hipError_t launch_f32(const SdpaArgs& a, float scale, int causal, hipStream_t st) {
  dim3 grid((unsigned)((a.n_q + 63) / 64), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((sdpa_f32_kernel<DH>), grid, dim3(64), 0, st, a, scale, causal);
  return hipGetLastError();
}

}  // namespace

int sdpa_rows_per_workgroup(int dtype, int causal, int64_t n_q, int64_t n_k, int64_t heads, int d) {
  if (dtype == DT_F32) return 64;
  if (d > 128) return 32;  // the wide-head kernel
  if (!causal && n_q == 1 && (d == 64 || d == 128) && n_k >= 512) return 1;  // the decoding-step kernel
  if (causal && SDPA_CAUSAL_PAIRS && d >= 64) return pairs_waves(n_q, heads, d, true) * 32;
  if (use_split(n_q, n_k, heads, causal != 0)) return 32;
  if (!causal && noncausal_pairs(n_q, heads, d)) return pairs_waves(n_q, heads, d, false) * 32;
  if (!causal && noncausal_eight_waves(n_q, heads, d)) return 512;
  return waves_per_wg(n_q, heads, causal != 0) * 64;
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
  if (d > 128) return launch_sdpa_wide(a, dtype, causal, d, st);
  if (a.window) return launch_sdpa_window(a, dtype, d, st);
  if (sdpa_decode_applies(a, dtype, causal, d)) return launch_sdpa_decode(a, dtype, d, st);
  return dtype == DT_BF16 ? launch_dim<DT_BF16>(a, causal, d, st) : launch_dim<DT_F16>(a, causal, d, st);
}

}  // namespace mha
