// Scaled dot-product attention: the fp32 kernel, the launchers of the flash
// kernel (sdpa_fwd_kernel.h) for the unmasked, causal and key-split forms,
// and the dispatch of a route (sdpa_route.cpp chooses kernel and workgroup
// size).  The restricted-window launches are in sdpa_window.hip.

#include "sdpa_fwd_kernel.h"

namespace mha {

namespace {

// ---------------------------------------------------------------- fp32 path
//
// Plain fp32 attention for small problems and the 1e-5 parity case: LPR
// lanes per query row (1, or 4 where one lane a row would leave most SIMDs
// idle), each holding DH / LPR of the row's columns of Q and O; K/V tiles of
// 32 keys broadcast from LDS; the online softmax taken one key at a time (the
// running max moves only when a key beats it, and only then are O and the
// sum rescaled).  Any head dimension in {16, 32, 64, 128}.  Inputs and the
// output accumulator are fp32; each dot product, the running max and the
// exponent argument are formed in fp64 (four partial sums per lane, then the
// LPR lanes' partials added pairwise, which gives the row's lanes identical
// bits), so the scores carry no fp32 summation error even when they are
// large (an unscaled softmax), and the only fp32 roundings left are expf and
// the weighted sum of V.  The key loop is not unrolled: the row's registers
// stay in registers and nothing spills.
template <int DH, int LPR>
__global__ __launch_bounds__(64) void sdpa_f32_kernel(SdpaArgs p, float scale, int causal) {
  constexpr int TK = 32, DS = DH / LPR, RPW = 64 / LPR;  // columns per lane, rows per workgroup
  static_assert(DS % 4 == 0, "four partial sums per lane");
  __shared__ __attribute__((aligned(16))) float Ks[TK * DH];
  __shared__ __attribute__((aligned(16))) float Vs[TK * DH];
  const int b = blockIdx.z, hh = blockIdx.y;
  const int row = blockIdx.x * RPW + (int)threadIdx.x / LPR;
  const int c0 = ((int)threadIdx.x % LPR) * DS;  // this lane's first column
  const float* Qg = (const float*)p.Q + b * p.q_sb + hh * p.q_sh;
  const float* Kg = (const float*)p.K + b * p.k_sb + hh * p.k_sh;
  const float* Vg = (const float*)p.V + b * p.v_sb + hh * p.v_sh;
  float* Og = (float*)p.O + b * p.o_sb + hh * p.o_sh;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  const int r_end = min((int)(blockIdx.x + 1) * RPW, p.n_q);  // one past the block's last row
  int kend = n_eff;
  if (causal) kend = min(kend, r_end);
  int jlo = 0;  // restricted window: the keys the block's rows can reach
  if (p.window) {
    kend = min(kend, r_end - 1 + p.win_right + 1);
    jlo = max(0, (int)blockIdx.x * RPW - p.win_left) / TK;
  }
  const int ntiles = kend > 0 ? (kend + TK - 1) / TK : 0;
  // this row's visible keys: [lo, hi)
  int lo = 0, hi = n_eff;
  if (causal) hi = min(hi, row + 1);
  if (p.window) {
    lo = max(lo, row - p.win_left);
    hi = min(hi, row + p.win_right + 1);
  }

  // (one test for the whole row, so that the loads go out together rather
  // than one branch and one wait per element)
  float q[DS], o[DS];
#pragma unroll
  for (int d = 0; d < DS; ++d) q[d] = o[d] = 0.f;
  if (row < p.n_q) {
#pragma unroll
    for (int d = 0; d < DS; ++d) q[d] = Qg[(int64_t)row * p.q_sr + c0 + d];
  }
  double m = -INFINITY;
  float l = 0.f;

  for (int j = jlo; j < ntiles; ++j) {
    __syncthreads();
    // a fixed trip count, and keys past the valid length read from the last
    // valid key and then cleared (no branch around the loads), so that the
    // loads of a thread can all be in flight together (n_eff >= 1 here: a
    // tile exists only below kend <= n_eff)
    constexpr int PER_T = TK * DH / 4 / 64;  // float4 pieces per thread and tile
    static_assert(TK * DH / 4 % 64 == 0, "whole pieces per thread");
#pragma unroll
    for (int it = 0; it < PER_T; ++it) {
      const int e = (int)threadIdx.x + 64 * it;
      const int key = j * TK + (e * 4) / DH, d = (e * 4) % DH;
      const int64_t kr = min(key, n_eff - 1);
      float4 kv = *(const float4*)(Kg + kr * p.k_sr + d);
      float4 vv = *(const float4*)(Vg + kr * p.v_sr + d);
      if (key >= n_eff) kv = vv = float4{0.f, 0.f, 0.f, 0.f};
      *(float4*)&Ks[e * 4] = kv;
      *(float4*)&Vs[e * 4] = vv;
    }
    __syncthreads();
    // a masked key is skipped outright (not added with weight 0), so the
    // values it holds -- NaN included -- never reach this row.  The bounds
    // are the row's, the same for its LPR lanes, which therefore run the
    // loop (and its lane exchanges) together.
    const int k0 = max(lo - j * TK, 0), k1 = min(hi - j * TK, TK);
#pragma unroll 1
    for (int k = k0; k < k1; ++k) {
      const float* kr = &Ks[k * DH + c0];
      double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int d = 0; d < DS; ++d) a[d % 4] = __builtin_fma((double)q[d], (double)kr[d], a[d % 4]);
      double acc = (a[0] + a[1]) + (a[2] + a[3]);
      // x + partner(x) is the same sum on both lanes of a pair
      if constexpr (LPR >= 2) acc += __shfl_xor(acc, 1, 64);
      if constexpr (LPR >= 4) acc += __shfl_xor(acc, 2, 64);
      const double sc = acc * (double)scale;
      if (sc > m) {  // a new running max: rescale what has been summed
        const float alpha = (m == -INFINITY) ? 0.f : expf((float)(m - sc));
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DS; ++d) o[d] *= alpha;
        m = sc;
      }
      // a score of −∞ (an infinite key element) has weight 0, also while the
      // running max is still −∞
      const float e = sc == -INFINITY ? 0.f : expf((float)(sc - m));
      l += e;
      const float* vr = &Vs[k * DH + c0];
#pragma unroll
      for (int d = 0; d < DS; ++d) o[d] = __builtin_fmaf(e, vr[d], o[d]);
    }
  }
  if (row < p.n_q) {
    const float inv = row_sum_inverse(l, hi > lo);
#pragma unroll
    for (int d = 0; d < DS; ++d) Og[(int64_t)row * p.o_sr + c0 + d] = o[d] * inv;
  }
}

template <int DT, int DH, int NW>
hipError_t launch_split(const SdpaArgs& a, hipStream_t st) {
  const int64_t grid = (a.n_q + 31) / 32 * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, false, NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// the two-block layout
template <int DT, int DH, bool CAUSAL, int NW>
hipError_t launch_nw(const SdpaArgs& a, hipStream_t st) {
  // causal: one wave per pair of 32-row blocks (see the kernel)
  const int64_t units = ((a.n_q + 31) / 32 + 1) / 2;
  const int64_t nqb = CAUSAL ? (units + NW - 1) / NW : (a.n_q + NW * 64 - 1) / (NW * 64);
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, CAUSAL, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// the pair layout: a workgroup of NW waves takes NW consecutive 32-row blocks
// Causal, d = 64, at most four waves: 64 KB of LDS and at most two waves a
// SIMD, so two workgroups share a CU; a grid of at most 512 (and more than
// 256) workgroups is resident at once, workgroup x beside x + 256 (the
// dispatcher deals them round-robin to the 8 XCDs and within an XCD to its
// 32 CUs in turn).  The row groups of the second round then run shortest
// first (pair_split, the kernel): [16,8,512,64] pairs row groups 3 and 0,
// 2 and 1 on a CU instead of 3 and 1, 2 and 0.
template <int DT, int DH, bool CAUSAL, int NW>
hipError_t launch_pairs_nw(const SdpaArgs& a, hipStream_t st) {
  const int64_t grid = (a.n_q + NW * 32 - 1) / (NW * 32) * a.B * a.H;
  SdpaArgs b = a;
  b.pair_split = (CAUSAL && DH == 64 && NW <= 4 && (a.B * a.H) % 8 == 0 && grid > 256 && grid <= 512) ? 32 : 0;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, CAUSAL, NW, false, false, true>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, st, b);
  return hipGetLastError();
}

// Instantiate what the route names.  Eight-wave workgroups exist for the
// pair layout at d <= 64 and the unmasked two-block layout at d = 64 (d = 128
// holds one wave a SIMD, so eight waves would not fit a compute unit).
template <int DT, int DH, bool CAUSAL>
hipError_t launch_mfma(const SdpaArgs& a, const SdpaRoute& r, hipStream_t st) {
  switch (r.kernel) {
    case SDPA_K_PAIRS:
      if constexpr (DH >= 64) {
        switch (r.waves) {
          case 1: return launch_pairs_nw<DT, DH, CAUSAL, 1>(a, st);
          case 2: return launch_pairs_nw<DT, DH, CAUSAL, 2>(a, st);
          case 4: return launch_pairs_nw<DT, DH, CAUSAL, 4>(a, st);
          case 8:
            if constexpr (DH == 64) return launch_pairs_nw<DT, DH, CAUSAL, 8>(a, st);
            break;
        }
      }
      break;
    case SDPA_K_SPLIT:
      if constexpr (!CAUSAL)
        if (r.waves == split_waves(DH)) return launch_split<DT, DH, split_waves(DH)>(a, st);
      break;
    case SDPA_K_BLOCKS:
      // (causal at d >= 64 always takes the pair layout)
      if constexpr (!(CAUSAL && DH >= 64)) {
        switch (r.waves) {
          case 1: return launch_nw<DT, DH, CAUSAL, 1>(a, st);
          case 2: return launch_nw<DT, DH, CAUSAL, 2>(a, st);
          case 4: return launch_nw<DT, DH, CAUSAL, 4>(a, st);
          case 8:
            if constexpr (!CAUSAL && DH == 64) return launch_nw<DT, DH, CAUSAL, 8>(a, st);
            break;
        }
      }
      break;
  }
  return hipErrorInvalidValue;  // the route does not fit these arguments
}

template <int DT, int DH>
hipError_t launch_mask(const SdpaArgs& a, const SdpaRoute& r, int causal, hipStream_t st) {
  return causal ? launch_mfma<DT, DH, true>(a, r, st) : launch_mfma<DT, DH, false>(a, r, st);
}

template <int DT>
hipError_t launch_dim(const SdpaArgs& a, const SdpaRoute& r, int causal, int d, hipStream_t st) {
  switch (d) {
    case 16: return launch_mask<DT, 16>(a, r, causal, st);
    case 32: return launch_mask<DT, 32>(a, r, causal, st);
    case 64: return launch_mask<DT, 64>(a, r, causal, st);
    case 128: return launch_mask<DT, 128>(a, r, causal, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DH>
hipError_t launch_f32(const SdpaArgs& a, const SdpaRoute& r, float scale, int causal, hipStream_t st) {
  dim3 grid((unsigned)((a.n_q + r.rows - 1) / r.rows), (unsigned)a.H, (unsigned)a.B);
  if (r.rows == 16)
    hipLaunchKernelGGL((sdpa_f32_kernel<DH, 4>), grid, dim3(64), 0, st, a, scale, causal);
  else if (r.rows == 64)
    hipLaunchKernelGGL((sdpa_f32_kernel<DH, 1>), grid, dim3(64), 0, st, a, scale, causal);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa(const SdpaArgs& a, const SdpaRoute& r, int dtype, int causal, int d,
                       float scale, hipStream_t st) {
  switch (r.kernel) {
    case SDPA_K_F32:
      if (dtype != DT_F32) break;
      switch (d) {
        case 16: return launch_f32<16>(a, r, scale, causal, st);
        case 32: return launch_f32<32>(a, r, scale, causal, st);
        case 64: return launch_f32<64>(a, r, scale, causal, st);
        case 128: return launch_f32<128>(a, r, scale, causal, st);
      }
      break;
    case SDPA_K_WIDE: return launch_sdpa_wide(a, dtype, causal, d, r.waves, r.rows, st);
    case SDPA_K_WINDOW: return launch_sdpa_window(a, r, dtype, d, st);
    case SDPA_K_DECODE:
      if (causal || a.window) break;
      return launch_sdpa_decode(a, dtype, d, st);
    default:
      if (a.window) break;
      if (dtype == DT_BF16) return launch_dim<DT_BF16>(a, r, causal, d, st);
      if (dtype == DT_F16) return launch_dim<DT_F16>(a, r, causal, d, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mha
