// One query row against a cache of keys and values (a decoding step), bf16 /
// fp16, d = 64 or 128: eq. (1) of "Lire « Attention Is All You Need »"
// (nickwang.xyz), §3.2.1, for a single query position, as in the
// auto-regressive decoder of §3.1 ("Trois usages de l'attention dans le
// modèle": each new position attends to the positions already produced).
//
// With one query row there is no matrix product to speak of: 4·d flops per
// 4·d bytes of K and V, so the kernel is bound by HBM and the matrix cores
// (and the LDS staging they need) only cost.  Here the keys and values go
// straight from memory into registers.
//
// One workgroup of 8 waves per (batch, head); wave w takes a contiguous run
// of keys.  A lane holds 16 bytes (8 elements) of one key row per load, so
// LPK = d/8 lanes share a key and one wave load covers KPI = 64/LPK whole
// rows (1 KB).  Each lane forms the partial dot product of its 8 elements
// with the query, the LPK lanes of a key add theirs (butterfly), and every
// lane then runs the online softmax over the keys of its slot (lane / LPK),
// keeping the row max m, the sum l and its 8 output elements o.  The loads
// of U = 8 rows of K and of V are in flight at a time per lane (16 KB per
// wave).  At the end the slots of a wave are merged (butterfly on m, l, o),
// then the 8 waves through LDS, and wave 0 writes O = o / l.
//
// Rows past the key length are not read (the buffer range ends there, loads
// past it return zero) and get weight 0; a head with no valid key gives 0.
// Used for one query row with at least 512 keys (shorter caches, several
// rows: the flash kernel).

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kDecWaves = 8;  // waves per workgroup
constexpr int kDecU = 8;      // key loads (of K and of V) in flight per lane

template <int DT>
__device__ __forceinline__ void unpack8(u32x4 w, float (&x)[8]) {
  const f32x4 a = unpack4<DT>(u32x2{w[0], w[1]}), b = unpack4<DT>(u32x2{w[2], w[3]});
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// x + the value of lane `ctrl` picks (DPP, within a row of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf,
                                                                   0xf, false));
}

// Sum over the N = 8 or 16 aligned lanes of a key, left in all of them:
// quad_perm [1,0,3,2] and [2,3,0,1] sum a quad, the half-row mirror (lane i
// and 7 − i of 8) adds the other quad, the row mirror (i and 15 − i) the
// other half-row.
template <int N>
__device__ __forceinline__ float key_sum(float x) {
  x = dpp_add<0xb1>(x);
  x = dpp_add<0x4e>(x);
  x = dpp_add<0x141>(x);
  if constexpr (N == 16) x = dpp_add<0x140>(x);
  return x;
}

template <int DT, int D>
__global__ __launch_bounds__(kDecWaves * 64) void sdpa_decode_kernel(SdpaArgs p) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPI = 64 / LPK;  // key rows per wave load
  constexpr int STEP = kDecU * KPI;
  static_assert(D == 64 || D == 128, "decode head dimension");

  __shared__ float xs[kDecWaves][LPK][10];  // per wave and chunk: m, l, o[8]

  const int bh = blockIdx.x;
  const int b = bh / p.H, hh = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPK, ch = lane % LPK;

  int n_eff = p.n_k;
  if (p.lens) n_eff = min(max(p.lens[b], 0), p.n_k);
  // this wave's keys [k_lo, k_hi), whole steps except for the last wave
  const int per = (n_eff + kDecWaves * STEP - 1) / (kDecWaves * STEP) * STEP;
  const int k_lo = min(wave * per, n_eff), k_hi = min(k_lo + per, n_eff);

  const uint16_t* Qg = (const uint16_t*)p.Q + b * p.q_sb + hh * p.q_sh;
  const uint16_t* Kg = (const uint16_t*)p.K + b * p.k_sb + hh * p.k_sh;
  const uint16_t* Vg = (const uint16_t*)p.V + b * p.v_sb + hh * p.v_sh;
  // buffer ranges ending at the valid keys
  __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kg, (short)0, (int)((int64_t)n_eff * p.k_sr * 2), 0x00020000);
  __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vg, (short)0, (int)((int64_t)n_eff * p.v_sr * 2), 0x00020000);

  // this lane's 8 query elements, sign of the scale folded in (exact)
  float q[8];
  unpack8<DT>(*(const u32x4*)(Qg + ch * 8), q);
  const float c = p.c;
  if (p.neg) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = -q[e];
  }

  float m = -INFINITY, mc = 0.f, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int k0 = k_lo; k0 < k_hi; k0 += STEP) {
    u32x4 kw[kDecU], vw[kDecU];
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const uint32_t key = (uint32_t)(k0 + u * KPI + slot);
      kw[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(key * (uint32_t)p.k_sr * 2u + ch * 16), 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const uint32_t key = (uint32_t)(k0 + u * KPI + slot);
      vw[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)(key * (uint32_t)p.v_sr * 2u + ch * 16), 0, 0);
    }
    // all 2·U loads out before any of them is used
    __builtin_amdgcn_sched_barrier(0);
    float s[kDecU];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      float kx[8];
      unpack8<DT>(kw[u], kx);
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        d0 = __builtin_fmaf(q[e], kx[e], d0);
        d1 = __builtin_fmaf(q[e + 1], kx[e + 1], d1);
      }
      const float sc = key_sum<LPK>(d0 + d1);
      // keys past this wave's run: weight 0, and their value words cleared
      // so that 0·inf cannot turn into NaN (runs are whole steps, so these
      // are past the key length and read as zero already; the clearing keeps
      // that from depending on the split)
      const int key = k0 + u * KPI + slot;
      const bool in = key < k_hi;
      s[u] = in ? sc : -INFINITY;
      if (!in) vw[u] = u32x4{0u, 0u, 0u, 0u};
      mx = fmaxf(mx, s[u]);
    }
    if (mx > m) {
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mx) * c);
      m = mx;
      mc = m * c;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u], c, -mc));
      float vx[8];
      unpack8<DT>(vw[u], vx);
      l += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(w, vx[e], o[e]);
    }
  }

  // merge the key slots of the wave: lanes ch, ch + LPK, ... hold one chunk
  auto merge = [&](float m2, float l2, const float (&o2)[8]) __attribute__((always_inline)) {
    const float M = fmaxf(m, m2);
    const float e1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - M) * c);
    const float e2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m2 - M) * c);
    m = M;
    l = l * e1 + l2 * e2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * e1 + o2[e] * e2;
  };
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[e], off, 64);
    merge(m2, l2, o2);
  }
  if (lane < LPK) {
    xs[wave][ch][0] = m;
    xs[wave][ch][1] = l;
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[wave][ch][2 + e] = o[e];
  }
  __syncthreads();
  if (wave != 0 || lane >= LPK) return;
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) {
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = xs[w][ch][2 + e];
    merge(xs[w][ch][0], xs[w][ch][1], o2);
  }
  const float inv = row_sum_inverse(l, n_eff > 0);
  const u32x4 out = {pack2<DT>(o[0] * inv, o[1] * inv), pack2<DT>(o[2] * inv, o[3] * inv),
                     pack2<DT>(o[4] * inv, o[5] * inv), pack2<DT>(o[6] * inv, o[7] * inv)};
  uint16_t* Og = (uint16_t*)p.O + b * p.o_sb + hh * p.o_sh;
  *(u32x4*)(Og + ch * 8) = out;
}

template <int DT>
hipError_t launch_dt(const SdpaArgs& a, int d, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.B * a.H)), block(kDecWaves * 64);
  if (d == 64)
    hipLaunchKernelGGL((sdpa_decode_kernel<DT, 64>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((sdpa_decode_kernel<DT, 128>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_decode(const SdpaArgs& a, int dtype, int d, hipStream_t st) {
  if (a.n_q != 1 || (d != 64 && d != 128)) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_dt<DT_BF16>(a, d, st) : launch_dt<DT_F16>(a, d, st);
}

}  // namespace mha
