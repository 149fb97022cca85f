// Residual connection and layer normalisation ("Add & Norm") for gfx950.
//
// out = LayerNorm(x + sub), per position: nickwang.xyz "Lire « Attention Is
// All You Need »", the section on the encoder and decoder stacks (paper
// §3.1) -- every sub-layer is wrapped as LayerNorm(x + Sublayer(x)), the
// normalisation after the addition.  LayerNorm is the standard one (the page
// does not write it out): over the d features of one position, the mean mu
// and the mean squared deviation var, then
//   gamma ⊙ (z − mu) / sqrt(var + eps) + beta.
//
// One wave per row (position), four rows per workgroup.  The row is read
// once, 4 consecutive features per lane and 256 per wave instruction, and
// kept in registers (NC = ceil(d / 256) such chunks, a template argument, so
// every load of the row -- and of gamma and beta -- is issued before the
// first reduction waits on any of them), so the two wave reductions -- the
// sum for mu, then the sum of squared deviations for var (two passes over
// registers: no cancellation from a sum of squares) -- and the normalised
// store cost no further memory traffic.  Bound by HBM: the bytes are the
// inputs and the output, once.  Sums and the normalisation are fp32; the
// output is rounded once to the storage dtype.
//
// Input forms: two rows of the storage dtype added in fp32 (mha_add_norm),
// or one fp32 row that already holds x + sub (written by the output
// projection's epilogue in mha_forward_add_norm).

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

// four consecutive elements of a storage-dtype array, as floats
template <int DT>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t i) {
  if constexpr (DT == DT_F32) {
    return *(const f32x4*)((const float*)base + i);
  } else {
    return unpack4<DT>(*(const u32x2*)((const uint16_t*)base + i));
  }
}

template <int DT>
__device__ __forceinline__ void store4(void* base, int64_t i, f32x4 v) {
  if constexpr (DT == DT_F32) {
    *(f32x4*)((float*)base + i) = v;
  } else {
    const u32x2 w = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
    *(u32x2*)((uint16_t*)base + i) = w;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  // butterfly: every lane ends with the same sum
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int DT, bool ZF32, int NC>
__global__ __launch_bounds__(256) void add_norm_kernel(AddNormArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.rows) return;  // whole wave: nothing below synchronises
  const int d = a.d;
  const int64_t base = row * d;

  // all loads first (chunks past d: zeros, never stored)
  f32x4 z[NC], g[NC], bt[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = c * 256 + lane * 4;
    const bool in = i < d;
    const int ii = in ? i : 0;  // an in-range address for lanes past d
    f32x4 v;
    if constexpr (ZF32)
      v = *(const f32x4*)((const float*)a.z + base + ii);
    else
      v = load4<DT>(a.x, base + ii) + load4<DT>(a.sub, base + ii);
    z[c] = in ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    g[c] = load4<DT>(a.gamma, ii);
    bt[c] = load4<DT>(a.beta, ii);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) s += (z[c][0] + z[c][1]) + (z[c][2] + z[c][3]);
  const float inv_d = 1.f / (float)d;
  const float mu = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = c * 256 + lane * 4;
    if (i < d) {
      const f32x4 dev = z[c] - mu;
      q += (dev[0] * dev[0] + dev[1] * dev[1]) + (dev[2] * dev[2] + dev[3] * dev[3]);
    }
  }
  const float var = wave_sum(q) * inv_d;
  const float rstd = 1.f / sqrtf(var + a.eps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = c * 256 + lane * 4;
    if (i < d) store4<DT>(a.out, base + i, (z[c] - mu) * rstd * g[c] + bt[c]);
  }
}

template <int DT, int NC>
hipError_t launch_nc(const AddNormArgs& a, bool z_f32, hipStream_t st) {
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (z_f32)
    hipLaunchKernelGGL((add_norm_kernel<DT, true, NC>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((add_norm_kernel<DT, false, NC>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// chunks of 256 features: the smallest power of two that covers d
template <int DT>
hipError_t launch_dt(const AddNormArgs& a, bool z_f32, hipStream_t st) {
  const int nc = (a.d + 255) / 256;
  if (nc <= 1) return launch_nc<DT, 1>(a, z_f32, st);
  if (nc <= 2) return launch_nc<DT, 2>(a, z_f32, st);
  if (nc <= 4) return launch_nc<DT, 4>(a, z_f32, st);
  if (nc <= 8) return launch_nc<DT, 8>(a, z_f32, st);
  return launch_nc<DT, 16>(a, z_f32, st);
}

}  // namespace

hipError_t launch_add_norm(const AddNormArgs& a, int dtype, bool z_f32, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.d <= 0 || a.d > kAddNormMaxD || a.d % 4 != 0) return hipErrorInvalidValue;
  switch (dtype) {
    case DT_F32: return launch_dt<DT_F32>(a, z_f32, st);
    case DT_BF16: return launch_dt<DT_BF16>(a, z_f32, st);
    case DT_F16: return launch_dt<DT_F16>(a, z_f32, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mha
