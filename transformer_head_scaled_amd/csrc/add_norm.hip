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
// kept in registers (d <= 4096: at most 16 such chunks), so the two wave
// reductions -- the sum for mu, then the sum of squared deviations for var
// (two passes over registers: no cancellation from a sum of squares) -- and
// the normalised store cost no further memory traffic.  Bound by HBM: the
// bytes are the inputs and the output, once.  Sums and the normalisation are
// fp32; the output is rounded once to the storage dtype.
//
// Input forms: two rows of the storage dtype added in fp32 (mha_add_norm),
// or one fp32 row that already holds x + sub (written by the output
// projection's epilogue in mha_forward_add_norm).

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kChunks = kAddNormMaxD / 256;

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

template <int DT, bool ZF32>
__global__ __launch_bounds__(256) void add_norm_kernel(AddNormArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.rows) return;  // whole wave: nothing below synchronises
  const int d = a.d;
  const int64_t base = row * d;

  f32x4 z[kChunks];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = c * 256 + lane * 4;
    z[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < d) {
      if constexpr (ZF32)
        z[c] = *(const f32x4*)((const float*)a.z + base + i);
      else
        z[c] = load4<DT>(a.x, base + i) + load4<DT>(a.sub, base + i);
      s += (z[c][0] + z[c][1]) + (z[c][2] + z[c][3]);
    }
  }
  const float inv_d = 1.f / (float)d;
  const float mu = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = c * 256 + lane * 4;
    if (i < d) {
      const f32x4 dev = z[c] - mu;
      q += (dev[0] * dev[0] + dev[1] * dev[1]) + (dev[2] * dev[2] + dev[3] * dev[3]);
    }
  }
  const float var = wave_sum(q) * inv_d;
  const float rstd = 1.f / sqrtf(var + a.eps);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = c * 256 + lane * 4;
    if (i < d) {
      const f32x4 g = load4<DT>(a.gamma, i);
      const f32x4 b = load4<DT>(a.beta, i);
      store4<DT>(a.out, base + i, (z[c] - mu) * rstd * g + b);
    }
  }
}

template <int DT>
hipError_t launch_dt(const AddNormArgs& a, bool z_f32, hipStream_t st) {
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (z_f32)
    hipLaunchKernelGGL((add_norm_kernel<DT, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((add_norm_kernel<DT, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
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
