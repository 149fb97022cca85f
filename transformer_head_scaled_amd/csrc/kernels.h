// Internal interface between the libmha host layer and its HIP kernels.
// Not part of the public C ABI (that is include/mha.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

// Strides are in elements.  Q/K/V/O rows are d contiguous elements.
struct SdpaArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int32_t B, H, n_q, n_k;
  float c;              // max(|scale| * log2(e), 1e-30)   (MFMA path)
  int32_t neg;          // scale < 0: the MFMA path negates Q exactly
  const int32_t* lens;  // device int32[B] valid key counts, or null
  // restricted attention: key c visible to query r iff
  // r - win_left <= c <= r + win_right (window != 0; reaches clamped to
  // [0, n_q] and [0, n_k])
  int32_t window, win_left, win_right;
  // launch the workgroups in the opposite order (the flash kernel; the
  // results are the same, which the determinism tests check)
  int32_t reverse;
  // pair layout, whole grid resident at once: the first slot of each XCD's
  // second round (the row groups there run shortest first); 0: longest
  // first throughout
  int32_t pair_split;
};

// The attention kernel a problem runs on, and its workgroup shape
// (sdpa_route.cpp).  The values are those of MHA_KERNEL_* in mha.h.
enum SdpaKernel : int {
  SDPA_K_F32 = 0,     // fp32 kernel
  SDPA_K_BLOCKS = 1,  // flash kernel, two 32-row blocks a wave
  SDPA_K_PAIRS = 2,   // flash kernel, one 32-row block a wave, two key tiles a step
  SDPA_K_SPLIT = 3,   // flash kernel, the waves of a workgroup split the keys
  SDPA_K_DECODE = 4,  // one query row, registers only
  SDPA_K_WINDOW = 5,  // flash kernel, restricted window
  SDPA_K_WIDE = 6     // d = 256, 512: the waves of a workgroup split d
};
struct SdpaRoute {
  int kernel;          // SdpaKernel
  int waves;           // waves per workgroup
  int rows;            // query rows per workgroup
  int64_t workgroups;  // grid size
};
// win_left / win_right: the reaches after clamping to [0, n_q] and [0, n_k]
SdpaRoute sdpa_route(int dtype, bool causal, bool window, int64_t B, int64_t H, int64_t n_q,
                     int64_t n_k, int d, int64_t win_left, int64_t win_right);

// Launch what the route names (errors if the route does not fit the
// arguments).
hipError_t launch_sdpa(const SdpaArgs& a, const SdpaRoute& r, int dtype, int causal, int d,
                       float scale, hipStream_t st);
// the flash kernel's window form (bf16 / fp16), sdpa_window.hip
hipError_t launch_sdpa_window(const SdpaArgs& a, const SdpaRoute& r, int dtype, int d, hipStream_t st);
// wide heads, d = 256 or 512 (bf16 / fp16, no window), sdpa_wide.hip; 8
// waves: 32 rows (causal, the key tiles split between two groups of 4) or
// 64 rows (two 32-row blocks sharing the staged tiles)
hipError_t launch_sdpa_wide(const SdpaArgs& a, int dtype, int causal, int d, int waves, int rows,
                            hipStream_t st);
// the smallest head dimension whose causal form splits the key tiles
#ifndef SDPA_WIDE_SPLIT_MIN_D
#define SDPA_WIDE_SPLIT_MIN_D 512
#endif
// one query row against a long key/value cache (bf16 / fp16, d = 64, 128,
// no mask but key lengths), sdpa_decode.hip
hipError_t launch_sdpa_decode(const SdpaArgs& a, int dtype, int d, hipStream_t st);

// One GEMM C = A·W of the projections: A [M, K] row-major (row stride lda),
// W [K, N] row-major (row stride ldw).  Output element (m, n) is written to
//   C + (m / rows_per_b) * c_sb + (m % rows_per_b) * c_st
//     + (n / head_dim) * c_sh + (n % head_dim)
// which expresses both the head-split layout [B, h, n, d] and a plain
// row-major [M, N] matrix.  head_dim is 16 or a multiple of 32.
// With R set, the epilogue adds the residual R[m·ldr + n] (storage dtype)
// and stores fp32 to C + m·c_st + n instead (the plain map only).
struct GemmProblem {
  const void* A;
  const void* W;
  void* C;
  const void* R;
  int64_t lda, ldw, ldr;
  int64_t c_sb, c_st, c_sh;
  int32_t M, rows_per_b, head_dim, pad_;
};

struct GemmArgs {
  GemmProblem prob[3];
  int32_t nprob;
  int32_t N, K;
  int32_t pad_;
};

// Chooses the tile shape from the problem sizes.
hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t st);

// The Q/K/V projections and the attention of each (batch, head) in one
// workgroup, for n_q, n_k in [1, 64], head dimension 64, no causal mask
// (mha_short.hip).  x_q [B, n_q, d_model], x_kv [B, n_k, d_model] (the same
// pointer as x_q with self set), W* [d_model, H·64]; C receives the concat
// [B, n_q, H·64].  c = scale·log2(e).
struct ShortArgs {
  const void* xq;
  const void* xkv;
  const void* Wq;
  const void* Wk;
  const void* Wv;
  void* C;
  const int32_t* lens;  // device int32[B] valid key counts, or null
  int32_t B, H, n_q, n_k, d_model, self;
  float c;
};
hipError_t launch_mha_short(const ShortArgs& a, int dtype, hipStream_t st);

// out = LayerNorm(x + sub) per row of d features (contiguous rows):
// z_f32 = false: x and sub in the storage dtype; true: z already holds
// x + sub in fp32.  gamma, beta [d] and out in the storage dtype.
constexpr int kAddNormMaxD = 4096;
struct AddNormArgs {
  const void* x;
  const void* sub;
  const void* z;
  const void* gamma;
  const void* beta;
  void* out;
  int64_t rows;
  int32_t d;
  float eps;
};
hipError_t launch_add_norm(const AddNormArgs& a, int dtype, bool z_f32, hipStream_t st);

}  // namespace mha
