// Projection GEMMs of the multi-head attention sublayer for gfx950.
//
// "Lire « Attention Is All You Need »" (nickwang.xyz), §3.2.2 "Attention
// multi-têtes": head_i uses x·W_i^Q, x·W_i^K, x·W_i^V with
// W_i ∈ R^{d_model×d_k}, and the sublayer ends with Concat(heads)·W^O.
// The h per-head matrices are the column blocks of one [d_model, h·d_k]
// row-major matrix (head i = columns [i·d_k, (i+1)·d_k)), multiplied on the
// right, as in the "32 Transformer" PyTorch sketch (ml-canon.vercel.app).
//
// C = A·W with A [M, K] (K contiguous) and W [K, N] (N contiguous), bf16 or
// fp16 in, fp32 accumulate, rounded once (RNE) on store.  The MFMA needs 8
// consecutive k per lane in both operands, so the kernel computes
// Cᵀ = Wᵀ·Aᵀ: A tiles are staged to LDS as they are, W tiles are transposed
// while being staged (four k-rows per thread, written as 8-byte runs along
// k).  In the Cᵀ result layout a lane holds 4 consecutive n of one row m,
// written as one 8-byte store, and the head split / concat is folded into
// the store address (see GemmProblem).
//
// Up to three independent problems (the Q, K and V projections) share one
// launch: blockIdx.y selects the problem.

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int BK = 32;       // k per LDS stage (two 16-k MFMA steps)
constexpr int AST = BK + 8;  // LDS row stride (elements) of both tiles: 80 B

template <int DT, int TM, int TN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int WM = TM / 64;  // 32-row m blocks per wave (waves tiled 2 x 2)
  constexpr int WN = TN / 64;  // 32-col n blocks per wave
  constexpr int ACH = TM * BK / 8 / 256;  // 16-byte A chunks per thread
  constexpr int VN = TN / 32;             // n values per thread per k row (4 k rows per thread)
  static_assert(ACH >= 1 && (VN == 2 || VN == 4), "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][TM * AST];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][TN * AST];

  const GemmProblem& P = g.prob[blockIdx.y];
  const int tiles_n = g.N / TN;
  const int tiles_m = (P.M + TM - 1) / TM;
  const int tile = blockIdx.x;
  if (tile >= tiles_m * tiles_n) return;
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  const uint16_t* Ag = (const uint16_t*)P.A;
  const uint16_t* Wg = (const uint16_t*)P.W;

  u32x4 areg[ACH];
  typedef uint32_t wrow_t __attribute__((ext_vector_type(VN / 2)));
  wrow_t wreg[4];
  constexpr int NG = TN / VN;  // threads along n
  const int w_nq = tid % NG, w_kg = tid / NG;  // w_kg in [0, 8): k rows 4*w_kg .. +3

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int ch = tid + r * 256;
      const int row = m0 + ch / (BK / 8);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < P.M) v = *(const u32x4*)(Ag + (int64_t)row * P.lda + k0 + (ch % (BK / 8)) * 8);
      areg[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wreg[r] = *(const wrow_t*)(Wg + (int64_t)(k0 + w_kg * 4 + r) * P.ldw + n0 + w_nq * VN);
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int ch = tid + r * 256;
      *(u32x4*)&As[buf][(ch / (BK / 8)) * AST + (ch % (BK / 8)) * 8] = areg[r];
    }
#pragma unroll
    for (int nn = 0; nn < VN; ++nn) {
      const int sh = (nn & 1) * 16;
      const uint32_t e0 = (wreg[0][nn >> 1] >> sh) & 0xFFFFu;
      const uint32_t e1 = (wreg[1][nn >> 1] >> sh) & 0xFFFFu;
      const uint32_t e2 = (wreg[2][nn >> 1] >> sh) & 0xFFFFu;
      const uint32_t e3 = (wreg[3][nn >> 1] >> sh) & 0xFFFFu;
      *(u32x2*)&Ws[buf][(w_nq * VN + nn) * AST + w_kg * 4] = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
  };

  f32x16 acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x16{};

  const int nk = g.K / BK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[WN], bf[WM];
#pragma unroll
      for (int i = 0; i < WN; ++i)
        af[i] = *(const u32x4*)&Ws[buf][(wn * (TN / 2) + i * 32 + l32) * AST + ks * 16 + hi * 8];
#pragma unroll
      for (int j = 0; j < WM; ++j)
        bf[j] = *(const u32x4*)&As[buf][(wm * (TM / 2) + j * 32 + l32) * AST + ks * 16 + hi * 8];
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WM; ++j) acc[i][j] = mfma_32x32x16<DT>(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) swrite(buf ^ 1);
    __syncthreads();
  }

  uint16_t* Cg = (uint16_t*)P.C;
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int m = m0 + wm * (TM / 2) + j * 32 + l32;
    if (m >= P.M) continue;
    const int bb = m / P.rows_per_b, tt = m % P.rows_per_b;
    uint16_t* crow = Cg + (int64_t)bb * P.c_sb + (int64_t)tt * P.c_st;
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * (TN / 2) + i * 32 + gq * 8 + hi * 4;
        const int head = n / P.head_dim, jj = n % P.head_dim;
        const u32x2 w = {pack2<DT>(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]),
                         pack2<DT>(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
        *(u32x2*)(crow + (int64_t)head * P.c_sh + jj) = w;
      }
  }
}

template <int DT, int TM, int TN>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int max_tiles = 0;
  for (int i = 0; i < a.nprob; ++i) {
    const int t = ((a.prob[i].M + TM - 1) / TM) * (a.N / TN);
    max_tiles = t > max_tiles ? t : max_tiles;
  }
  if (max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<DT, TM, TN>), dim3(max_tiles, a.nprob), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs& a, hipStream_t st) {
  // Large tiles when they still give every CU at least two workgroups.
  int64_t big = 0;
  for (int i = 0; i < a.nprob; ++i) big += ((a.prob[i].M + 127) / 128) * (int64_t)(a.N / 128);
  if (a.N % 128 == 0 && big >= 512) return launch_t<DT, 128, 128>(a, st);
  return launch_t<DT, 64, 64>(a, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t st) {
  if (a.N % 64 != 0 || a.K % BK != 0) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_dt<DT_BF16>(a, st) : launch_dt<DT_F16>(a, st);
}

}  // namespace mha
