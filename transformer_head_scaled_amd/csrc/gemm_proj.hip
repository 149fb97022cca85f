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
// Cᵀ = Wᵀ·Aᵀ with the 32x32x16 MFMA: the B operand (Aᵀ) is a 16-byte read
// of an A row, the A operand (Wᵀ) comes from transposing LDS reads
// (ds_read_b64_tr_b16) of the row-major W tile.  In the Cᵀ result a lane
// holds 4 consecutive n of one row m; the two lanes of a row exchange
// pieces so that each writes 8 consecutive n with one 16-byte store, and
// the head split / concat is folded into the store address (GemmProblem).
//
// Tiles: TM × TN outputs per workgroup of 4 waves (2 × 2, each TM/2 × TN/2),
// two LDS stages of 64 k (64 × 64 tiles; 128 k for grids of at most two
// tiles a CU) or 32 k (128 × 128 tiles: 32 KB of
// LDS, so three workgroups share a compute unit where 64 k left room for two;
// the big cross-attention's Q/K/V launch then runs its 704 tiles in one
// round, measured 1.5-2 % faster on its sub-layer, identical results).
// A and W tiles go from memory straight
// into LDS (buffer loads with an LDS destination; the buffer range ends at
// row M of A, so rows past it read as zero).  LDS rows are stored with
// their 16-byte chunks XOR-permuted by row bits so that every fragment read
// phase touches each bank once.
//
// Up to three independent problems (the Q, K and V projections) share one
// launch: blockIdx.y selects the problem.

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

#ifndef GEMM_BK_128
#define GEMM_BK_128 32  // k per LDS stage of the 128 x 128 tiles
#endif
#ifndef GEMM_SMALL_GRID
#define GEMM_SMALL_GRID 512  // 64 x 64 grids up to this many tiles (two a CU) take 128 k a stage
#endif

#ifndef GEMM_STAGES_128
#define GEMM_STAGES_128 2
#endif
#ifndef GEMM_STAGES_64
#define GEMM_STAGES_64 2
#endif
#ifndef GEMM_WTM_128
#define GEMM_WTM_128 64  // per-wave tile of the 128 x 128 workgroup tile
#endif
#ifndef GEMM_WTN_128
#define GEMM_WTN_128 64
#endif
#ifndef GEMM_BIG_MIN
#define GEMM_BIG_MIN 256   // 128 x 128 tiles once there are enough to give each CU one
#endif

// TM x TN outputs per workgroup; each wave computes WTM x WTN of them.
// BK: k per LDS stage (BK / 16 MFMA steps; A rows of 2·BK bytes).
template <int DT, int TM, int TN, int WTM, int WTN, int NSTAGE, int BK>
__global__ __launch_bounds__((TM / WTM) * (TN / WTN) * 64) void gemm_kernel(GemmArgs g) {
  constexpr int NWN = TN / WTN;              // waves along n
  constexpr int NWAVES = (TM / WTM) * NWN;
  constexpr int WM = WTM / 32;               // 32-row m blocks per wave
  constexpr int WN = WTN / 32;               // 32-col n blocks per wave
  constexpr int ACR = BK / 8;                        // 16-byte chunks per A row
  constexpr int ACH = TM * BK * 2 / 1024 / NWAVES;   // 1 KB A pieces per wave and stage
  constexpr int WCH = BK * TN * 2 / 1024 / NWAVES;  // 1 KB W pieces per wave and stage
  constexpr int WCR = TN / 8;         // 16-byte chunks per W row
  static_assert(ACH >= 1 && WCH >= 1 && (TN == 64 || TN == 128) && (BK == 32 || BK == 64 || BK == 128), "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t As[NSTAGE][TM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[NSTAGE][BK * TN];

  // Workgroups are dealt to the 8 XCDs round-robin (in linear order); the
  // remap gives each XCD a contiguous run of tiles, i.e. whole row blocks
  // of A (n is the fastest tile index), which then share that XCD's L2.
  const uint32_t lin = xcd_remap(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const GemmProblem& P = g.prob[lin / gridDim.x];
  const int tiles_n = g.N / TN;
  const int tiles_m = (P.M + TM - 1) / TM;
  const int tile = lin % gridDim.x;
  if (tile >= tiles_m * tiles_n) return;
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5, i16 = lane & 15, g16 = (lane >> 4) & 1;
  const int wm = wave / NWN, wn = wave % NWN;

  // chunk permutations: A rows (ACR chunks) by the row's index among the
  // rows of one 256-byte bank cycle (16 / ACR of them), so that 16 lanes
  // reading one chunk index of 16 consecutive rows cover all banks; W rows
  // (128 or 256 bytes) by the row's position among 4 consecutive k, so that
  // the 4 (or 2 x 4) rows a transposing read touches fall on distinct banks
  auto a_swz = [](int m) { return (m / (16 / ACR)) & (ACR - 1); };
  auto w_swz = [](int k) { return TN == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); };

  // A: descriptor over this workgroup's rows; per lane, the byte offset of
  // its chunk within a k stage
  const int a_rows = min(TM, P.M - m0);
  const u32x4 ars = raw_rsrc((const uint16_t*)P.A + (int64_t)m0 * P.lda,
                             (uint32_t)((int64_t)a_rows * P.lda * 2));
  uint32_t a_off[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = (wave * ACH + i) * 64 + lane;  // LDS chunk this lane fills
    const int m = q / ACR;
    a_off[i] = (uint32_t)(m * P.lda * 2 + ((q % ACR) ^ a_swz(m)) * 16);
  }
  uint32_t w_off[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int q = (wave * WCH + i) * 64 + lane;
    const int k = q / WCR;
    w_off[i] = (uint32_t)(k * P.ldw * 2 + ((q % WCR) ^ w_swz(k)) * 16);
  }
  const uint16_t* Wg = (const uint16_t*)P.W + n0;

  auto gload = [&](int kt, int stage) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      load_lds_b128(ars,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&As[stage][(wave * ACH + i) * 512]),
                    a_off[i] + k0 * 2);
    // W: a descriptor per stage (k rows k0 .. k0 + 63 of this column block)
    const u32x4 wrs = raw_rsrc(Wg + (int64_t)k0 * P.ldw, (uint32_t)(BK * P.ldw * 2));
#pragma unroll
    for (int i = 0; i < WCH; ++i)
      load_lds_b128(wrs,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
                        __attribute__((address_space(3))) void*)&Ws[stage][(wave * WCH + i) * 512]),
                    w_off[i]);
  };

  // fragments: Aᵀ (MFMA B operand) for m block j, 16-k step ks
  auto afrag = [&](int buf, int j, int ks) {
    const int m = wm * WTM + j * 32 + l32;
    return *(const u32x4*)&As[buf][m * BK + (((2 * ks + hi) ^ a_swz(m)) * 8)];
  };
  // Wᵀ (MFMA A operand) for n block i, 16-k step ks: lane l32 = column n,
  // k = 8·hi + 0..7, from two transposing reads of 4 k rows each (lane i16
  // of a 16-lane group points at row i16 / 4 and at columns 4·(i16 % 4)..+3)
  auto wfrag = [&](int buf, int i, int ks) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = ks * 16 + 8 * hi + 4 * e + (i16 >> 2);
      const int n = wn * WTN + i * 32 + 16 * g16 + 4 * (i16 & 3);
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)&Ws[buf][k * TN + (((n >> 3) ^ w_swz(k)) * 8) + (n & 7)]);
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * e] = w[0];
      r[2 * e + 1] = w[1];
    }
    return r;
  };

  f32x16 acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x16{};

  // Loads run NSTAGE - 1 stages ahead.  Before each barrier a wave waits
  // until its loads of the next stage have landed; the ones issued for
  // later stages (ACH + WCH instructions each) may stay in flight.
  constexpr int PER = ACH + WCH;
  auto wait_next = [&](int ahead) {  // ahead = stages issued beyond the next one
    if (ahead >= 2 && NSTAGE >= 4)
      __builtin_amdgcn_s_waitcnt(0x0070 | ((2 * PER) & 15) | (((2 * PER) >> 4) << 14));
    else if (ahead >= 1 && NSTAGE >= 3)
      __builtin_amdgcn_s_waitcnt(0x0070 | (PER & 15) | ((PER >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  };
  const int nk = g.K / BK;
#pragma unroll
  for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
    if (s0 < nk) gload(s0, s0);
  wait_next(min(nk - 1, NSTAGE - 1) - 1);
  asm volatile("s_barrier" ::: "memory");
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % NSTAGE;
    // stage (kt - 1) % NSTAGE was last read in step kt - 1, which every wave has left
    if (kt + NSTAGE - 1 < nk) gload(kt + NSTAGE - 1, (kt + NSTAGE - 1) % NSTAGE);
    // fragments of the next 16-k step are read while this step's MFMAs run
    u32x4 wf[2][WN], af[2][WM];
#pragma unroll
    for (int i = 0; i < WN; ++i) wf[0][i] = wfrag(buf, i, 0);
#pragma unroll
    for (int j = 0; j < WM; ++j) af[0][j] = afrag(buf, j, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < WN; ++i) wf[cur ^ 1][i] = wfrag(buf, i, ks + 1);
#pragma unroll
        for (int j = 0; j < WM; ++j) af[cur ^ 1][j] = afrag(buf, j, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WM; ++j) acc[i][j] = mfma_32x32x16<DT>(wf[cur][i], af[cur][j], acc[i][j]);
    }
    // stage kt + 1 landed, this stage's reads done (lgkmcnt 0)
    wait_next(min(nk - 1, kt + NSTAGE - 1) - (kt + 1));
    asm volatile("s_barrier" ::: "memory");
  }

  if (P.R) {
    // residual added, fp32 output in the plain [M, N] layout
    const uint16_t* Rg = (const uint16_t*)P.R;
    float* Cf = (float*)P.C;
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int m = m0 + wm * WTM + j * 32 + l32;
      if (m >= P.M) continue;
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * WTN + i * 32 + gq * 8 + hi * 4;
          const f32x4 r = unpack4<DT>(*(const u32x2*)(Rg + (int64_t)m * P.ldr + n));
          const f32x4 v = {acc[i][j][4 * gq] + r[0], acc[i][j][4 * gq + 1] + r[1],
                           acc[i][j][4 * gq + 2] + r[2], acc[i][j][4 * gq + 3] + r[3]};
          *(f32x4*)(Cf + (int64_t)m * P.c_st + n) = v;
        }
    }
    return;
  }
  // The head split is computed once per 32-column block.  A lane stores
  // columns 8·gq + 4·hi .. +3 of the block; with head_dim a multiple of 32
  // they all belong to the block's head, with head_dim 16 the block holds
  // two heads and gq >= 2 falls in the second (head_dim is 16 or a multiple
  // of 32).
  int64_t col_off[WN];
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const int nb = n0 + wn * WTN + i * 32;
    col_off[i] = (int64_t)(nb / P.head_dim) * P.c_sh + nb % P.head_dim;
  }
  const int64_t half_step = P.head_dim == 16 ? P.c_sh : 16;  // offset of columns 16..31
  uint16_t* Cg = (uint16_t*)P.C;
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int m = m0 + wm * WTM + j * 32 + l32;
    if (m >= P.M) continue;
    const int bb = m / P.rows_per_b, tt = m % P.rows_per_b;
    uint16_t* crow = Cg + (int64_t)bb * P.c_sb + (int64_t)tt * P.c_st;
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int ga = 2 * gp, gb = 2 * gp + 1;
        const u32x2 wa = {pack2<DT>(acc[i][j][4 * ga], acc[i][j][4 * ga + 1]),
                          pack2<DT>(acc[i][j][4 * ga + 2], acc[i][j][4 * ga + 3])};
        const u32x2 wb = {pack2<DT>(acc[i][j][4 * gb], acc[i][j][4 * gb + 1]),
                          pack2<DT>(acc[i][j][4 * gb + 2], acc[i][j][4 * gb + 3])};
        // one 16-byte store per lane (the stores of every tile go out
        // together at the end; half as many requests measured the big
        // cross-attention sub-layer 7.9 % faster)
        const u32x4 w = row_pair_pieces(wa, wb, hi);
        *(u32x4*)(crow + col_off[i] + gp * half_step + 8 * hi) = w;
      }
  }
}

template <int DT, int TM, int TN, int WTM, int WTN, int NSTAGE, int BK = 64>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  if (a.K % BK != 0) return hipErrorInvalidValue;
  int max_tiles = 0;
  for (int i = 0; i < a.nprob; ++i) {
    const int t = ((a.prob[i].M + TM - 1) / TM) * (a.N / TN);
    max_tiles = t > max_tiles ? t : max_tiles;
  }
  if (max_tiles == 0) return hipSuccess;
  constexpr int threads = (TM / WTM) * (TN / WTN) * 64;
  hipLaunchKernelGGL((gemm_kernel<DT, TM, TN, WTM, WTN, NSTAGE, BK>), dim3(max_tiles, a.nprob), dim3(threads), 0,
                     st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs& a, hipStream_t st) {
  // The largest tile that still gives every CU a workgroup: bigger tiles
  // load fewer bytes per flop.
  auto tiles = [&](int tm, int tn) {
    int64_t t = 0;
    for (int i = 0; i < a.nprob; ++i) t += ((a.prob[i].M + tm - 1) / tm) * (int64_t)(a.N / tn);
    return t;
  };
  // (256 x 128 tiles of eight 64 x 64 waves, 192 x 128, 384 x 128 and
  // 64 x 128 tiles measured slower: three 128 x 128 workgroups a CU balance
  // the bytes staged per flop against the waves that hide each other's waits)
  if (a.N % 128 == 0 && tiles(128, 128) >= GEMM_BIG_MIN)
    return launch_t<DT, 128, 128, GEMM_WTM_128, GEMM_WTN_128, GEMM_STAGES_128, GEMM_BK_128>(a, st);
  // 64 x 64 tiles: 128 k a stage (64 KB of LDS, two workgroups a CU, half
  // the dependent load-and-multiply steps) where the grid fits at two a CU
  // (the base encoder's W^O: 1.3 % on its sub-layer; the 768 tiles of the
  // big cross-attention's W^O lost 4 % to the lower occupancy)
  if (a.K % 128 == 0 && tiles(64, 64) <= GEMM_SMALL_GRID)
    return launch_t<DT, 64, 64, 32, 32, GEMM_STAGES_64, 128>(a, st);
  return launch_t<DT, 64, 64, 32, 32, GEMM_STAGES_64>(a, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t st) {
  if (a.N % 64 != 0 || a.K % 64 != 0) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_dt<DT_BF16>(a, st) : launch_dt<DT_F16>(a, st);
}

}  // namespace mha
