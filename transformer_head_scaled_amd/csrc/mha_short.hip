// Short sequences: the Q/K/V projections of one (batch, head) and its
// attention in one workgroup, for mha_forward with n_q, n_k <= 64,
// d_k = d_v = 64 and no causal mask.
//
// "Lire « Attention Is All You Need »" (nickwang.xyz), §3.2.2 "Attention
// multi-têtes": head i attends with Q_i = x_q·W_i^Q, K_i = x_kv·W_i^K,
// V_i = x_kv·W_i^V, where W_i^Q is the i-th 64-column block of the
// [d_model, h·64] matrix; §3.2.1 (eq. (1)): softmax(Q_i·K_iᵀ/√64)·V_i, the
// padding keys of a sequence masked.  The head's output goes into columns
// [i·64, i·64 + 64) of the concat; the W^O product runs afterwards (the
// projection GEMM).
//
// For these sizes the separate launches are bound by latency (a few k
// steps each, one key tile) rather than by MFMA or HBM rate, and the
// projected Q/K/V make a round trip through memory.  Here one workgroup of
// 4 waves computes, per 64-wide k step of d_model, the three 64×64 products
// of its head (waves 0, 1, 2: Q, K, V, each Cᵀ = Wᵀ·Xᵀ with the 32x32x16
// MFMA, fragments as in the projection GEMM), rounds them to the storage
// type once (as the separate path does when it stores them), writes them
// into LDS in the layouts of the flash kernel's tiles, and then waves 0 and
// 1 each take one 32-row query block against the (at most 64) keys: scores
// Sᵀ = K·Qᵀ, the exact softmax of one tile (row max first), Oᵀ = Vᵀ·Pᵀ,
// normalised and stored into the concat.
//
// Key padding: rows of x_kv at or past the sequence's key length enter the
// K and V products as zeros (their fragments are cleared), so K and V rows
// there are exactly 0 whatever x_kv holds, and their scores are masked.

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int SBK = 64;  // k per stage
#ifndef MHA_SHORT_STAGES
#define MHA_SHORT_STAGES 4
#endif
constexpr int SN = 64;   // rows (queries, keys) and head columns per tile

// chunk permutations (16-byte chunks, 8 per 128-byte row).  X tiles and the
// Q/K tiles: chunk c of row r at c ^ ((r >> 1) & 7), so that 16 lanes
// reading one chunk index of 16 consecutive rows cover all banks; W tiles:
// chunk c of k row k at c ^ 4·((k >> 1) & 1), for the transposing reads of
// 4 consecutive k rows; V tile: chunk c of key k at c ^ 4·((k >> 1) & 1),
// likewise.
__device__ __forceinline__ int row_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int pair_swz(int k) { return 4 * ((k >> 1) & 1); }

// A ring of NST stages: the loads run NST − 1 steps ahead (one step's
// products take far less time than the loads' latency).
template <int DT, bool SELF, int NST>
__global__ __launch_bounds__(256) void mha_short_kernel(ShortArgs a) {
  // per stage: X_q, X_kv (cross-attention only) and the three W column blocks
  constexpr int XT = SN * SBK, WT = SBK * SN;  // elements per tile
  constexpr int NX = SELF ? 1 : 2;             // X tiles per stage
  constexpr int NPIECE = NX * 8 + 24;          // 1 KB pieces per stage
  constexpr int PER = NPIECE / 4;              // load instructions per wave and stage
  static_assert(NPIECE % 4 == 0 && (NST - 2) * PER < 64, "loads per wave, vmcnt range");
  __shared__ __attribute__((aligned(16))) uint16_t lds[NST][NX * XT + 3 * WT];
  const uint32_t total = (uint32_t)a.B * a.H;
  const uint32_t t = xcd_remap(blockIdx.x, total);  // the heads of a batch on one XCD
  const int b = (int)(t / a.H), hh = (int)(t % a.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5, i16 = lane & 15, g16 = (lane >> 4) & 1;

  int n_eff = a.n_k;
  if (a.lens) n_eff = min(max(a.lens[b], 0), a.n_k);
  const int64_t dm = a.d_model, ldw = (int64_t)a.H * SN;

  // ---- staging: X tiles (64 rows × 64 k) and W tiles (64 k × 64 columns)
  // go from memory straight into LDS; X rows past the range read as zero
  const uint16_t* xq = (const uint16_t*)a.xq + (int64_t)b * a.n_q * dm;
  const uint16_t* xkv = (const uint16_t*)a.xkv + (int64_t)b * a.n_k * dm;
  const u32x4 rq = raw_rsrc(xq, (uint32_t)(a.n_q * dm * 2));
  const u32x4 rkv = raw_rsrc(xkv, (uint32_t)(n_eff * dm * 2));
  // the 1 KB piece p of a tile: lane -> LDS chunk q = 64p + lane
  auto x_off = [&](int p) {
    const int q = p * 64 + lane, r = q >> 3;
    return (uint32_t)(r * dm * 2 + ((q & 7) ^ row_swz(r)) * 16);
  };
  auto w_off = [&](int p) {
    const int q = p * 64 + lane, k = q >> 3;
    return (uint32_t)(k * ldw * 2 + ((q & 7) ^ pair_swz(k)) * 16);
  };
  // pieces 0..7: X_q; then 8..15: X_kv (cross only); then W_q, W_k, W_v
  auto gload = [&](int kt, int stage) {
    const int k0 = kt * SBK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = wave + 4 * i;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&lds[stage][p * 512]);
      if (p < NX * 8) {
        load_lds_b128(p < 8 ? rq : rkv, dst, x_off(p & 7) + k0 * 2);
      } else {
        const int w = (p - NX * 8) >> 3;
        const uint16_t* wsrc = (const uint16_t*)(w == 0 ? a.Wq : w == 1 ? a.Wk : a.Wv) + hh * SN;
        const u32x4 rw = raw_rsrc(wsrc + (int64_t)k0 * ldw, (uint32_t)(SBK * ldw * 2));
        load_lds_b128(rw, dst, w_off((p - NX * 8) & 7));
      }
    }
  };
  // wait until this wave's loads of the next stage have landed, leaving
  // those of the `ahead` stages issued after it in flight
  auto wait_next = [&](int ahead) {
    if (ahead >= 2 && NST >= 4)
      __builtin_amdgcn_s_waitcnt(0x0070 | ((2 * PER) & 15) | (((2 * PER) >> 4) << 14));
    else if (ahead >= 1 && NST >= 3)
      __builtin_amdgcn_s_waitcnt(0x0070 | (PER & 15) | ((PER >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  };

  // ---- phase 1: wave w < 3 computes projection w (Q, K, V) of this head
  const int mat = wave;
  const int xsel = (mat == 0 || SELF) ? 0 : 1;  // its X tile
  // K and V: rows at or past the key length enter as zeros
  const int rows_valid = mat == 0 ? a.n_q : n_eff;
  auto xfrag = [&](int buf, int j, int ks) {  // Xᵀ (B operand), row block j
    const int m = j * 32 + l32;
    u32x4 v = *(const u32x4*)&lds[buf][xsel * XT + m * SBK + (((2 * ks + hi) ^ row_swz(m)) * 8)];
    if (m >= rows_valid) v = u32x4{0u, 0u, 0u, 0u};
    return v;
  };
  auto wfrag = [&](int buf, int i, int ks) {  // Wᵀ (A operand), column block i
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = ks * 16 + 8 * hi + 4 * e + (i16 >> 2);
      const int n = i * 32 + 16 * g16 + 4 * (i16 & 3);
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)&lds[buf][NX * XT + mat * WT + k * SN + (((n >> 3) ^ pair_swz(k)) * 8) + (n & 7)]);
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * e] = w[0];
      r[2 * e + 1] = w[1];
    }
    return r;
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = a.d_model / SBK;
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < nk) gload(s0, s0);
  wait_next(min(nk - 1, NST - 1) - 1);
  asm volatile("s_barrier" ::: "memory");
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % NST;
    // stage (kt − 1) % NST was last read in step kt − 1, which every wave has left
    if (kt + NST - 1 < nk) gload(kt + NST - 1, (kt + NST - 1) % NST);
    if (mat < 3) {
      // every fragment of the stage first, then its MFMAs (pinned by the
      // schedule groups): with one wave a SIMD nothing else hides a read's
      // latency, and the compiler would otherwise read each 16-k step's
      // fragments just before their MFMAs (+2-3 % on the base encoder
      // sub-layer, identical results)
      u32x4 wf[SBK / 16][2], xf[SBK / 16][2];
#pragma unroll
      for (int ks = 0; ks < SBK / 16; ++ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) wf[ks][i] = wfrag(buf, i, ks);
#pragma unroll
        for (int j = 0; j < 2; ++j) xf[ks][j] = xfrag(buf, j, ks);
      }
#pragma unroll
      for (int ks = 0; ks < SBK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16<DT>(wf[ks][i], xf[ks][j], acc[i][j]);
      __builtin_amdgcn_sched_group_barrier(0x100, (SBK / 16) * 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, (SBK / 16) * 4, 0);
    }
    // stage kt + 1 landed, this stage's reads done
    wait_next(min(nk - 1, kt + NST - 1) - (kt + 1));
    asm volatile("s_barrier" ::: "memory");
  }

  // ---- the projections into LDS (stage 0 is free now), rounded once:
  // Q and K at chunk c ^ row_swz(row), V at c ^ pair_swz(key).  A lane holds
  // columns 8·gq + 4·hi .. +3 of column block i for row j·32 + l32.
  static_assert(NX * XT + 3 * WT >= 3 * XT, "stage 0 holds the three tiles");
  uint16_t* const tq = &lds[0][0];
  uint16_t* const tk = &lds[0][XT];
  uint16_t* const tv = &lds[0][2 * XT];
  if (mat < 3) {
    uint16_t* const dst = mat == 0 ? tq : mat == 1 ? tk : tv;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = j * 32 + l32;
      const int sw = mat == 2 ? pair_swz(r) : row_swz(r);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int ch = i * 4 + gq;
          const u32x2 w = {pack2<DT>(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]),
                           pack2<DT>(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
          *(u32x2*)&dst[r * SN + ((ch ^ sw) * 8) + 4 * hi] = w;
        }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");

  // ---- phase 2: waves 0 and 1, query rows [32·wave, 32·wave + 32)
  if (wave >= 2 || wave * 32 >= a.n_q) return;
  const int row = wave * 32 + l32;
  u32x4 qf[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) qf[st] = *(const u32x4*)&tq[row * SN + (((2 * st + hi) ^ row_swz(row)) * 8)];
  // Sᵀ of key block kb: lane holds keys kb·32 + 8·(i / 4) + 4·hi + i % 4
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    const int key = kb * 32 + l32;
#pragma unroll
    for (int st = 0; st < 4; ++st)
      s[kb] = mfma_32x32x16<DT>(*(const u32x4*)&tk[key * SN + (((2 * st + hi) ^ row_swz(key)) * 8)], qf[st],
                                s[kb]);
    const int lim = n_eff - kb * 32 - 4 * hi;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) >= lim) s[kb][i] = -INFINITY;
  }
  // the exact softmax of the one tile: row max, weights, row sum
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  mx = pair_max(mx);
  const float mc = (mx == -INFINITY ? 0.f : mx) * a.c;
  uint32_t pw[2][8];
  float l = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * i], a.c, -mc));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * i + 1], a.c, -mc));
      pw[kb][i] = pack2<DT>(e0, e1);
      r0 += e0;
      r1 += e1;
    }
    l += r0 + r1;
  }
  // Oᵀ = Vᵀ·Pᵀ.  Vᵀ fragment (kb, t2, db): d = db·32 + column, the 8 keys
  // the score registers hold for this lane half, two transposing reads of 4
  const int v_key_l = 4 * hi + (i16 >> 2);
  const int v_col = 16 * g16 + 4 * (i16 & 3);
  f32x16 o[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        u32x4 vf;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int key = kb * 32 + t2 * 16 + 8 * e + v_key_l;
          const int d = db * 32 + v_col;
          const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)&tv[key * SN + (((d >> 3) ^ pair_swz(key)) * 8) + (d & 7)]);
          const u32x2 w = __builtin_bit_cast(u32x2, v);
          vf[2 * e] = w[0];
          vf[2 * e + 1] = w[1];
        }
        const u32x4 bv = {pw[kb][4 * t2], pw[kb][4 * t2 + 1], pw[kb][4 * t2 + 2], pw[kb][4 * t2 + 3]};
        o[db] = mfma_32x32x16<DT>(vf, bv, o[db]);
      }
  // normalise, store columns hh·64 + d of the concat row
  const float L = pair_sum(l);
  const float inv = row_sum_inverse(L, n_eff > 0);
  if (row < a.n_q) {
    uint16_t* crow = (uint16_t*)a.C + ((int64_t)b * a.n_q + row) * ldw + hh * SN;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x2 w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int g = 2 * gp + e;
          w[e] = u32x2{pack2<DT>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                       pack2<DT>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        }
        *(u32x4*)(crow + db * 32 + gp * 16 + 8 * hi) = row_pair_pieces(w[0], w[1], hi);
      }
  }
}

}  // namespace

hipError_t launch_mha_short(const ShortArgs& a, int dtype, hipStream_t st) {
  if (a.n_q < 1 || a.n_q > 64 || a.n_k < 1 || a.n_k > 64 || a.d_model % SBK != 0 || a.d_model <= 0 ||
      (a.self && a.n_q != a.n_k))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)a.B * a.H));
  // four stages: 128 KB of LDS (self-attention), 160 KB (cross)
  constexpr int S = MHA_SHORT_STAGES;
  if (dtype == DT_BF16) {
    if (a.self)
      hipLaunchKernelGGL((mha_short_kernel<DT_BF16, true, S>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((mha_short_kernel<DT_BF16, false, S>), grid, dim3(256), 0, st, a);
  } else if (dtype == DT_F16) {
    if (a.self)
      hipLaunchKernelGGL((mha_short_kernel<DT_F16, true, S>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((mha_short_kernel<DT_F16, false, S>), grid, dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mha
