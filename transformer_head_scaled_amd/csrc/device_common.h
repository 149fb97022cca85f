// Device-side helpers shared by the libmha kernels (gfx950 / CDNA4 only).
//
// Vector types for the 32x32x16 MFMA operands, raw 16-byte LDS/global
// words, dtype tags and conversions.  Nothing here computes attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;  // LDS-qualified, for ds_read_tr

// D(32x32, fp32) += A(32x16) * B(16x32); 8 half-precision values per lane.
// Operand layout (lane l, element j): A[row l%32][k 8*(l/32)+j],
// B[k 8*(l/32)+j][col l%32].  Result (lane l, element i):
// D[row 8*(i/4) + 4*(l/32) + i%4][col l%32].
template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 values -> one dword holding two half-precision values (RNE),
// low half = a.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == DT_BF16) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Four half-precision values (two dwords, element 0 in the low half of the
// first) -> floats, exactly.  (fp16: one bit cast of the whole 8 bytes;
// casting the two dwords to half pairs one by one was compiled as if both
// held the first pair.)
template <int DT>
__device__ __forceinline__ f32x4 unpack4(u32x2 w) {
  if constexpr (DT == DT_BF16) {
    return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xffff0000u),
                 __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xffff0000u)};
  } else {
    const f16x4 h = __builtin_bit_cast(f16x4, w);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
}

// Non-finite half-precision values.  A 16-bit value is NaN or ±inf exactly
// when its magnitude bits (sign cleared) reach the all-ones exponent:
// 0x7f80 for bf16, 0x7c00 for fp16.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ constexpr unsigned short nonfinite_from() {
  return DT == DT_BF16 ? 0x7f80 : 0x7c00;
}
// Running per-half maximum of the magnitude bits of packed words (two
// instructions per word: an AND and a packed 16-bit max).
__device__ __forceinline__ u16x2 magnitude_max(u16x2 acc, uint32_t w) {
  return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w & 0x7fff7fffu));
}
// A packed word with its non-finite halves replaced by +0.
template <int DT>
__device__ __forceinline__ uint32_t zero_nonfinite(uint32_t w) {
  constexpr uint32_t lim = nonfinite_from<DT>();
  const uint32_t lo = (w & 0x7fffu) >= lim ? 0u : 0x0000ffffu;
  const uint32_t hi = ((w >> 16) & 0x7fffu) >= lim ? 0u : 0xffff0000u;
  return w & (lo | hi);
}

// Sign bit of each 16-bit lane of a packed word (used to negate operands
// exactly).
__device__ __forceinline__ u32x4 flip_signs(u32x4 v) {
  const uint32_t s = 0x80008000u;
  return u32x4{v[0] ^ s, v[1] ^ s, v[2] ^ s, v[3] ^ s};
}

// Combine a value with the one held by the lane 32 positions away
// (lane l and lane l^32).  v_permlane32_swap exchanges the upper half of
// one register with the lower half of the other; applied to two copies of
// x it leaves x's lower half in one result and its upper half in the
// other, in every lane, so max/sum of the two is the pair's max/sum.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Output stores of a 32x32 MFMA result held one row per lane pair: lanes
// l and l + 32 hold the same row, lane hi = 0 columns 0..3 and 8..11 of a
// 16-column group, lane hi = 1 columns 4..7 and 12..15 (each 4-column
// piece as two packed pairs: a = the piece at 4·hi, b = the one at
// 8 + 4·hi).  Swapping one piece with the partner gives lane hi = 0
// columns 0..7 and lane hi = 1 columns 8..15: one 16-byte store per lane
// at column 8·hi instead of two of 8 bytes.  Both lanes of a pair must be
// active.
__device__ __forceinline__ u32x4 row_pair_pieces(u32x2 a, u32x2 b, int hi) {
  const u32x2 send = hi ? a : b;
  const auto r0 = __builtin_amdgcn_permlane32_swap(send[0], send[0], false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(send[1], send[1], false, false);
  // lanes 0..31 find the partner's value in the second result, 32..63 in the first
  const uint32_t q0 = hi ? (uint32_t)r0[0] : (uint32_t)r0[1];
  const uint32_t q1 = hi ? (uint32_t)r1[0] : (uint32_t)r1[1];
  return hi ? u32x4{q0, q1, b[0], b[1]} : u32x4{a[0], a[1], q0, q1};
}

// 1 / (a row's weight sum), for the normalisation.  A sum of 0 means no
// visible key (the row's output is 0) or, with visible keys, only scores of
// −∞ among them -- infinite inputs; the exact softmax is then 0/0, NaN.  (A
// visible key with a finite score adds exp2(0) = 1 to the sum: the largest
// one is the reference value or beats it.)
__device__ __forceinline__ float row_sum_inverse(float sum, bool visible) {
  return sum > 0.f ? 1.f / sum : (visible ? __builtin_nanf("") : 0.f);
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// 16 bytes per lane from a raw buffer (descriptor rsrc, byte offset voff)
// straight into LDS: lane i writes bytes [lds + 16i, lds + 16i + 16).  Out-of-
// range offsets read as zero.  Written as inline assembly so that the
// compiler does not treat every later LDS read as a possible alias of the
// transfer and wait for it; the caller orders it with explicit waits and
// barriers instead.  M0 (the LDS base of the transfer) is set here; nothing
// else in these kernels reads M0, and the compiler treats it as reserved.
__device__ __forceinline__ void load_lds_b128(u32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

// Raw buffer descriptor words for `base` with a range of `bytes` bytes
// (stride 0, the data format word the gfx950 raw buffer loads use).  Loads
// at offsets >= bytes return zero.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Map the hardware workgroup index onto a logical tile index so that
// consecutive logical tiles run on the same XCD (workgroups are dealt to
// the 8 XCDs round-robin; each XCD has its own L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t hw, uint32_t total) {
  const uint32_t nx = 8;
  const uint32_t xcd = hw % nx, slot = hw / nx;
  const uint32_t per = total / nx, extra = total % nx;
  return xcd * per + (xcd < extra ? xcd : extra) + slot;
}

}  // namespace mha
