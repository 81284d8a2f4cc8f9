// device_common.h -- gfx950 device helpers shared by the libgdn kernels.
//
// Matrix products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16: 16x16 fp32
// accumulator, contraction 32, one 64-lane wave).  The state and every intermediate
// of the chunk transform are fp32; a product with an fp32 operand splits it into a sum
// of bf16 terms (x = t0 + t1 [+ t2], each term the bf16 rounding of what the earlier
// terms left) and accumulates the cross products whose combined order is small
// enough.  With bf16 inputs: two terms, products of order <= 1 (error ~2^-16
// relative per product); with fp32 inputs: three terms, order <= 2 (~2^-24).  bf16
// input values are exact in one term.
//
// Register layout of the 16x16x32 bf16 MFMA (lane l, g = l / 16):
//   A (16 x 32): row l % 16, contraction elements 8g .. 8g+7
//   B (32 x 16): column l % 16, contraction elements 8g .. 8g+7
//   C (16 x 16): column l % 16, rows 4g .. 4g+3
// The contraction index is a dummy, so any permutation applied to both operands
// gives the same sum.  All products here use the permutation
//   kappa(s, g, e) = 32 s + 16 (e / 4) + 4 g + (e % 4)      (k-step s, element e),
// under which the C layout of one product (rows 16 m + 4 g + r of tile m) is directly
// the B operand of the next one (tiles 2s and 2s+1 give elements 0..3 and 4..7).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint16_t bf16_bits;

// Precision policy per io type: terms of an input operand, terms of an fp32 operand,
// highest product order kept.
template <typename IO>
struct Prec;
template <>
struct Prec<bf16_bits> {
  static constexpr int NTI = 1, NTF = 2, ORD = 1;
};
template <>
struct Prec<float> {
  static constexpr int NTI = 3, NTF = 3, ORD = 2;
};

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even (the conversion instruction of gfx950).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_bits, h);
}
// Two values rounded to bf16 (nearest even) in one conversion; lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
}
__device__ __forceinline__ float to_f32(bf16_bits x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename IO>
__device__ __forceinline__ IO from_f32(float x);
template <>
__device__ __forceinline__ bf16_bits from_f32<bf16_bits>(float x) { return f32_to_bf16(x); }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Split x into NT bf16 terms; returns their bit patterns.
template <int NT>
__device__ __forceinline__ void split_terms(float x, bf16_bits (&t)[NT]) {
  float r = x;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i] = f32_to_bf16(r);
    if (i + 1 < NT) r = r - bf16_to_f32(t[i]);
  }
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += sum over term pairs (i, j) with i + j <= ORD of A_i * B_j; the smallest
// orders are accumulated first.
template <int NA, int NB, int ORD>
__device__ __forceinline__ void mma_terms(f32x4& acc, const bf16x8 (&a)[NA], const bf16x8 (&b)[NB]) {
#pragma unroll
  for (int o = ORD; o >= 0; --o) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int j = o - i;
      if (j >= 0 && j < NB) acc = mfma(a[i], b[j], acc);
    }
  }
}

// Pack 8 bf16 bit patterns into an MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const bf16_bits (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = __builtin_bit_cast(__bf16, v[e]);
  return r;
}

// Operand from two runs of 4 bf16 in LDS (elements 0..3 at p0, 4..7 at p1).
__device__ __forceinline__ bf16x8 lds_operand(const bf16_bits* p0, const bf16_bits* p1) {
  uint2 lo = *reinterpret_cast<const uint2*>(p0);
  uint2 hi = *reinterpret_cast<const uint2*>(p1);
  typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
  u32x4 w = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, w);
}

// Operand terms from fp32 register values laid out as the C tiles 2s and 2s+1:
// v0 = tile 2s rows 0..3, v1 = tile 2s+1 rows 0..3 (pass zeros for a missing tile).
// Elements are split two at a time: one packed conversion gives a pair's term, whose
// two halves widen back to fp32 by a shift and a mask (the same values split_terms
// forms one element at a time).
template <int NT>
__device__ __forceinline__ void reg_operand(const f32x4& v0, const f32x4& v1, bf16x8 (&out)[NT]) {
  typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
  const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t w[NT][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a = x[2 * k], b = x[2 * k + 1];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint32_t pr = pack_bf16x2(a, b);  // element 2k in the low half
      w[i][k] = pr;
      if (i + 1 < NT) {
        a = a - __uint_as_float(pr << 16);
        b = b - __uint_as_float(pr & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) out[i] = __builtin_bit_cast(bf16x8, u32x4_t{w[i][0], w[i][1], w[i][2], w[i][3]});
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-byte store written through to device-coherent memory (sc1): the lines do not sit
// dirty in the L2 of one XCD until the end-of-kernel write-back, so for a state written
// once and read by a later launch the write traffic overlaps the rest of the kernel.
// No builtin sets the scope bits of a 16-byte store (atomic stores stop at 8 bytes, and
// two 8-byte halves of each 16-byte piece leave every write partial), hence the asm.
// The compiler checks no hazards for the instructions inside an asm statement: the
// leading 24 wait states cover a read of a matrix-core result (19 for the longest
// 16-pass instructions); its write-after-read check on the data registers does hold.
__device__ __forceinline__ void store16_through(float* p, const f32x4& v) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\tglobal_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wave-wide inclusive prefix sum (64 lanes), fixed combination order, in DPP moves (no
// LDS round trips): within each 16-lane row by right shifts of 1, 2, 4 and 8 lanes,
// then the total of rows 0 and 2 (their lane 15) into rows 1 and 3, then the total of
// rows 0-1 (lane 31) into rows 2 and 3.  Lanes a shift leaves without a source add 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x = dpp_add<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// The same prefix sum through LDS lane permutes (ds_bpermute), doubling the shift from
// 1 to 32 lanes.
__device__ __forceinline__ float wave_inclusive_scan_lds(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x = x + y;
  }
  return x;
}

// Value of x in lane i (i wave-uniform).
__device__ __forceinline__ float lane_value(float x, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}

}  // namespace gdn
