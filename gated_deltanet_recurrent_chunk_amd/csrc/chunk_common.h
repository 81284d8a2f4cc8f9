// chunk_common.h -- device helpers shared by the chunk kernels (prefill and replay flush).
//
// The chunked (WY / UT transform) form of the gated delta rule (Yang, Kautz &
// Hatamizadeh, "Gated Delta Networks", ICLR 2025; the chunkwise delta rule of Yang et
// al., "Parallelizing Linear Transformers with the Delta Rule over Sequence Length",
// NeurIPS 2024).  For a chunk of n <= 64 rows entering with state S_0 (d_v x d_k):
//
//   g_t   = sum_{i<=t} log a_i
//   A_ts  = b_t exp(g_t - g_s) k_t . k_s   (s < t),     T = (I + A)^-1
//   R     = diag(b) (V - diag(exp g) K S_0^T)           Delta = T R
//   O     = scale (diag(exp g) Q S_0^T + P Delta),       P_ts = exp(g_t - g_s) q_t . k_s (s <= t)
//   S_n   = exp(g_n) S_0 + Delta^T diag(exp(g_n - g)) K
//
// Row t of Delta is b_t (v_t - a_t S_{t-1} k_t), the correction written at token t.
// Gates stay in log space and only exp(g_t - g_s) with s <= t is formed, so no factor
// exceeds one.  Rows past the chunk length n are excluded by selection wherever they
// could reach a result, never by multiplying with a mask.
//
// LDS operand planes.  A matrix used as an MFMA A operand is kept in LDS as bf16 planes
// (one per term), row-major, with the columns of every 32-wide block stored in the
// order swz(): 4-column groups 0,4,1,5,2,6,3,7.  The eight contraction elements a lane
// supplies for k-step s (kappa(s, g, 0..7), see device_common.h) are then the eight
// adjacent physical columns 32 s + 8 g .. +7: one 16-byte LDS read per operand.
// Two row layouts are used:
//   padded: rows of phys_width + 8 elements (16 bytes more than a multiple of 128);
//   xor:    unpadded rows whose 16-byte pieces are permuted by an XOR with a key taken
//           from the row index (xkey), so that the 16 rows of one operand read land in
//           16 distinct 16-byte bank slots.  Unpadded rows can be filled by LDS DMA.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "plan.h"

namespace gdn {
namespace chunk {


// Physical column of logical column c inside its 32-column block (see above).
__host__ __device__ constexpr int swz(int c) {
  return (c & ~31) | (((((c >> 2) & 3) << 1) | ((c >> 4) & 1)) << 2) | (c & 3);
}

// Physical width (elements) of an operand row of logical length len, and its padded stride.
__host__ __device__ constexpr int phys_width(int len) { return len < 32 ? 32 : len; }
__host__ __device__ constexpr int row_stride(int len) { return phys_width(len) + 8; }

__device__ __forceinline__ bf16x8 op_read(const bf16_bits* plane, int ld, int row, int s, int g) {
  return *reinterpret_cast<const bf16x8*>(plane + row * ld + 32 * s + 8 * g);
}

template <int NT>
__device__ __forceinline__ void op_terms(const bf16_bits* planes, int pstride, int ld, int row, int s, int g,
                                         bf16x8 (&out)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) out[i] = op_read(planes + i * pstride, ld, row, s, g);
}

// 16-byte global load (zeros when !pred: the row is not read).
__device__ __forceinline__ uint4 load16(const void* p, bool pred) {
  if (pred) return *reinterpret_cast<const uint4*>(p);
  return uint4{0u, 0u, 0u, 0u};
}

template <typename IO>
__device__ __forceinline__ float elem(const uint4& v, int e) {
  if constexpr (sizeof(IO) == 2) {
    uint32_t w = (&v.x)[e >> 1];
    return bf16_to_f32((bf16_bits)((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
  } else {
    return __uint_as_float((&v.x)[e]);
  }
}

// Store the 16 bytes of io elements at logical row t, columns j0.. into NT swizzled
// bf16 planes (terms of each value).
template <typename IO, int NT>
__device__ __forceinline__ void store_row_terms(const uint4& v, bf16_bits* planes, int pstride, int ld, int t,
                                                int j0) {
  constexpr int VEC = 16 / sizeof(IO);
#pragma unroll
  for (int grp4 = 0; grp4 < VEC / 4; ++grp4) {
    const int c = j0 + 4 * grp4;
    bf16_bits* dst = planes + t * ld + swz(c);
    if constexpr (NT == 1 && sizeof(IO) == 2) {
      *reinterpret_cast<uint2*>(dst) = uint2{(&v.x)[2 * grp4], (&v.x)[2 * grp4 + 1]};
    } else {
      bf16_bits tt[4][NT];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_terms<NT>(elem<IO>(v, 4 * grp4 + e), tt[e]);
#pragma unroll
      for (int i = 0; i < NT; ++i)
        *reinterpret_cast<uint2*>(dst + i * pstride) =
            uint2{(uint32_t)tt[0][i] | ((uint32_t)tt[1][i] << 16), (uint32_t)tt[2][i] | ((uint32_t)tt[3][i] << 16)};
    }
  }
}

__device__ __forceinline__ void zero_lds(void* p, int bytes, int tid, int nth) {
  uint4* q = reinterpret_cast<uint4*>(p);
  for (int i = tid; i < bytes / 16; i += nth) q[i] = uint4{0u, 0u, 0u, 0u};
}

// K^T planes (rows j, swizzled columns t, row stride dld) from the swizzled key-row
// planes Ks (row stride KP): 4 columns per 8-byte store.
template <int CT, int D, int NTI>
__device__ __forceinline__ void transpose_keys(const bf16_bits* Ks, int KP, bf16_bits* dst, int dps, int dld,
                                               int tid, int nth) {
  for (int task = tid; task < NTI * D * (CT / 4); task += nth) {
    const int i = task / (D * (CT / 4));
    const int rem = task % (D * (CT / 4));
    const int j = rem / (CT / 4), t0 = (rem % (CT / 4)) * 4;
    const bf16_bits* src = Ks + i * CT * KP + swz(j);
    const uint32_t w0 = (uint32_t)src[(t0 + 0) * KP] | ((uint32_t)src[(t0 + 1) * KP] << 16);
    const uint32_t w1 = (uint32_t)src[(t0 + 2) * KP] | ((uint32_t)src[(t0 + 3) * KP] << 16);
    *reinterpret_cast<uint2*>(dst + i * dps + j * dld + swz(t0)) = uint2{w0, w1};
  }
}

// Barrier among the waves of a workgroup that orders LDS traffic only (outstanding
// global loads, stores and LDS DMA are not waited for).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Barrier that also completes this wave's outstanding vector memory operations (LDS DMA
// and stores included) before any wave passes it.  The wait is the builtin, so the
// compiler's own wait accounting sees it: no memory operation issued before the barrier
// is waited for again after it (an inline-asm wait is invisible to that accounting, and
// the compiler would then wait again, for everything pending, at its first read of
// copied data).  The empty asm statements keep memory accesses on their side.
__device__ __forceinline__ void full_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0); expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------------------------
// Chunk factorization shared by the prefill pre-pass and the replay flush.  One wave.
//   Ks: NTI swizzled planes (row stride KP) of the chunk's key rows (rows >= n zero).
//   g, bb: this lane's g_t and b_t for t = lane (t >= n: g_t = g_{n-1}, b_t = 0).
// Writes T = (I + A)^-1 as NTF swizzled bf16 planes (row stride tld, plane stride
// tps) and the four per-row vectors g, exp(g), b, exp(g_n - g) into vec_out.
// FOLD: writes T'' = diag(exp(g_n - g)) T diag(b) to Tout instead, and T^T (unscaled,
// row j = column j of T) to Ttr in the same plane format.
// SPLIT (32-row chunks, no FOLD): the substitution runs on both halves of the wave, see
// below; it holds half the registers of the one-half form.
// Barriers: the first publishes the row vectors to the whole workgroup.  The second
// orders this wave's A tiles before its own substitution reads them: with LOCAL_A it
// is a wait for this wave's LDS traffic only, so the other waves match one barrier and
// are not held while the A tiles are formed.
template <int CT, int D, int NTI, int NTF, int ORD, bool FOLD = false, bool SPLIT = false, bool LOCAL_A = false>
__device__ __forceinline__ void factorize_chunk(const bf16_bits* Ks, int kps, float (*As)[CT + 4], int n,
                                                float g, float bb, bf16_bits* Tout, int tps, int tld,
                                                float* vec_out, float* vec_lds, bf16_bits* Ttr = nullptr) {
  constexpr int KP = row_stride(D);
  constexpr int KSD = (D + 31) / 32;
  constexpr int MT = CT / 16;
  static_assert(!SPLIT || (CT == 32 && !FOLD), "the split substitution covers 32-row chunks");
  // SPLIT layout of A: two planes by the parity of the column s, A[t][s] at
  // (s & 1) * SPL + t * (CT / 2) + (s >> 1); plane 1 starts 4 words further so that the
  // two halves' row reads fall in different banks
  constexpr int HS = CT / 2, SPL = CT * HS + 4;
  float* const A2 = &As[0][0];
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;

  const float gn = __shfl(g, n - 1, 64);
  const bool live = lane < n;
  const float eg = __expf(g);
  const float edec = live ? __expf(gn - g) : 0.f;
  if (lane < CT) {
    vec_lds[lane] = g;
    vec_lds[CT + lane] = bb;
    vec_out[lane] = g;
    vec_out[CT + lane] = eg;
    vec_out[2 * CT + lane] = bb;
    vec_out[3 * CT + lane] = edec;
  }
  lds_barrier();

  // A = strict lower part of diag(b) exp(g_t - g_s) K K^T
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // SPLIT: the substitution never reads rows t >= n, so their tiles are not formed
    if (SPLIT && 16 * mt >= n) break;
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        bf16x8 a[NTI], b[NTI];
        op_terms<NTI>(Ks, kps, KP, 16 * mt + col, s, grp, a);
        op_terms<NTI>(Ks, kps, KP, 16 * nt + col, s, grp, b);
        mma_terms<NTI, NTI, ORD>(acc, a, b);
      }
      const int sc = 16 * nt + col;
      const float gs = vec_lds[sc];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * grp + r;
        // computed for every element (pinned, so that the compiler does not move the LDS
        // reads into a branch per element) and kept or dropped by the select
        float dec = __expf(vec_lds[t] - gs), bt = vec_lds[CT + t];
        asm volatile("" : "+v"(dec), "+v"(bt));
        const float val = (sc < t && t < n) ? bt * dec * acc[r] : 0.f;
        if constexpr (SPLIT)
          A2[(sc & 1) * SPL + t * HS + (sc >> 1)] = val;
        else
          As[t][sc] = val;
      }
    }
  }
  if constexpr (LOCAL_A)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  else
    lds_barrier();

  if constexpr (SPLIT) {
    // Lane (h, j) = (lane >> 5, lane & 31) owns column j of T at the rows s = 2k + h and
    // sums A[t][s] T[s][j] over those rows; one swap of the wave's halves adds the other
    // parity's sum (own + other in both halves: the same value).  The own-parity row t + 1
    // of A is requested before the sums of row t run.  Row t's count is the even
    // parity's, ceil(t / 2); for the odd parity its last term is A[t][t] = 0 times a
    // not yet computed (zero) T entry.  Rows t >= n of A are zero, so T's rows there are
    // those of the identity: with n <= 16 only the first 16 rows are substituted (one
    // uniform branch between two unrolled forms; a branch per row would hold more
    // registers).
    const int hf = lane >> 5, j = lane & 31;
    const float* Ah = A2 + hf * SPL;
    float Tc[HS];
#pragma unroll
    for (int k = 0; k < HS; ++k) Tc[k] = 0.f;
    auto substitute = [&](auto nr_) {
      constexpr int NR = decltype(nr_)::value;
      f32x4 arow[2][HS / 4];
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        if (t + 1 < NR) {
#pragma unroll
          for (int i = 0; i < ((t + 2) / 2 + 3) / 4; ++i)
            arow[(t + 1) & 1][i] = *reinterpret_cast<const f32x4*>(Ah + (t + 1) * HS + 4 * i);
        }
        asm volatile("" ::: "memory");
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int k = 0; k < (t + 1) / 2; ++k) {
          const float av = arow[t & 1][k >> 2][k & 3];
          if ((k & 1) == 0) p0 = fmaf(av, Tc[k], p0);
          else p1 = fmaf(av, Tc[k], p1);
        }
        const float own = p0 + p1;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(own), __float_as_uint(own), false, false);
        const float val = (t == j ? 1.f : 0.f) - (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
        if ((t & 1) == hf) Tc[t >> 1] = val;
        asm volatile("" : "+v"(Tc[t >> 1]) : : "memory");
      }
#pragma unroll
      for (int t = NR; t < CT; ++t)
        if ((t & 1) == hf) Tc[t >> 1] = t == j ? 1.f : 0.f;
    };
    if (n <= CT / 2)
      substitute(std::integral_constant<int, CT / 2>{});
    else
      substitute(std::integral_constant<int, CT>{});
    const int pc = swz(j);
#pragma unroll
    for (int k = 0; k < HS; ++k) {
      bf16_bits tt[NTF];
      split_terms<NTF>(Tc[k], tt);
#pragma unroll
      for (int i = 0; i < NTF; ++i) Tout[i * tps + (2 * k + hf) * tld + pc] = tt[i];
    }
    return;
  }

  // Forward substitution, lane j owns column j:  T[t][j] = [t == j] - sum_{s<t} A[t][s] T[s][j].
  // The sum runs as four interleaved partial sums (s mod 4) added in a fixed order.  Row
  // t + 1 of A is requested from LDS before the sums of row t run, so the LDS latency
  // overlaps them; two rows of A are live in registers.
  float Tc[CT];
  f32x4 arow[2][CT / 4];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    if (t + 1 < CT) {
#pragma unroll
      for (int i = 0; i < (t + 4) / 4; ++i) arow[(t + 1) & 1][i] = *reinterpret_cast<const f32x4*>(&As[t + 1][4 * i]);
    }
    asm volatile("" ::: "memory");
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int s = 0; s < t; ++s) {
      const float av = arow[t & 1][s >> 2][s & 3];
      if ((s & 3) == 0) p0 = fmaf(av, Tc[s], p0);
      if ((s & 3) == 1) p1 = fmaf(av, Tc[s], p1);
      if ((s & 3) == 2) p2 = fmaf(av, Tc[s], p2);
      if ((s & 3) == 3) p3 = fmaf(av, Tc[s], p3);
    }
    Tc[t] = (t == lane ? 1.f : 0.f) - ((p0 + p1) + (p2 + p3));
    // row t is finished before the requests for row t + 2 are issued
    asm volatile("" : "+v"(Tc[t]) : : "memory");
  }
  if (lane < CT) {
    const int pc = swz(lane);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      bf16_bits tt[NTF];
      float x = Tc[t];
      if constexpr (FOLD) x = (x * vec_out[3 * CT + t]) * bb;
      split_terms<NTF>(x, tt);
#pragma unroll
      for (int i = 0; i < NTF; ++i) Tout[i * tps + t * tld + pc] = tt[i];
    }
    if constexpr (FOLD) {
      // row `lane` of T^T: runs of four columns are contiguous in the swizzled order
#pragma unroll
      for (int t0 = 0; t0 < CT; t0 += 4) {
        bf16_bits tt[4][NTF];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_terms<NTF>(Tc[t0 + e], tt[e]);
#pragma unroll
        for (int i = 0; i < NTF; ++i)
          *reinterpret_cast<uint2*>(Ttr + i * tps + lane * tld + swz(t0)) =
              uint2{(uint32_t)tt[0][i] | ((uint32_t)tt[1][i] << 16), (uint32_t)tt[2][i] | ((uint32_t)tt[3][i] << 16)};
      }
    }
  }
}


// ---------------------------------------------------------------- xor-layout planes
// Inverse of swz.
__host__ __device__ constexpr int unswz(int p) {
  return (p & ~31) | (((((p >> 2) & 7) >> 1) | ((((p >> 2) & 7) & 1) << 2)) << 2) | (p & 3);
}

// XOR key of row r in a plane with RB-byte rows (RB in 32 .. 256): 16 consecutive rows
// get 16 distinct (row, piece) bank slots within 256 bytes.
template <int RB>
__device__ __forceinline__ int xkey(int r) {
  constexpr int NP = RB / 16;
  constexpr int SH = NP >= 16 ? 0 : NP == 8 ? 1 : NP == 4 ? 2 : 3;
  return (r >> SH) & (NP - 1);
}
// Element offset (bf16 units) of logical 16-byte piece lp of row r.
template <int RB>
__device__ __forceinline__ int xoff(int r, int lp) {
  return r * (RB / 2) + 8 * (lp ^ xkey<RB>(r));
}
// Operand read from an xor-layout plane: k-step s, lane group g.
template <int RB>
__device__ __forceinline__ bf16x8 xop_read(const bf16_bits* plane, int row, int s, int g) {
  return *reinterpret_cast<const bf16x8*>(plane + xoff<RB>(row, 4 * s + g));
}
template <int RB, int NT>
__device__ __forceinline__ void xop_terms(const bf16_bits* planes, int pstride, int row, int s, int g,
                                          bf16x8 (&out)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) out[i] = xop_read<RB>(planes + i * pstride, row, s, g);
}
// Element offset of the 4-element kappa run starting at kappa position pc (pc % 4 == 0).
template <int RB>
__device__ __forceinline__ int xrun(int r, int pc) {
  return xoff<RB>(r, pc >> 3) + (pc & 4);
}

// Store the 16 bytes of io elements at logical row t, columns j0.. into NT xor-layout
// bf16 planes (terms of each value).
template <typename IO, int NT, int RB>
__device__ __forceinline__ void xstore_row_terms(const uint4& v, bf16_bits* planes, int pstride, int t, int j0) {
  constexpr int VEC = 16 / sizeof(IO);
#pragma unroll
  for (int grp4 = 0; grp4 < VEC / 4; ++grp4) {
    bf16_bits* dst = planes + xrun<RB>(t, swz(j0 + 4 * grp4));
    if constexpr (NT == 1 && sizeof(IO) == 2) {
      *reinterpret_cast<uint2*>(dst) = uint2{(&v.x)[2 * grp4], (&v.x)[2 * grp4 + 1]};
    } else {
      bf16_bits tt[4][NT];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_terms<NT>(elem<IO>(v, 4 * grp4 + e), tt[e]);
#pragma unroll
      for (int i = 0; i < NT; ++i)
        *reinterpret_cast<uint2*>(dst + i * pstride) =
            uint2{(uint32_t)tt[0][i] | ((uint32_t)tt[1][i] << 16), (uint32_t)tt[2][i] | ((uint32_t)tt[3][i] << 16)};
    }
  }
}

// LDS DMA: each active lane copies 4 (or 16) bytes from its own global address to
// lds_base + lane * 4 (or 16); lds_base is uniform over the wave.
__device__ __forceinline__ void lds_dma4(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 4, 0, 0);
#endif
}
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
#endif
}

// A wave-uniform fp32 through the constant address space: a scalar load into an SGPR.
__device__ __forceinline__ float uniform_load(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

// Compiler-only fence between phases of a chunk: memory accesses are not moved across
// it, which bounds how many operands the scheduler keeps live in registers.
__device__ __forceinline__ void phase_fence() { asm volatile("" ::: "memory"); }


}  // namespace chunk
}  // namespace gdn
