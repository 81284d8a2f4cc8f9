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

// Column c of Tb = (I + Ab)^-1 for the 16 x 16 diagonal block Ab of a strictly lower
// triangular fp32 matrix (rows of stride CT + 4, the block's first row and column at
// 16 bi), by forward substitution X[r] = [r == c] - sum_{s<r} Ab[r][s] X[s] as four
// interleaved partial sums added in a fixed order.  The coefficients of row r are the
// same for every lane that works on block bi (LDS broadcast reads), requested one row
// ahead.
template <int CT>
__device__ __forceinline__ void diag_inverse_column(const float (*As)[CT + 4], int bi, int c, float (&X)[16]) {
  const float(*Ab)[CT + 4] = reinterpret_cast<const float(*)[CT + 4]>(&As[16 * bi][16 * bi]);
  f32x4 arow[2][4];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r + 1 < 16) {
#pragma unroll
      for (int i = 0; i < (r + 4) / 4; ++i) arow[(r + 1) & 1][i] = *reinterpret_cast<const f32x4*>(&Ab[r + 1][4 * i]);
    }
    asm volatile("" ::: "memory");
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int sv = 0; sv < r; ++sv) {
      const float av = arow[r & 1][sv >> 2][sv & 3];
      if ((sv & 3) == 0) p0 = fmaf(av, X[sv], p0);
      if ((sv & 3) == 1) p1 = fmaf(av, X[sv], p1);
      if ((sv & 3) == 2) p2 = fmaf(av, X[sv], p2);
      if ((sv & 3) == 3) p3 = fmaf(av, X[sv], p3);
    }
    X[r] = (r == c ? 1.f : 0.f) - ((p0 + p1) + (p2 + p3));
    // row r is finished before the requests for row r + 2 are issued
    asm volatile("" : "+v"(X[r]) : : "memory");
  }
}

// Tile (mt, nt) of A = strict lower part of diag(b) exp(g_t - g_s) K K^T (one wave):
// Ks holds NTI swizzled key-row planes, vec_lds the rows' g (first CT) and b (next CT).
template <int CT, int D, int NTI, int ORD>
__device__ __forceinline__ void form_a_tile(const bf16_bits* Ks, int kps, float (*As)[CT + 4], int n, int mt, int nt,
                                            const float* vec_lds) {
  constexpr int KP = row_stride(D);
  constexpr int KSD = (D + 31) / 32;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
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
    As[t][sc] = (sc < t && t < n) ? bt * dec * acc[r] : 0.f;
  }
}

// ----------------------------------------------------------------------------------
// Chunk factorization of the replay kernels (flush and outputs).  One wave.
//   Ks: NTI swizzled planes (row stride KP) of the chunk's key rows (rows >= n zero).
//   g, bb: this lane's g_t and b_t for t = lane (t >= n: g_t = g_{n-1}, b_t = 0).
// Writes T = (I + A)^-1 as NTF swizzled bf16 planes (row stride tld, plane stride
// tps) and the four per-row vectors g, exp(g), b, exp(g_n - g) into vec_out.
// T is formed by 16-row blocks (32- and 64-row chunks), see below.
// Barriers: the first publishes the row vectors to the whole workgroup.  The second
// orders this wave's A tiles before its own substitution reads them: with LOCAL_A it
// is a wait for this wave's LDS traffic only, so the other waves match one barrier and
// are not held while the A tiles are formed.  HELPED (32-row chunks, not with LOCAL_A):
// this wave forms only the first row tile of A; the caller's other waves form the second
// (tiles (1, 0) and (1, 1), form_a_tile) between the two barriers.
template <int CT, int D, int NTI, int NTF, int ORD, bool LOCAL_A = false, bool HELPED = false>
__device__ __forceinline__ void factorize_chunk(const bf16_bits* Ks, int kps, float (*As)[CT + 4], int n,
                                                float g, float bb, bf16_bits* Tout, int tps, int tld,
                                                float* vec_out, float* vec_lds) {
  constexpr int MT = CT / 16;
  static_assert(CT == 32 || CT == 64, "the blocked inverse covers 32- and 64-row chunks");
  static_assert(!(HELPED && LOCAL_A), "helper waves need the full second barrier");
  static_assert(!HELPED || CT == 32, "helper waves form the second row tile of a 32-row chunk");
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;

  const float gn = lane_value(g, n - 1);
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
    // row tiles at or past n are zero; their diagonal tiles are stored as zeros
    // (the substitution reads them) and the others are not read
    if (16 * mt >= n) {
#pragma unroll
      for (int m2 = mt; m2 < MT; ++m2)
#pragma unroll
        for (int r = 0; r < 4; ++r) As[16 * m2 + 4 * grp + r][16 * m2 + col] = 0.f;
      break;
    }
    // HELPED: row tiles past the first are formed by other waves (form_a_tile) between
    // this function's two barriers
    if (HELPED && mt >= 1) break;
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) form_a_tile<CT, D, NTI, ORD>(Ks, kps, As, n, mt, nt, vec_lds);
  }
  if constexpr (LOCAL_A)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  else
    lds_barrier();

  if constexpr (CT == 64) {
    // Block forward substitution over four 16-row blocks: block row i of T's column tile
    // W is Tii (E - U), U = A[block i, 0 : 16 i] T[0 : 16 i, tile W], Tii = (I + Aii)^-1
    // (E: the identity's block, zero off the diagonal).  Lane group grp inverts diagonal
    // block grp; the off-diagonal blocks follow on the matrix cores, column tile by
    // column tile, each block row's C layout serving as the B operand of the next ones.
    float X[16];
    diag_inverse_column<CT>(As, grp, col, X);
    {
      const int pc = swz(16 * grp + col);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bf16_bits tt[NTF];
        split_terms<NTF>(X[r], tt);
#pragma unroll
        for (int q = 0; q < NTF; ++q) Tout[q * tps + (16 * grp + r) * tld + pc] = tt[q];
      }
      // zeros above the diagonal: tiles (0,1) (0,2) (0,3) (1,2) (1,3) (2,3), as runs of
      // eight columns (192 runs, three per lane)
      const uint2 z{0u, 0u};
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int task = lane + 64 * k, ti = task >> 5, zr = (task & 31) >> 1, zc = 8 * (task & 1);
        const int tr = ti < 3 ? 0 : ti < 5 ? 1 : 2, tc = ti < 3 ? ti + 1 : ti < 5 ? ti - 1 : 3;
#pragma unroll
        for (int q = 0; q < NTF; ++q) {
          bf16_bits* p = Tout + q * tps + (16 * tr + zr) * tld;
          *reinterpret_cast<uint2*>(p + swz(16 * tc + zc)) = z;
          *reinterpret_cast<uint2*>(p + swz(16 * tc + zc + 4)) = z;
        }
      }
    }
    // the diagonal blocks, read back by other lanes of this wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
#pragma unroll
    for (int W = 0; W < 3; ++W) {
      f32x4 Tb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Tb[i] = zero4();
        if (i < W) continue;
        if (i > W && 16 * i >= n) {
          // rows at or past n: identity rows, zero off the diagonal
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < NTF; ++q) Tout[q * tps + (16 * i + 4 * grp + r) * tld + swz(16 * W + col)] = 0;
          continue;
        }
        f32x4 u = zero4();
        if (i > W) {
#pragma unroll
          for (int sp = 0; sp < (16 * i + 31) / 32; ++sp) {
            // A rows 16 i + col; contraction elements at or past 16 i are dropped
            const bool keep_hi = 32 * sp + 16 < 16 * i;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(&As[16 * i + col][32 * sp + 4 * grp]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(&As[16 * i + col][32 * sp + 16 + 4 * grp]);
            bf16x8 a[NTF], b[NTF];
            reg_operand<NTF>(lo, keep_hi ? hi : zero4(), a);
            reg_operand<NTF>(Tb[2 * sp], keep_hi ? Tb[2 * sp + 1] : zero4(), b);
            mma_terms<NTF, NTF, ORD>(u, a, b);
          }
        }
        f32x4 em;
#pragma unroll
        for (int r = 0; r < 4; ++r) em[r] = (16 * i + 4 * grp + r == 16 * W + col ? 1.f : 0.f) - u[r];
        bf16x8 tii[NTF], e_op[NTF];
#pragma unroll
        for (int q = 0; q < NTF; ++q) {
          const uint2 w = *reinterpret_cast<const uint2*>(Tout + q * tps + (16 * i + col) * tld + swz(16 * i + 4 * grp));
          tii[q] = __builtin_bit_cast(bf16x8, u32x4_t{w.x, w.y, 0u, 0u});
        }
        reg_operand<NTF>(em, zero4(), e_op);
        mma_terms<NTF, NTF, ORD>(Tb[i], tii, e_op);
        if (i > W) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16_bits tt[NTF];
            split_terms<NTF>(Tb[i][r], tt);
#pragma unroll
            for (int q = 0; q < NTF; ++q) Tout[q * tps + (16 * i + 4 * grp + r) * tld + swz(16 * W + col)] = tt[q];
          }
        }
      }
    }
    return;
  } else {
    // With A = [A00 0; A10 A11] in 16-row blocks, T = [T00 0; -T11 A10 T00 T11],
    // Tii = (I + Aii)^-1.
    // Diagonal blocks, both at once: lane (grp, c) owns column c of block bi = grp & 1
    // (groups 2 and 3 repeat 0 and 1).
    const int bi = grp & 1;
    float X[16];
    diag_inverse_column<CT>(As, bi, col, X);
    if (grp < 2) {
      const int pc = swz(16 * bi + col);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bf16_bits tt[NTF];
        split_terms<NTF>(X[r], tt);
#pragma unroll
        for (int q = 0; q < NTF; ++q) Tout[q * tps + (16 * bi + r) * tld + pc] = tt[q];
      }
    } else {
      // groups 2 and 3: zeros into the upper right block and, with n <= 16, the lower
      // left one (lane u: row u / 2, eight columns from 8 (u % 2), two runs of four)
      const int u = lane - 32, zr = u >> 1, zc = 8 * (u & 1);
      const uint2 z{0u, 0u};
#pragma unroll
      for (int q = 0; q < NTF; ++q) {
        bf16_bits* p = Tout + q * tps;
        *reinterpret_cast<uint2*>(p + zr * tld + swz(16 + zc)) = z;
        *reinterpret_cast<uint2*>(p + zr * tld + swz(16 + zc + 4)) = z;
        if (n <= 16) {
          *reinterpret_cast<uint2*>(p + (16 + zr) * tld + swz(zc)) = z;
          *reinterpret_cast<uint2*>(p + (16 + zr) * tld + swz(zc + 4)) = z;
        }
      }
    }
    if (n > 16) {
      // T00 and T11 as written above, read back by other lanes of this wave
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // U = A10 T00 in C layout (lane (col, grp): U[4 grp + r][col]); the contraction
      // runs over 16 elements, so elements 4..7 of both operands are zero
      bf16x8 a10[NTF], t00[NTF];
      reg_operand<NTF>(*reinterpret_cast<const f32x4*>(&As[16 + col][4 * grp]), zero4(), a10);
#pragma unroll
      for (int q = 0; q < NTF; ++q) {
        bf16_bits v8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) v8[r] = Tout[q * tps + (4 * grp + r) * tld + swz(col)];
#pragma unroll
        for (int r = 4; r < 8; ++r) v8[r] = 0;
        t00[q] = pack8(v8);
      }
      f32x4 u = zero4();
      mma_terms<NTF, NTF, ORD>(u, a10, t00);
      // T10 = T11 (-U): the C layout of U is the B operand; A = rows of T11
      bf16x8 t11[NTF], mu[NTF];
      typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
#pragma unroll
      for (int q = 0; q < NTF; ++q) {
        const uint2 w = *reinterpret_cast<const uint2*>(Tout + q * tps + (16 + col) * tld + swz(16 + 4 * grp));
        t11[q] = __builtin_bit_cast(bf16x8, u32x4_t{w.x, w.y, 0u, 0u});
      }
      f32x4 nu;
#pragma unroll
      for (int r = 0; r < 4; ++r) nu[r] = -u[r];
      reg_operand<NTF>(nu, zero4(), mu);
      f32x4 t10 = zero4();
      mma_terms<NTF, NTF, ORD>(t10, t11, mu);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16_bits tt[NTF];
        split_terms<NTF>(t10[r], tt);
#pragma unroll
        for (int q = 0; q < NTF; ++q) Tout[q * tps + (16 + 4 * grp + r) * tld + swz(col)] = tt[q];
      }
    }
    return;
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
