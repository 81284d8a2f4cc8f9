// prefill_kernels.hip -- chunked varlen prefill of the gated delta rule on gfx950.
//
// Two kernels (the chunk algebra is stated in chunk_common.h):
//   factorize_kernel: one wave per (chunk, value head), all of them at once.  Computes
//     everything about a chunk that does not depend on the state: the gate vectors,
//     T = (I + A)^-1 (the WY / UT transform), the causal decayed scores
//     P = scale * exp(g_t - g_s) q_t.k_s (s <= t) and the keys transposed.  It writes
//     T'' = diag(exp(g_n - g)) T diag(b), PT'' = P T diag(b) and K^T as ready-made MFMA
//     A-operand fragments (1 KiB each, 16 bytes per lane) into one record per (value
//     head, chunk).
//   scan_kernel: one workgroup per (sequence, value head, 16-row slab of the state),
//     walking the sequence's chunks in order with its slab in registers.  Rows of the
//     state evolve independently, so the slabs never exchange data; for head dim >= 64
//     the slab's key columns are split over two waves, which add their partial
//     contractions through LDS.
//
// Chunks are cut at every multiple of 64 tokens, of the cache block and at the call
// ends (plan.cpp); when a chunk ends on a block boundary the scan stores the bits of
// the state into that boundary's checkpoint page, the state the next chunk starts
// from ("Prefix caching on Gated DeltaNet hybrids", "Why hits were wrong": a full block
// keeps the recurrent state after its last token), so a resume from the page computes
// exactly what the cold run computes after that point.
//
// Scan memory access.  Every load and store of the chunk loop is a buffer instruction
// whose descriptor (SGPRs) holds the chunk's base address and its length in bytes; the
// per-lane offsets are fixed for the whole kernel.  Rows past the end of a ragged chunk
// fall outside the descriptor's range, so the hardware returns zeros for them and drops
// their stores: they are excluded by selection, never read, never written.  Each phase
// of a chunk requests the operands of the next phase before it computes.
#include <hip/hip_runtime.h>

#include "call_table.h"
#include "chunk_common.h"
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace gdn {

using namespace chunk;

namespace {

constexpr int CT = kChunk;

// The (row tile mt, k-step s) pairs of a 64 x 64 lower triangular matrix whose k-steps
// are not all zero: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
constexpr int kFragCombos = 6;
__host__ __device__ constexpr int frag_combo(int mt, int s) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + s; }

template <typename IO, int D>
struct PrefillCfg {
  static constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  static constexpr int DT = D / 16;
  // The staged scan (bf16 inputs, d >= 64) forms its K^T operands from the key rows it
  // stages anyway (transposing LDS reads); the register scan reads them from the record.
  static constexpr bool HAS_KT = !(sizeof(IO) == 2 && D >= 64);
  // factor record: [T'' fragments][PT'' fragments][K^T fragments (HAS_KT)][row vectors]
  // [chunk scalar], with T'' = diag(exp(g_n - g)) T diag(b) and PT'' = (scale P) T diag(b)
  static constexpr int T_OFF = 0;
  static constexpr int P_OFF = kFragCombos * NTF * 1024;
  static constexpr int KT_OFF = 2 * kFragCombos * NTF * 1024;
  static constexpr int VEC_OFF = KT_OFF + (HAS_KT ? DT * 2 * NTI * 1024 : 0);
  // row vector planes (kChunk floats each): exp(g), scale exp(g)
  static constexpr int V_EG = 0, V_EGS = 1, NVEC = 2;
  static constexpr int EGN_OFF = VEC_OFF + NVEC * CT * 4;  // exp(g_n)
  static constexpr int REC_BYTES = EGN_OFF + 16;
  static_assert(REC_BYTES <= (int)factor_record_bytes_c(NTF, NTI, D), "factor record layout");
};

// ---------------------------------------------------------------- buffer access
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor: base, length in bytes (accesses at or past it read 0 and
// write nothing), 32-bit data format (gfx9 word 3).  Both are wave-uniform; they are
// passed through readfirstlane so that a value the compiler happened to compute on
// the vector unit still lands in SGPRs (a descriptor in VGPRs costs a waterfall loop
// around every access).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(join_address(lo, hi));
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, soff, 0));
}
__device__ __forceinline__ f32x4 ld16f(rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(f32x4, ld16(r, off, soff));
}
__device__ __forceinline__ bf16x8 ld16h(rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(bf16x8, ld16(r, off, soff));
}
template <typename IO>
__device__ __forceinline__ float ld_elem(rsrc_t r, uint32_t off) {
  if constexpr (sizeof(IO) == 2)
    return bf16_to_f32((bf16_bits)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
  else
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st4(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}

// Key-column order of the scan's registers.  Register position (state tile jt, lane
// group g, element r) holds key column kcol(jt, g) + r.  For d >= 32 this makes the 8
// contraction elements a lane supplies at k-step s (tiles 2s and 2s+1, see the kappa
// order in device_common.h) the 8 adjacent columns 32 s + 8 g .. + 7 of a key or query
// row: one 16-byte load.  d = 16 keeps the natural order 4 g + r.
template <int D>
__host__ __device__ constexpr int kcol(int jt, int g) {
  return D >= 32 ? 32 * (jt >> 1) + 8 * g + 4 * (jt & 1) : 4 * g;
}

// One A-operand load of a row-major input matrix (K or Q rows) in the kcol order.
// off: byte offset of this lane's row and first column.  bf16 inputs are one exact
// term; fp32 inputs are kept raw and split at use.
template <typename IO>
struct RowOp;
template <>
struct RowOp<bf16_bits> {
  bf16x8 v;
};
template <>
struct RowOp<float> {
  f32x4 lo, hi;
};

template <typename IO, int D>
__device__ __forceinline__ RowOp<IO> load_row_op(rsrc_t r, uint32_t off, int s) {
  RowOp<IO> o;
  if constexpr (sizeof(IO) == 2) {
    if constexpr (D >= 32) {
      o.v = ld16h(r, off + 64 * s, 0);
    } else {
      const u32x2 lo = ld8(r, off);
      o.v = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], 0u, 0u});
    }
  } else {
    o.lo = ld16f(r, off + 128 * s, 0);
    o.hi = D >= 32 ? ld16f(r, off + 128 * s + 16, 0) : zero4();
  }
  return o;
}
template <int NT>
__device__ __forceinline__ void row_terms(const RowOp<bf16_bits>& o, bf16x8 (&t)[NT]) {
  static_assert(NT == 1, "bf16 rows are one term");
  t[0] = o.v;
}
template <int NT>
__device__ __forceinline__ void row_terms(const RowOp<float>& o, bf16x8 (&t)[NT]) {
  reg_operand<NT>(o.lo, o.hi, t);
}

}  // namespace

// ==================================================================================
// Pre-pass: one 4-wave workgroup per (chunk, value head).  Four workgroups fit a compute
// unit (34 KiB of LDS each at d = 128 with bf16 inputs), so every SIMD runs four of these
// waves.
//
//   P0 (all waves)  key rows into LDS; each wave loads the query rows of its own row tile
//                   straight into registers (they are only ever the B operand of P);
//                   wave 0 forms the gates g, exp(g), b, exp(g_n - g) and writes the
//                   record's row vectors.
//   P1 (per wave)   its share of A = strict-lower(b exp(g_t - g_s) K K^T) into LDS (five
//                   tiles of the ten lower 16 x 16 tiles per wave, counting P's below),
//                   the P fragments of its own row tile ut = W (kept in registers), and
//                   K^T fragments.
//   P2              T = (I + A)^-1 by 16-row blocks: one wave inverts the four 16 x 16
//                   diagonal blocks at once; then each wave forms block row i of its 16
//                   columns as T_ii (E_i - U_i), U_i = A[block i, 0 : 16 i] T[0 : 16 i, :],
//                   both products on MFMA with the earlier blocks kept in registers.
//                   Writes T^T rows, and the record's T'' fragments from registers.
//   P3 (per wave)   the PT'' fragments of row tile W.
//
// The blocked product runs on split bf16 terms like every other product (fp32 class for
// bf16 inputs: two terms, order <= 1; fp32 inputs: three terms, order <= 2).
template <typename IO, int D>
struct FactorLds {
  using Cfg = PrefillCfg<IO, D>;
  // T^T planes unpadded (rows of 64 elements, 128 bytes), in the xor layout (16-byte
  // pieces permuted by row) so that 16-row operand reads stay free of bank conflicts.
  // The query rows and T'' need no LDS: the queries are loaded as operands, and T''
  // leaves through registers.  34,816 bytes at d = 128 with bf16 inputs (113 VGPRs):
  // four workgroups per CU.
  static constexpr int KP = row_stride(D), TP = CT;
  static constexpr int KS = Cfg::NTI * CT * KP;  // bf16 elements of the key planes
  static constexpr int TT = Cfg::NTF * CT * TP;  // bf16 elements of the T^T planes
  static constexpr int KT = KS > TT ? KS : TT;   // key planes, later T^T
  // The T_ii planes (NTF terms x 16 bf16 per row of a diagonal block) fit in the
  // diagonal 16 x 16 fp32 blocks of A for NTF <= 2; A is not read there once they exist.
  static constexpr bool TD_IN_A = Cfg::NTF <= 2;
};

// Row vectors of the chunk (k = 0: g, 1: exp(g), 2: b, 3: exp(g_n - g)) live in the four
// padding columns of A's rows: element t of vector k is A[t][CT + k].
__device__ __forceinline__ float& rowvec(float (*As)[CT + 4], int k, int t) { return As[t][CT + k]; }

// Row r of the T_ii plane for term q of diagonal block bi (16 bf16).
template <bool IN_A>
__device__ __forceinline__ bf16_bits* td_row(float (*As)[CT + 4], float (*Ub)[24], int q, int bi, int r) {
  if constexpr (IN_A)
    return reinterpret_cast<bf16_bits*>(&As[16 * bi + r][16 * bi + 8 * q]);
  else
    return reinterpret_cast<bf16_bits*>(&Ub[0][0]) + ((q * 4 + bi) * 16 + r) * 16;
}

// The ten lower 16 x 16 tiles of A, dealt 4, 3, 2, 1 to waves 0..3 (P's tiles of row
// tile ut = W are 1, 2, 3, 4: five tiles per wave).
__host__ __device__ constexpr int a_tile_mt(int i) { return i < 1 ? 0 : i < 3 ? 1 : i < 6 ? 2 : 3; }
__host__ __device__ constexpr int a_tile_nt(int i) { return i - (i < 1 ? 0 : i < 3 ? 1 : i < 6 ? 3 : 6); }
__host__ __device__ constexpr int a_tiles_begin(int w) { return w == 0 ? 0 : w == 1 ? 4 : w == 2 ? 7 : w == 3 ? 9 : 10; }

// The query rows of one row tile as B operands of P, straight from memory: lane (col,
// grp) holds row col of the tile at the contraction elements kappa(s, grp, 0..7), i.e.
// the runs of four columns 32 s + 4 grp and 32 s + 16 + 4 grp (the order of the key
// planes).  Rows past the chunk read as zeros (the descriptor ends at the last row);
// columns past a short row (d = 16) are zero.
template <typename IO, int D>
struct QRows {
  static constexpr int KSD = (D + 31) / 32;
  using Run = std::conditional_t<sizeof(IO) == 2, u32x2, u32x4>;
  Run run[KSD][2];
};
template <typename IO, int D>
__device__ __forceinline__ QRows<IO, D> load_q_rows(rsrc_t rq, uint32_t row_off, int grp) {
  QRows<IO, D> o;
#pragma unroll
  for (int s = 0; s < QRows<IO, D>::KSD; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c0 = 32 * s + 16 * h + 4 * grp;
      if constexpr (sizeof(IO) == 2)
        o.run[s][h] = c0 < D ? ld8(rq, row_off + (uint32_t)c0 * 2u) : u32x2{0u, 0u};
      else
        o.run[s][h] = c0 < D ? ld16(rq, row_off + (uint32_t)c0 * 4u, 0) : u32x4{0u, 0u, 0u, 0u};
    }
  return o;
}
// Operand terms of k-step s (the same splits the key planes hold).
template <typename IO, int D, int NT>
__device__ __forceinline__ void q_terms(const QRows<IO, D>& q, int s, bf16x8 (&out)[NT]) {
  if constexpr (sizeof(IO) == 2) {
    static_assert(NT == 1, "bf16 rows are one term");
    out[0] = __builtin_bit_cast(bf16x8, u32x4{q.run[s][0][0], q.run[s][0][1], q.run[s][1][0], q.run[s][1][1]});
  } else {
    bf16_bits tt[8][NT];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_terms<NT>(__uint_as_float(q.run[s][e >> 2][e & 3]), tt[e]);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      bf16_bits v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = tt[e][i];
      out[i] = pack8(v8);
    }
  }
}

template <typename IO, int D, int W>
__device__ __forceinline__ void factorize_wave(const FactorizeArgs<IO>& p, const int n, uint8_t* rec,
                                               bf16_bits* Ks, const QRows<IO, D>& qrows, float (*As)[CT + 4],
                                               float (*Ub)[24], const int p2_wave) {
  using Cfg = PrefillCfg<IO, D>;
  using L = FactorLds<IO, D>;
  constexpr int NTI = Cfg::NTI, NTF = Cfg::NTF, ORD = Cfg::ORD;
  constexpr int KP = L::KP, TP = L::TP;
  constexpr int KSD = (D + 31) / 32, DT = D / 16;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  constexpr bool TDA = L::TD_IN_A;
  bf16_bits* Tt = Ks;  // T^T planes, once P1 has read the key rows

  // ---------------------------------------------------------------- P1
  // A tiles: acc = K_mt K_nt^T; element (t, s) with t = 16 mt + 4 grp + r, s = 16 nt + col
#pragma unroll
  for (int ti = a_tiles_begin(W); ti < a_tiles_begin(W + 1); ++ti) {
    const int mt = a_tile_mt(ti), nt = a_tile_nt(ti);
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 a[NTI], b[NTI];
      op_terms<NTI>(Ks, CT * KP, KP, 16 * mt + col, s, grp, a);
      op_terms<NTI>(Ks, CT * KP, KP, 16 * nt + col, s, grp, b);
      mma_terms<NTI, NTI, ORD>(acc, a, b);
    }
    const int sc = 16 * nt + col;
    const float gs = rowvec(As, 0, sc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * grp + r;
      // computed for every element (pinned, so the LDS reads are not moved into a
      // branch per element) and kept or dropped by the select
      float dec = __expf(rowvec(As, 0, t) - gs), bt = rowvec(As, 2, t);
      asm volatile("" : "+v"(dec), "+v"(bt));
      As[t][sc] = (sc < t && t < n) ? bt * dec * acc[r] : 0.f;
    }
  }

  // P fragments of row tile W: tile (ms, W) of P^T = K Q^T has the C layout "lane (col,
  // grp) holds P[16 W + col][16 ms + 4 grp + r]", i.e. elements 0..3 (ms = 2s) or 4..7
  // (ms = 2s + 1) of the A operand of P for (W, s).  They stay in registers: they are the
  // B operands of PT^T = T^T P^T in P3.
  constexpr int NPS = (W >> 1) + 1;
  bf16x8 Pfr[NPS][NTF];
#pragma unroll
  for (int s = 0; s < NPS; ++s) {
    const bool two = 2 * s + 1 <= W;  // tile 2s+1 lies above the diagonal otherwise
    f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      bf16x8 bq[NTI], a0[NTI], a1[NTI];
      q_terms<IO, D, NTI>(qrows, ks, bq);
      op_terms<NTI>(Ks, CT * KP, KP, 32 * s + col, ks, grp, a0);
      mma_terms<NTI, NTI, ORD>(acc0, a0, bq);
      if (two) {
        op_terms<NTI>(Ks, CT * KP, KP, 32 * s + 16 + col, ks, grp, a1);
        mma_terms<NTI, NTI, ORD>(acc1, a1, bq);
      }
    }
    const int t = 16 * W + col;
    const float gt = rowvec(As, 0, t);
    f32x4 vals[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sp = 32 * s + 16 * (e >> 2) + 4 * grp + (e & 3);
      const float dot = e < 4 ? acc0[e] : acc1[e - 4];
      // the exponent g_t - g_s is <= 0 on the causal side kept by the select
      float dec = __expf(gt - rowvec(As, 0, sp));
      asm volatile("" : "+v"(dec));
      vals[e >> 2][e & 3] = (sp <= t && t < n && (e < 4 || two)) ? p.scale * dec * dot : 0.f;
    }
    reg_operand<NTF>(vals[0], vals[1], Pfr[s]);  // terms split two elements at a time
  }

  // K^T fragments of state tiles jt = W, W + 4, ... (register scan only): row col of
  // tile jt is the key column the scan keeps at register position (jt, col / 4, col % 4)
  // (kcol order); contraction over the chunk rows t = kappa(s, grp, e)
#pragma unroll
  for (int jt = W; jt < (Cfg::HAS_KT ? DT : 0); jt += 4) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < NTI; ++i) {
        bf16_bits v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * s + 16 * (e >> 2) + 4 * grp + (e & 3);
          v8[e] = Ks[i * CT * KP + t * KP + swz(kcol<D>(jt, col >> 2) + (col & 3))];
        }
        *reinterpret_cast<bf16x8*>(rec + Cfg::KT_OFF + ((jt * 2 + s) * NTI + i) * 1024 + lane * 16) = pack8(v8);
      }
    }
  }
  __syncthreads();  // A complete; the query rows are read

  // ---------------------------------------------------------------- P2
  // T = (I + A)^-1 by blocks of 16 rows.  With A_ii the diagonal blocks and
  // U_i = A[block i, 0 : 16 i] T[0 : 16 i, :], block row i of T is T_ii (E_i - U_i),
  // T_ii = (I + A_ii)^-1.
  //
  // P2a (one wave; which one rotates with the workgroup): the four T_ii at once, lane
  // 16 bi + c owning column c of T_bi,bi (forward substitution over 16 rows, the shared
  // diag_inverse_column).  Written as bf16 terms, row-major, to Td.
  if (W == p2_wave) {
    const int bi = lane >> 4, c = lane & 15;
    float X[16];
    diag_inverse_column<CT>(As, bi, c, X);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bf16_bits tt[NTF];
      split_terms<NTF>(X[r], tt);
#pragma unroll
      for (int q = 0; q < NTF; ++q) td_row<TDA>(As, Ub, q, bi, r)[c] = tt[q];
    }
  }
  __syncthreads();  // T_ii complete

  // P2b (every wave, column tile W): block rows of T in MFMA C layout, lane (col, grp)
  // holding T[16 i + 4 grp + r][16 W + col].  A C-layout tile is directly elements 0..3
  // of the B operand over its 16 rows, so the earlier blocks feed U_i and E_i - U_i
  // feeds the product by T_ii without leaving registers.
  {
    // unit B operand of the transposing products below: element e of lane (col, grp) is
    // one where 4 grp + e == col (e < 4)
    bf16_bits u8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u8[e] = (e < 4 && 4 * grp + e == col) ? (bf16_bits)0x3F80 : (bf16_bits)0;
    const bf16x8 unit = pack8(u8);
    f32x4 Tb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 u = zero4();
#pragma unroll
      for (int sp = 0; sp < (16 * i + 31) / 32; ++sp) {
        // A rows 16 i + col (fp32, split into terms); contraction elements at or past
        // 16 i are the block's own triangle or above it and are dropped
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&As[16 * i + col][32 * sp + 4 * grp]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&As[16 * i + col][32 * sp + 16 + 4 * grp]);
        const bool keep_hi = 32 * sp + 16 < 16 * i;
        bf16x8 a[NTF], b[NTF];
        reg_operand<NTF>(lo, keep_hi ? hi : zero4(), a);
        reg_operand<NTF>(Tb[2 * sp], keep_hi ? Tb[2 * sp + 1] : zero4(), b);
        mma_terms<NTF, NTF, ORD>(u, a, b);
      }
      f32x4 em;
#pragma unroll
      for (int r = 0; r < 4; ++r) em[r] = (16 * i + 4 * grp + r == 16 * W + col ? 1.f : 0.f) - u[r];
      bf16x8 tii[NTF], e_op[NTF];
#pragma unroll
      for (int q = 0; q < NTF; ++q) {
        // A operand of T_ii: row col, columns 4 grp .. + 3 (contraction past 16 is zero)
        const uint2 w = *reinterpret_cast<const uint2*>(td_row<TDA>(As, Ub, q, i, col) + 4 * grp);
        tii[q] = __builtin_bit_cast(bf16x8, u32x4{w.x, w.y, 0u, 0u});
      }
      reg_operand<NTF>(em, zero4(), e_op);
      Tb[i] = zero4();
      mma_terms<NTF, NTF, ORD>(Tb[i], tii, e_op);
      // row 16 W + col of T^T (columns 16 i + 4 grp .. + 3, contiguous in the swizzled
      // order)
      const float bj = rowvec(As, 2, 16 * W + col);
      {
        bf16x8 tq[NTF];
        reg_operand<NTF>(Tb[i], zero4(), tq);
#pragma unroll
        for (int q = 0; q < NTF; ++q) {
          const u32x4 w4 = __builtin_bit_cast(u32x4, tq[q]);
          *reinterpret_cast<uint2*>(Tt + q * CT * TP + xrun<2 * TP>(16 * W + col, swz(16 * i + 4 * grp))) =
              uint2{w4[0], w4[1]};
        }
      }
      // T''[t][j] = exp(g_n - g_t) T[t][j] b_j: this block's 16 x 16 values, transposed,
      // are half of the record's T'' fragment (i, W / 2) (lane (col, grp): row 16 i + col,
      // kappa elements 4 (W % 2) .. + 3).  A product with the unit operand moves each term
      // exactly from this C layout to the transposed one, and the lane stores it from
      // there.  Blocks i < 2 (W / 2) lie above the diagonal of every fragment.
      if (i >= 2 * (W >> 1)) {
        f32x4 tv;
#pragma unroll
        for (int r = 0; r < 4; ++r) tv[r] = (Tb[i][r] * rowvec(As, 3, 16 * i + 4 * grp + r)) * bj;
        bf16x8 t2[NTF];
        reg_operand<NTF>(tv, zero4(), t2);  // elements 4 .. 7 zero
#pragma unroll
        for (int q = 0; q < NTF; ++q) {
          const f32x4 tr = mfma(t2[q], unit, zero4());
          *reinterpret_cast<uint2*>(rec + Cfg::T_OFF + (frag_combo(i, W >> 1) * NTF + q) * 1024 + lane * 16 +
                                    8 * (W & 1)) = uint2{pack_bf16x2(tr[0], tr[1]), pack_bf16x2(tr[2], tr[3])};
        }
      }
    }
  }
  __syncthreads();  // T^T complete

  // ---------------------------------------------------------------- P3
  // PT'' = (scale P) T diag(b) for row tile ut = W, through its transpose: tile (jt, W)
  // of PT^T = T^T P^T, A = T^T rows (planes Tt), B = P^T, whose B operand at k-step s' is
  // the A operand of P for (W, s').  Its C layout "lane (col, grp) holds
  // PT[16 W + col][16 jt + 4 grp + r]" is elements 0..3 (jt = 2s) or 4..7 (jt = 2s + 1)
  // of the A operand of PT'' for (W, s).  T^T[j][t'] is zero for t' < j and P[u][t'] for
  // t' > u, so s' runs over jt/2 .. W/2.
#pragma unroll
  for (int s = 0; s < NPS; ++s) {
    f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int jt = 2 * s + h2;
      if (jt > W) continue;  // above the diagonal: zero
#pragma unroll
      for (int sp = jt >> 1; sp < NPS; ++sp) {
        bf16x8 a[NTF];
        xop_terms<2 * TP, NTF>(Tt, CT * TP, 16 * jt + col, sp, grp, a);
        mma_terms<NTF, NTF, ORD>(acc[h2], a, Pfr[sp]);
      }
    }
    f32x4 vals[2];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vals[e >> 2][e & 3] = acc[e >> 2][e & 3] * rowvec(As, 2, 32 * s + 16 * (e >> 2) + 4 * grp + (e & 3));
    bf16x8 fr[NTF];
    reg_operand<NTF>(vals[0], vals[1], fr);
#pragma unroll
    for (int q = 0; q < NTF; ++q)
      *reinterpret_cast<bf16x8*>(rec + Cfg::P_OFF + (frag_combo(W, s) * NTF + q) * 1024 + lane * 16) = fr[q];
  }
}

template <typename IO, int D>
__global__ __launch_bounds__(256) void factorize_kernel(FactorizeArgs<IO> p) {
  using Cfg = PrefillCfg<IO, D>;
  using L = FactorLds<IO, D>;
  constexpr int NTI = Cfg::NTI;
  constexpr int KP = L::KP;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;
  constexpr int PIECES = CT * PER_ROW, PER_THR = (PIECES + 255) / 256;
  // 34,816 bytes at d = 128 with bf16 inputs: four workgroups per CU
  __shared__ __attribute__((aligned(16))) bf16_bits Ks[L::KT];  // key rows, later T^T
  // A; its diagonal blocks later hold the T_ii planes, its padding columns the row vectors
  __shared__ __attribute__((aligned(16))) float As[CT][CT + 4];
  __shared__ __attribute__((aligned(16))) float Ub[L::TD_IN_A ? 1 : CT][24];  // T_ii planes otherwise

  const int h = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this chunk's rows, from its sequence's table entry
  const_table* tab = kernarg_table();
  const SeqEntry se = seq_entry(tab, unit_sequence(tab, c));
  const uint32_t start = chunk_start((uint32_t)se.p0, (uint32_t)(c - se.unit0), (uint32_t)tab->block, tab->lcm);
  const ChunkPos cd = chunk_at(se, start, (uint32_t)tab->block);
  const int n = cd.len;
  const int hk = h / p.group;
  uint8_t* rec = p.factors + ((size_t)c * p.Hv + h) * p.factor_stride;

  // For d < 32 the kappa groups past a 16-wide key row are contracted: keep them zero.
  if constexpr (D < 32) {
    zero_lds(Ks, sizeof(Ks), tid, 256);
    __syncthreads();
  }

  // ---------------------------------------------------------------- P0
  // every row load first: buffer loads whose descriptor ends at the chunk's last row, so
  // rows past n read as zeros without a branch
  const uint32_t qsb = (uint32_t)p.qk_stride * sizeof(IO);
  const rsrc_t rk = make_rsrc(p.k + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)n * qsb);
  const rsrc_t rq = make_rsrc(p.q + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)n * qsb);
  u32x4 kv[PER_THR];
#pragma unroll
  for (int i = 0; i < PER_THR; ++i) {
    const int idx = tid + 256 * i;
    const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    // pieces past the tile (small d) read past the descriptor's end: zeros, not stored
    const uint32_t off = idx < PIECES ? t * qsb + j0 * sizeof(IO) : 0xFFFFFFF0u & (n * qsb + 16u);
    kv[i] = ld16(rk, off, 0);
  }
  const QRows<IO, D> qrows = load_q_rows<IO, D>(rq, (uint32_t)(16 * wave + (lane & 15)) * qsb, lane >> 4);
  float av = 1.f, bb = 0.f;
  if (wave == 0) {
    const rsrc_t ra = make_rsrc(p.a + cd.row * p.Hv + h, (uint32_t)n * p.Hv * 4);
    const rsrc_t rb = make_rsrc(p.b + cd.row * p.Hv + h, (uint32_t)n * p.Hv * 4);
    av = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, lane * p.Hv * 4, 0, 0));
    bb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, lane * p.Hv * 4, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < PER_THR; ++i) {
    const int idx = tid + 256 * i;
    if (idx < PIECES) {
      const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
      const uint4 k4{kv[i][0], kv[i][1], kv[i][2], kv[i][3]};
      store_row_terms<IO, NTI>(k4, Ks, CT * KP, KP, t, j0);
    }
  }
  if (wave == 0) {
    const float la = lane < n ? __logf(av) : 0.f;  // rows past n: b = 0, log-decay 0
    const float g = wave_inclusive_scan(la);        // rows past n keep g_{n-1}
    const float gn = lane_value(g, n - 1);
    const float eg = __expf(g);
    rowvec(As, 0, lane) = g;
    rowvec(As, 1, lane) = eg;
    rowvec(As, 2, lane) = bb;
    rowvec(As, 3, lane) = lane < n ? __expf(gn - g) : 0.f;
    float* vo = reinterpret_cast<float*>(rec + Cfg::VEC_OFF);
    vo[Cfg::V_EG * CT + lane] = eg;
    vo[Cfg::V_EGS * CT + lane] = p.scale * eg;
    if (lane == 0) *reinterpret_cast<float*>(rec + Cfg::EGN_OFF) = __expf(gn);
  }
  __syncthreads();

  const int p2_wave = (blockIdx.x + blockIdx.y) & 3;
  switch (wave) {
    case 0: factorize_wave<IO, D, 0>(p, n, rec, Ks, qrows, As, Ub, p2_wave); break;
    case 1: factorize_wave<IO, D, 1>(p, n, rec, Ks, qrows, As, Ub, p2_wave); break;
    case 2: factorize_wave<IO, D, 2>(p, n, rec, Ks, qrows, As, Ub, p2_wave); break;
    default: factorize_wave<IO, D, 3>(p, n, rec, Ks, qrows, As, Ub, p2_wave); break;
  }
}

// ==================================================================================
// Scan: one workgroup per (sequence, value head, slab of 16 value rows), NSP waves.
//
// With NSP = 2 (head dim >= 64) the key columns of the slab are split between the two
// waves: each keeps its half of the state, forms its half of the contractions
// X = K S^T and Y = Q S^T over the key index, and the two halves are added through
// LDS (one barrier per chunk; fp addition is commutative, so both waves hold the same
// bits).  Both waves then form R' and Dt = T'' R'; each updates its half of the state
// and writes half of the output rows.
//
// Register layouts (lane = 16 grp + col):
//   state    S[j][r]  = S[16 slab + col][kcol(jt, grp) + r], jt = DTH w + j  (C layout of
//            S^T tiles)
//   X = K S^T, Y = Q S^T, R', Dt, O: [mt][r] = M[16 mt + 4 grp + r][16 slab + col]
// Per chunk, with R = diag(b) R' and the gates folded into the pre-pass factors
// (T'' = diag(exp(g_n - g)) T diag(b), PT'' = (scale P) T diag(b)):
//   A: X, Y            (K, Q rows and the state split into bf16 terms)
//   B: R' = V - exp(g) X;  Dt = T'' R'   (= diag(exp(g_n - g)) Delta)
//   C: O = scale exp(g) Y + PT'' R'      (= scale P Delta; stored)
//   D: S^T <- exp(g_n) S^T + K^T Dt;  checkpoint
template <int D>
struct ScanSplit {
  static constexpr int NSP = D >= 64 ? 2 : 1;
};

template <typename IO, int D>
__global__ __launch_bounds__(64 * ScanSplit<D>::NSP) void scan_kernel(ScanArgs<IO> p) {
  using Cfg = PrefillCfg<IO, D>;
  constexpr int NTI = Cfg::NTI, NTF = Cfg::NTF, ORD = Cfg::ORD;
  constexpr int DT = D / 16, KSD = (D + 31) / 32, NS = D / 16;
  constexpr int NSP = ScanSplit<D>::NSP;
  constexpr int KSH = KSD / NSP, DTH = DT / NSP;  // k-steps and state tiles per wave
  constexpr int MR = 4 / NSP;                     // output row tiles per wave
  constexpr int ESZ = sizeof(IO);
  static_assert(KSH * NSP == KSD && DTH * NSP == DT, "key split");

  // partial sums exchanged between the two waves: [chunk parity][wave][X 0..3, Y 4..7][lane]
  __shared__ f32x4 xch[NSP == 2 ? 2 * 2 * 8 * 64 : 1];

  // All slabs of one (sequence, head) go to the same XCD (workgroups are dealt to the
  // eight XCDs round robin), so their shared chunk operands meet in one L2.
  const int bid = blockIdx.x;
  const int u = (bid / (8 * NS)) * 8 + (bid & 7);
  const int sl = (bid >> 3) % NS;
  const_table* tab = kernarg_table();
  if (u >= tab->n_seqs * p.Hv) return;
  const int seq = u / p.Hv, h = u - seq * p.Hv;
  const int hk = h / p.group;
  const int w = NSP == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int my_row = 16 * sl + col;
  const SeqEntry se = seq_entry(tab, seq);
  const float* sq_src = static_cast<const float*>(se.src);
  float* sq_dst = static_cast<float*>(se.dst);
  const int cb = se.unit0, ce = se.unit0 + se.n_units;
  const uint32_t blk = (uint32_t)tab->block;
  const size_t head_off = (size_t)h * D * D;
  const int jt0 = DTH * w, s0 = KSH * w;  // first state tile and k-step of this wave
  const int mt0 = MR * w;                 // first output row tile of this wave

  f32x4 S[DTH];
#pragma unroll
  for (int j = 0; j < DTH; ++j) {
    if (sq_src)
      S[j] = *reinterpret_cast<const f32x4*>(sq_src + head_off + (size_t)my_row * D + kcol<D>(jt0 + j, grp));
    else
      S[j] = zero4();
  }
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int j = 0; j < DTH; ++j) *reinterpret_cast<f32x4*>(dst + kcol<D>(jt0 + j, grp)) = S[j];
  };
  if (cb >= ce) {
    store_state(sq_dst + head_off + (size_t)my_row * D);
    return;
  }

  // ---- per-lane byte offsets, fixed for the kernel
  const uint32_t qsb = (uint32_t)p.qk_stride * ESZ, vsb = (uint32_t)p.v_stride * ESZ;
  const uint32_t osb = (uint32_t)p.Hv * D * 4;
  uint32_t kq_off[4], v_off[4], o_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kq_off[i] = (16 * i + col) * qsb + kcol<D>(0, grp) * ESZ;
    v_off[i] = (4 * grp + i) * vsb + col * ESZ;
    o_off[i] = (4 * grp + i) * osb + col * 4;
  }
  const uint32_t frag_lane = 16 * lane;
  const uint32_t vec_lane = 16 * grp;  // + 64 mt: rows 16 mt + 4 grp .. + 3 of a vector plane

  auto rec_rsrc = [&](int c) {
    return make_rsrc(p.factors + ((size_t)c * p.Hv + h) * p.factor_stride, (uint32_t)Cfg::REC_BYTES);
  };

  // ---- operands of one chunk
  RowOp<IO> Kop[4][KSH], Qop[4][KSH];
  float Vv[4][4];
  f32x4 veg[4], vegs[MR];
  bf16x8 Tf[kFragCombos][NTF], Pf[MR][2][NTF], KTf[DTH][2][NTI];
  float egn;

  auto load_A = [&](const ChunkPos& cd) {
    const rsrc_t rk = make_rsrc(p.k + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)cd.len * qsb);
    const rsrc_t rq = make_rsrc(p.q + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)cd.len * qsb);
#pragma unroll
    for (int s = 0; s < KSH; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Kop[mt][s] = load_row_op<IO, D>(rk, kq_off[mt], s0 + s);
        Qop[mt][s] = load_row_op<IO, D>(rq, kq_off[mt], s0 + s);
      }
  };
  auto load_B = [&](const ChunkPos& cd, int c) {
    // one descriptor for the chunk's rows: the tile row goes into the offset, so the
    // descriptor's length bounds every row
    const rsrc_t rv = make_rsrc(p.v + cd.row * p.v_stride + (int64_t)h * D + 16 * sl, (uint32_t)cd.len * vsb);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Vv[mt][r] = ld_elem<IO>(rv, v_off[r] + 16 * mt * vsb);
    const rsrc_t rr = rec_rsrc(c);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) veg[mt] = ld16f(rr, vec_lane + 64 * mt, Cfg::VEC_OFF + Cfg::V_EG * CT * 4);
#pragma unroll
    for (int f = 0; f < kFragCombos; ++f)
#pragma unroll
      for (int i = 0; i < NTF; ++i) Tf[f][i] = ld16h(rr, frag_lane, Cfg::T_OFF + (f * NTF + i) * 1024);
  };
  auto load_C = [&](int c) {
    const rsrc_t rr = rec_rsrc(c);
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int mt = mt0 + i;
      vegs[i] = ld16f(rr, vec_lane, Cfg::VEC_OFF + Cfg::V_EGS * CT * 4 + 64 * mt);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s <= (mt >> 1))
#pragma unroll
          for (int t = 0; t < NTF; ++t)
            Pf[i][s][t] = ld16h(rr, frag_lane, Cfg::P_OFF + (frag_combo(mt, s) * NTF + t) * 1024);
    }
  };
  auto load_D = [&](int c) {
    const rsrc_t rr = rec_rsrc(c);
#pragma unroll
    for (int j = 0; j < DTH; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < NTI; ++i)
          KTf[j][s][i] = ld16h(rr, frag_lane, Cfg::KT_OFF + (((jt0 + j) * 2 + s) * NTI + i) * 1024);
    egn = uniform_load(reinterpret_cast<const float*>(p.factors + ((size_t)c * p.Hv + h) * p.factor_stride +
                                                      Cfg::EGN_OFF));
  };

  // The loads of a phase are issued where they are written: the scheduler may not sink
  // them below the computation that follows (which would cost the lookahead).
  auto issue_point = [] { __builtin_amdgcn_sched_barrier(0); };

  // One phase of lookahead: each phase first requests the operands of the next one
  // (the last phase those of the next chunk's first), then computes.  About 20-40
  // vector loads are in flight at a time, within the 63 the wave's counter tracks.
  uint32_t pos = (uint32_t)se.p0;
  ChunkPos cur = chunk_at(se, pos, blk);
  load_A(cur);

#pragma unroll 1
  for (int c = cb; c < ce; ++c) {
    // the next chunk (the last one loads itself again: in bounds, and unused)
    const uint32_t npos = c + 1 < ce ? pos + (uint32_t)cur.len : pos;
    const ChunkPos nxt = chunk_at(se, npos, blk);

    // ---- A: X = K S^T and Y = Q S^T (this wave's k-steps), eight accumulator chains
    load_B(cur, c);
    issue_point();
    f32x4 X[4], Y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) X[mt] = Y[mt] = zero4();
#pragma unroll
    for (int s = 0; s < KSH; ++s) {
      bf16x8 sop[NTF];
      reg_operand<NTF>(S[2 * s], (2 * s + 1 < DTH) ? S[2 * s + 1] : zero4(), sop);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        bf16x8 ak[NTI], aq[NTI];
        row_terms<NTI>(Kop[mt][s], ak);
        row_terms<NTI>(Qop[mt][s], aq);
        mma_terms<NTI, NTF, ORD>(X[mt], ak, sop);
        mma_terms<NTI, NTF, ORD>(Y[mt], aq, sop);
      }
    }
    // this wave's output rows of Y
    f32x4 Ym[MR];
    if constexpr (NSP == 1) {
#pragma unroll
      for (int i = 0; i < MR; ++i) Ym[i] = Y[i];
    } else {
      f32x4* mine = xch + (((c & 1) * 2 + w) * 8) * 64 + lane;
      f32x4* other = xch + (((c & 1) * 2 + (w ^ 1)) * 8) * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mine[mt * 64] = X[mt];
        mine[(4 + mt) * 64] = Y[mt];
      }
      lds_barrier();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 xo = other[mt * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r) X[mt][r] += xo[r];
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const f32x4 ya = mine[(4 + mt0 + i) * 64], yb = other[(4 + mt0 + i) * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ym[i][r] = ya[r] + yb[r];
      }
    }

    // ---- B: R' = V - exp(g) X (rows past the chunk end read as zeros, and the zero b
    //      there zeroes their columns of T''), Dt = T'' R' over the nonzero k-steps
    load_C(c);
    issue_point();
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) R[mt][r] = fmaf(-veg[mt][r], X[mt][r], Vv[mt][r]);
    bf16x8 Rop[2][NTF];
    reg_operand<NTF>(R[0], R[1], Rop[0]);
    reg_operand<NTF>(R[2], R[3], Rop[1]);
    f32x4 Dt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Dt[mt] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 2 * s; mt < 4; ++mt) mma_terms<NTF, NTF, ORD>(Dt[mt], Tf[frag_combo(mt, s)], Rop[s]);

    // ---- C: O = scale exp(g) Y + PT'' R' for this wave's row tiles
    load_D(c);
    issue_point();
    {
      const rsrc_t ro = make_rsrc(p.o + cur.row * (int64_t)p.Hv * D + (int64_t)h * D + 16 * sl, (uint32_t)cur.len * osb);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const int mt = mt0 + i;
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Ym[i][r] * vegs[i][r];
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (s <= (mt >> 1)) mma_terms<NTF, NTF, ORD>(acc, Pf[i][s], Rop[s]);
#pragma unroll
        for (int r = 0; r < 4; ++r) st4(ro, o_off[r] + 16 * mt * osb, acc[r]);
      }
    }

    // ---- D: S^T <- exp(g_n) S^T + K^T Dt for this wave's tiles
    load_A(nxt);
    issue_point();
    {
      bf16x8 Dtop[2][NTF];
      reg_operand<NTF>(Dt[0], Dt[1], Dtop[0]);
      reg_operand<NTF>(Dt[2], Dt[3], Dtop[1]);
#pragma unroll
      for (int j = 0; j < DTH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[j][r] *= egn;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < DTH; ++j) mma_terms<NTI, NTF, ORD>(S[j], KTf[j][s], Dtop[s]);
    }

    // ---- checkpoint: the state after this chunk, bit for bit
    if (cur.page_index >= 0) {
      const int32_t pid = *((const const_i32*)page_list(tab) + cur.page_index);
      if (pid >= 0)
        store_state(reinterpret_cast<float*>(p.ckpt_pool + (size_t)pid * p.page_bytes) + head_off +
                    (size_t)my_row * D);
    }
    cur = nxt;
    pos = npos;
  }
  store_state(sq_dst + head_off + (size_t)my_row * D);
}

// ==================================================================================
// Scan, staged form (bf16 inputs, head dim >= 64): one workgroup per (sequence, value
// head, pair of 16-row slabs), four waves (two slabs x two key halves).  The chunk
// operands that all slabs of a head share -- the factor record (T, P, K^T, the row
// vectors, exp(g_n)) -- and the value columns of the pair are copied into LDS once
// per workgroup by LDS DMA (buffer loads that write LDS directly), a chunk ahead, into
// two alternating buffers, and so are the chunk's key and query rows; each wave reads
// its operands from there one phase before it needs them.  Compared with one
// workgroup per slab, a compute unit moves about half the bytes per chunk and issues a
// quarter of the vector memory instructions.
//
// Per chunk c, with buffers Bc (chunk c) and Bn (chunk c + 1):
//   wait for this wave's copies into Bc; barrier (all copies landed, every wave is
//   done with chunk c - 1, so every buffer of chunk c + 1 and the exchange slots are
//   free); then phases A-D of scan_kernel with LDS operands, with the copies of chunk
//   c + 1 issued in three parts: the key rows at the top, the query rows after phase
//   A, the record and value rows after the exchange.  The copies share the compute
//   unit's path from L2 (about 60 bytes per cycle) and the LDS with the waves' own
//   reads; issued in one part (at the top, or all after the exchange) they cost
//   15-20% more time, and issued late in the chunk they held every wave at the next
//   barrier.
template <typename IO, int D>
struct ScanStaged {
  static constexpr bool OK = sizeof(IO) == 2 && D >= 64;
  static constexpr int NS = D / 16, NSP = 2, SP = 2, NW = SP * NSP, NG = NS / SP;
};

// LDS addresses of the staged scan are kept in the LDS address space: a generic pointer
// converted back costs a null check per copy.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
template <typename T>
__device__ __forceinline__ T lds_load(const lds_u8* p) {
  return *(const __attribute__((address_space(3))) T*)p;
}

__device__ __forceinline__ void dma16(rsrc_t r, lds_u8* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
}

// The work of wave Q of a staged-scan workgroup (slab Q / 2 of the pair, key half
// Q % 2), compiled once per wave index so that every register index and every copy
// assignment is a constant.
// Output row tiles of the key half w of a slab (two waves per slab): rows {0, 3} and
// {1, 2}, so that both hold the same number of score products (PT'' R' has one k-step
// for row tiles 0 and 1, two for 2 and 3).
// (With one wave per slab, the wave holds all four in order.)
template <int NSP>
__host__ __device__ constexpr int omt(int w, int i) { return NSP == 1 ? i : i == 0 ? w : 3 - w; }

template <typename IO, int D, int Q>
__device__ __forceinline__ void scan_staged_wave(const ScanArgs<IO>& p, const int u, const int sg, lds_u8* stage0,
                                                 lds_u8* stage1, lds_u8* kbuf0, lds_u8* kbuf1, lds_u8* qbuf0,
                                                 lds_u8* qbuf1, f32x4* xch) {
  using Cfg = PrefillCfg<IO, D>;
  using Shp = ScanStaged<IO, D>;
  constexpr int NTI = Cfg::NTI, NTF = Cfg::NTF, ORD = Cfg::ORD;
  constexpr int DT = D / 16, KSD = D / 32;
  constexpr int NSP = Shp::NSP, SP = Shp::SP, NW = Shp::NW;
  constexpr int KSH = KSD / NSP, DTH = DT / NSP, MR = 4 / NSP;
  constexpr int ESZ = sizeof(IO);
  // staged chunk: the factor record (its last 1 KiB granule partial), then 64 value
  // rows of the workgroup's 16 SP columns; 16-byte pieces of a value row are permuted by
  // an XOR with (row / 4) % VNP, so that the four row groups of one read hit distinct
  // banks
  constexpr int RG = (Cfg::REC_BYTES + 1023) / 1024;
  constexpr int VRB = SP * 16 * ESZ, VNP = VRB / 16, VG = 64 * VRB / 1024;
  constexpr int V_OFF = RG * 1024, G = RG + VG;
  constexpr int GPW = (G + NW - 1) / NW;  // copies per wave at most
  constexpr int BUF = GPW * NW * 1024;
  constexpr int XCH = NSP == 2 ? SP * NSP * 6 * 64 : 1;  // f32x4 exchange slots
  // key and query rows of a chunk (two buffers each, alternating like the record's):
  // rows of RB bytes whose 16-byte pieces are permuted by an XOR with the row index, so
  // that the 16 rows of one operand read land in distinct banks
  constexpr int RB = D * ESZ, PPR = RB / 16, RPG = 1024 / RB, KQG = 64 / RPG, KQPW = 2 * KQG / NW;
  static_assert(KSH * NSP == KSD && DTH * NSP == DT && (VNP == 4 || VNP == 8) && VG * 1024 == 64 * VRB, "shape");
  static_assert(RPG * RB == 1024 && KQPW * NW == 2 * KQG, "key/query staging");
  static_assert(2 * BUF + 16 * XCH + 4 * 64 * RB <= 160 * 1024, "LDS budget");
  const int seq = u / p.Hv, h = u - seq * p.Hv;
  const int hk = h / p.group;
  constexpr int q = Q, jj = Q / NSP, w = Q % NSP;  // slab within the pair, key half
  const int sl = SP * sg + jj;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int my_row = 16 * sl + col;
  const_table* tab = kernarg_table();
  const SeqEntry se = seq_entry(tab, seq);
  const float* sq_src = static_cast<const float*>(se.src);
  float* sq_dst = static_cast<float*>(se.dst);
  const int cb = se.unit0, ce = se.unit0 + se.n_units;
  const uint32_t blk = (uint32_t)tab->block;
  const size_t head_off = (size_t)h * D * D;
  constexpr int jt0 = DTH * w, s0 = KSH * w;  // first state tile and k-step of this wave

  f32x4 S[DTH];
#pragma unroll
  for (int j = 0; j < DTH; ++j) {
    if (sq_src)
      S[j] = *reinterpret_cast<const f32x4*>(sq_src + head_off + (size_t)my_row * D + kcol<D>(jt0 + j, grp));
    else
      S[j] = zero4();
  }
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int j = 0; j < DTH; ++j) *reinterpret_cast<f32x4*>(dst + kcol<D>(jt0 + j, grp)) = S[j];
  };
  if (cb >= ce) {
    store_state(sq_dst + head_off + (size_t)my_row * D);
    return;
  }

  // ---- per-lane byte offsets, fixed for the kernel
  const uint32_t qsb = (uint32_t)p.qk_stride * ESZ, vsb = (uint32_t)p.v_stride * ESZ;
  const uint32_t osb = (uint32_t)p.Hv * D * 4;
  uint32_t kq_off[4], o_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kq_off[i] = (16 * i + col) * qsb + kcol<D>(0, grp) * ESZ;
    o_off[i] = (4 * grp + i) * osb + col * 4;
  }
  // this lane's value column in a staged row (row t adds t * VRB); (t / 4) % 4 = grp
  // for every row the lane reads
  // this lane's value column in a staged row t = 16 mt + 4 grp + r (row t adds t * VRB;
  // (t / 4) % VNP depends on mt and grp only)
  const int v_byte = (16 * jj + col) * ESZ;
  auto v_rd = [&](int mt) { return V_OFF + 16 * ((v_byte >> 4) ^ ((4 * mt + grp) & (VNP - 1))) + (v_byte & 15); };

  // Chunks are derived from the sequence's entry (scalar arithmetic); the checkpoint
  // page id of a chunk that ends on a block boundary is fetched with a vector load a
  // chunk ahead (a scalar load would make every wait on LDS reads a wait for it too).
  // The descriptor bounds the page list, so the unused fetches of chunks that end off a
  // boundary (index clamped to 0) never leave it.
  const rsrc_t rpg = make_rsrc(page_list(tab), (uint32_t)tab->n_pages * 4u);
  auto page_raw = [&](const ChunkPos& cd) {
    return __builtin_amdgcn_raw_buffer_load_b32(rpg, (uint32_t)(cd.page_index > 0 ? cd.page_index : 0) * 4u, 0, 0);
  };

  // ---- copies of chunk c into buffer B: 1 KiB granules g = q, q + NW, ... < G.  A wave
  //      issues the same copies on every path (the last chunk stages itself again), so
  //      the compiler's counts of outstanding loads stay exact.  The bounds of both
  //      descriptors are in the per-lane offset: lanes past the record or past the
  //      chunk's last row write zeros.
  const IO* v_pair = p.v + (int64_t)h * D + 16 * SP * sg;
  auto stage_chunk = [&](const ChunkPos& cd, int c, lds_u8* B) {
    const rsrc_t rr = make_rsrc(p.factors + ((size_t)c * p.Hv + h) * p.factor_stride, (uint32_t)Cfg::REC_BYTES);
    const rsrc_t rv = make_rsrc(v_pair + cd.row * p.v_stride, (uint32_t)cd.len * vsb);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = q + gi * NW;  // a constant of this wave
      if (g >= G) continue;
      const bool is_v = g >= RG;
      const uint32_t t = (64u / VNP) * (uint32_t)(g - RG) + (uint32_t)lane / VNP;
      const uint32_t lp = ((uint32_t)lane % VNP) ^ ((t >> 2) & (VNP - 1));
      const uint32_t voff = g < RG ? 1024u * g + 16u * lane : is_v ? t * vsb + 16u * lp : (uint32_t)Cfg::REC_BYTES;
      dma16(is_v ? rv : rr, B + 1024 * g, voff);
    }
  };

  // copies of the chunk's key rows (into Kd) and query rows: KQPW granules per wave,
  // same on every path
  // which: 0 the key rows, 1 the query rows, 2 both
  auto stage_kq = [&](const ChunkPos& cd, lds_u8* Kd, lds_u8* Qd, const int which) {
    const rsrc_t rk = make_rsrc(p.k + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)cd.len * qsb);
    const rsrc_t rq = make_rsrc(p.q + cd.row * p.qk_stride + (int64_t)hk * D, (uint32_t)cd.len * qsb);
#pragma unroll
    for (int gi = 0; gi < KQPW; ++gi) {
      const int g = q + gi * NW;  // wave-uniform: granules 0 .. KQG-1 keys, then queries
      if (which != 2 && which != (g < KQG ? 0 : 1)) continue;
      const uint32_t r = RPG * (uint32_t)(g % KQG) + (uint32_t)lane / PPR;
      const uint32_t lp = ((uint32_t)lane % PPR) ^ (r % PPR);
      if (g < KQG)
        dma16(rk, Kd + 1024 * g, r * qsb + 16u * lp);
      else
        dma16(rq, Qd + 1024 * (g - KQG), r * qsb + 16u * lp);
    }
  };
  // this wave's A operands of X and Y: row 16 mt + col, key columns 32 (s0 + s) + 8 grp ..
  RowOp<IO> Kop[4][KSH], Qop[4][KSH];
  auto read_kq = [&](const lds_u8* Kb, const lds_u8* Qb, int s) {  // k-step s0 + s
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = 16 * mt + col;
      const int off = r * RB + 16 * ((grp + 4 * (s0 + s)) ^ (r % PPR));
      Kop[mt][s].v = lds_load<bf16x8>(Kb + off);
      Qop[mt][s].v = lds_load<bf16x8>(Qb + off);
    }
  };
  // A operands of K^T for the state update (state tile jt0 + j, k-step s over the chunk
  // rows), read transposed from the staged key rows.  In each 16-lane group of a
  // transposing 64-bit read, lane i receives, as its element e, the 16-bit value at the
  // address of lane 4 e + i / 4 plus i % 4 elements.  Lane L = 16 g + 4 e + c thus names
  // row t = 32 s + 16 h + 4 g + e (half h = 0, 1 of the eight kappa elements) at the four
  // key columns kcol(jt, c) .. + 3, and lane (col, g) receives K[t][key of its row col].
  typedef short v4s __attribute__((ext_vector_type(4)));
  auto read_kt = [&](const lds_u8* Kb, int j, int s) {
    const int jt = jt0 + j;
    const int pc = 4 * (jt >> 1) + (lane & 3), half8 = 8 * (jt & 1);  // 16-byte piece, 8-byte half
    u32x2 w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 32 * s + 16 * h + 4 * grp + ((lane >> 2) & 3);
      const lds_u8* a = Kb + t * RB + 16 * (pc ^ (t % PPR)) + half8;
      w[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (__attribute__((address_space(3))) v4s*)a));
    }
    return __builtin_bit_cast(bf16x8, u32x4{w[0][0], w[0][1], w[1][0], w[1][1]});
  };
  auto frag = [&](const lds_u8* B, int off, int f) {
    return lds_load<bf16x8>(B + off + 1024 * f + 16 * lane);
  };
  auto vrow4 = [&](const lds_u8* B, int plane, int mt) {  // rows 16 mt + 4 grp .. + 3 of a vector plane
    return lds_load<f32x4>(B + Cfg::VEC_OFF + plane * CT * 4 + 64 * mt + 16 * grp);
  };
  auto issue_point = [] { __builtin_amdgcn_sched_barrier(0); };

  // cur: the chunk in work; nxt: the one after it (the last chunk is its own next)
  uint32_t npos = ce - cb > 1 ? (uint32_t)se.p0 + (uint32_t)chunk_at(se, (uint32_t)se.p0, blk).len : (uint32_t)se.p0;
  ChunkPos cur = chunk_at(se, (uint32_t)se.p0, blk);
  ChunkPos nxt = chunk_at(se, npos, blk);
  uint32_t cur_pid = page_raw(cur);
  stage_chunk(cur, cb, stage0);
  stage_kq(cur, kbuf0, qbuf0, 2);

  // Stores are issued one chunk late, right after the next chunk's barrier: the
  // barrier's wait for this wave's copies (vmcnt) also counts stores, so a store issued
  // late in a chunk would hold every wave at the next barrier until it completed.  The
  // outputs of a chunk wait in registers, and a checkpoint is the state as it stands
  // until the next chunk's update.
  f32x4 o_pend[MR];
  ChunkPos o_chunk = cur;
  bool o_have = false;
  int32_t ck_pid = -1;
  auto flush_pending = [&]() {
    if (o_have) {
      const rsrc_t ro =
          make_rsrc(p.o + o_chunk.row * (int64_t)p.Hv * D + (int64_t)h * D + 16 * sl, (uint32_t)o_chunk.len * osb);
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) st4(ro, o_off[r] + 16 * omt<NSP>(w, i) * osb, o_pend[i][r]);
    }
    if (ck_pid >= 0)
      store_state(reinterpret_cast<float*>(p.ckpt_pool + (size_t)ck_pid * p.page_bytes) + head_off +
                  (size_t)my_row * D);
  };

  auto step = [&](const int c, const lds_u8* Bc, lds_u8* Bn, const lds_u8* Kc, lds_u8* Kn, const lds_u8* Qc,
                  lds_u8* Qn) {
    const bool more = c + 1 < ce;
    // Every wave's copies of this chunk (into Bc, Kc and Qc) have landed once each wave has
    // waited for all of its own vector memory operations and passed the barrier.  The
    // wait is explicit: the compiler's own count of outstanding LDS DMA follows the
    // data a wave reads itself, not the copies its partners read.  The copies were
    // issued most of a chunk earlier, so the wait rarely stalls.
    full_barrier();
    // the previous chunk's outputs and checkpoint
    flush_pending();
    // copies of the next chunk's key rows (the last chunk stages itself again: every
    // path issues the same copies, so the compiler's counts of outstanding loads stay
    // exact)
    stage_kq(nxt, Kn, Qn, 0);
    const uint32_t nxt_pid = page_raw(nxt);

    read_kq(Kc, Qc, 0);
    issue_point();

    // ---- A: X = K S^T and Y = Q S^T (this wave's k-steps), eight accumulator chains;
    //      each k-step's key and query operands are requested one k-step ahead
    f32x4 X[4], Y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) X[mt] = Y[mt] = zero4();
#pragma unroll
    for (int s = 0; s < KSH; ++s) {
      if (s + 1 < KSH) read_kq(Kc, Qc, s + 1);
      issue_point();
      bf16x8 sop[NTF];
      reg_operand<NTF>(S[2 * s], (2 * s + 1 < DTH) ? S[2 * s + 1] : zero4(), sop);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        bf16x8 ak[NTI], aq[NTI];
        row_terms<NTI>(Kop[mt][s], ak);
        row_terms<NTI>(Qop[mt][s], aq);
        mma_terms<NTI, NTF, ORD>(X[mt], ak, sop);
        mma_terms<NTI, NTF, ORD>(Y[mt], aq, sop);
      }
    }
    issue_point();
    // the next chunk's query rows
    stage_kq(nxt, Kn, Qn, 1);
    // with two waves per slab, add the partner's partial sums (X for all rows, Y for
    // this wave's output rows) through LDS
    f32x4 Ym[MR];
    float Vv[4][4];
    f32x4 veg[4];
    bf16x8 Tf[kFragCombos][NTF];
    auto read_b = [&]() {  // operands of phase B
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Vv[mt][r] = bf16_to_f32(lds_load<bf16_bits>(Bc + v_rd(mt) + (16 * mt + 4 * grp + r) * VRB));
        veg[mt] = vrow4(Bc, Cfg::V_EG, mt);
      }
#pragma unroll
      for (int f = 0; f < kFragCombos; ++f)
#pragma unroll
        for (int i = 0; i < NTF; ++i) Tf[f][i] = frag(Bc, Cfg::T_OFF, f * NTF + i);
    };
    if constexpr (NSP == 2) {
      f32x4* mine = xch + ((jj * NSP + w) * 6) * 64 + lane;
      const f32x4* other = xch + ((jj * NSP + (w ^ 1)) * 6) * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) mine[mt * 64] = X[mt];
#pragma unroll
      for (int i = 0; i < MR; ++i) mine[(4 + i) * 64] = Y[omt<NSP>(w ^ 1, i)];
      // the barrier waits for this wave's LDS traffic: the partial sums just written,
      // not the operands of phase B, which are requested after it (measured: issuing
      // them before the barrier held every wave there for all of them)
      lds_barrier();
      read_b();
      // the next chunk's record and value rows
      stage_chunk(nxt, more ? c + 1 : c, Bn);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 xo = other[mt * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r) X[mt][r] += xo[r];
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const f32x4 yo = other[(4 + i) * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ym[i][r] = Y[omt<NSP>(w, i)][r] + yo[r];
      }
    } else {
#pragma unroll
      for (int i = 0; i < MR; ++i) Ym[i] = Y[omt<NSP>(w, i)];
      read_b();
      stage_chunk(nxt, more ? c + 1 : c, Bn);
    }

    // ---- B: R' = V - exp(g) X, Dt = T'' R' over the nonzero k-steps
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) R[mt][r] = fmaf(-veg[mt][r], X[mt][r], Vv[mt][r]);
    bf16x8 Rop[2][NTF];
    reg_operand<NTF>(R[0], R[1], Rop[0]);
    reg_operand<NTF>(R[2], R[3], Rop[1]);
    f32x4 Dt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Dt[mt] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 2 * s; mt < 4; ++mt) mma_terms<NTF, NTF, ORD>(Dt[mt], Tf[frag_combo(mt, s)], Rop[s]);

    // ---- operands of phase C, requested while the products above run
    f32x4 vegs[MR];
    bf16x8 Pf[MR][2][NTF];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int mt = omt<NSP>(w, i);
      vegs[i] = vrow4(Bc, Cfg::V_EGS, mt);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s <= (mt >> 1))
#pragma unroll
          for (int t = 0; t < NTF; ++t) Pf[i][s][t] = frag(Bc, Cfg::P_OFF, frag_combo(mt, s) * NTF + t);
    }
    issue_point();

    // ---- C: O = scale exp(g) Y + PT'' R' for this wave's row tiles (stored after the
    //      next barrier)
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const int mt = omt<NSP>(w, i);
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = Ym[i][r] * vegs[i][r];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s <= (mt >> 1)) mma_terms<NTF, NTF, ORD>(acc, Pf[i][s], Rop[s]);
      o_pend[i] = acc;
    }
    o_chunk = cur;
    o_have = true;

    // ---- operands of phase D, requested while the products above run
    bf16x8 KTf[DTH][2][NTI];
#pragma unroll
    for (int j = 0; j < DTH; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s) KTf[j][s][0] = read_kt(Kc, j, s);
    const float egn = lds_load<float>(Bc + Cfg::EGN_OFF);
    issue_point();

    // ---- D: S^T <- exp(g_n) S^T + K^T Dt for this wave's tiles
    {
      bf16x8 Dtop[2][NTF];
      reg_operand<NTF>(Dt[0], Dt[1], Dtop[0]);
      reg_operand<NTF>(Dt[2], Dt[3], Dtop[1]);
#pragma unroll
      for (int j = 0; j < DTH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[j][r] *= egn;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < DTH; ++j) mma_terms<NTI, NTF, ORD>(S[j], KTf[j][s], Dtop[s]);
    }

    // ---- checkpoint: the state after this chunk, bit for bit (stored after the next
    //      barrier, before the next update changes it)
    ck_pid = cur.page_index >= 0 ? (int32_t)__builtin_amdgcn_readfirstlane(cur_pid) : -1;
    // advance: the chunk after next (the last chunk stays its own next)
    const uint32_t nnpos = c + 2 < ce ? npos + (uint32_t)nxt.len : npos;
    cur = nxt;
    cur_pid = nxt_pid;
    nxt = chunk_at(se, nnpos, blk);
    npos = nnpos;
  };

  // two steps per trip, so that each step's buffers are fixed LDS objects
#pragma unroll 1
  for (int c = cb; c < ce; c += 2) {
    step(c, stage0, stage1, kbuf0, kbuf1, qbuf0, qbuf1);
    if (c + 1 < ce) step(c + 1, stage1, stage0, kbuf1, kbuf0, qbuf1, qbuf0);
  }
  flush_pending();
  store_state(sq_dst + head_off + (size_t)my_row * D);
}

// LDS of a staged-scan workgroup (the layout is stated in scan_staged_wave).
template <typename IO, int D>
struct StagedLds {
  using Cfg = PrefillCfg<IO, D>;
  using Shp = ScanStaged<IO, D>;
  static constexpr int RG = (Cfg::REC_BYTES + 1023) / 1024;
  static constexpr int G = RG + 64 * Shp::SP * 16 * (int)sizeof(IO) / 1024;
  static constexpr int BUF = (G + Shp::NW - 1) / Shp::NW * Shp::NW * 1024;
  static constexpr int XCH = Shp::NSP == 2 ? Shp::SP * Shp::NSP * 6 * 64 : 1;
  static constexpr int KR = 64 * D * (int)sizeof(IO);  // one chunk's key (or query) rows
};

template <typename IO, int D>
__global__ __launch_bounds__(256) void scan_staged_kernel(ScanArgs<IO> p) {
  using L = StagedLds<IO, D>;
  constexpr int NG = ScanStaged<IO, D>::NG;
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[L::BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[L::BUF];
  // the key and query buffers as separate objects: the compiler tracks outstanding LDS
  // DMA per object, and a chunk's rows are read after the next chunk's are requested
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[L::KR];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[L::KR];
  __shared__ __attribute__((aligned(1024))) uint8_t qbuf0[L::KR];
  __shared__ __attribute__((aligned(1024))) uint8_t qbuf1[L::KR];
  // [slab][wave][X tiles 0..3, partner's Y tiles][lane]
  __shared__ __attribute__((aligned(16))) f32x4 xch[L::XCH];

  // All workgroups of one (sequence, head) go to the same XCD (workgroups are dealt
  // to the eight XCDs round robin), so their shared chunk data meets in one L2.
  const int blk = blockIdx.x;
  const int u = (blk / (8 * NG)) * 8 + (blk & 7);
  const int sg = (blk >> 3) % NG;
  if (u >= kernarg_table()->n_seqs * p.Hv) return;
  switch (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))) {
    case 0: scan_staged_wave<IO, D, 0>(p, u, sg, (lds_u8*)stage0, (lds_u8*)stage1, (lds_u8*)kbuf0,
                                                (lds_u8*)kbuf1, (lds_u8*)qbuf0, (lds_u8*)qbuf1, xch); break;
    case 1: scan_staged_wave<IO, D, 1>(p, u, sg, (lds_u8*)stage0, (lds_u8*)stage1, (lds_u8*)kbuf0,
                                                (lds_u8*)kbuf1, (lds_u8*)qbuf0, (lds_u8*)qbuf1, xch); break;
    case 2: scan_staged_wave<IO, D, 2>(p, u, sg, (lds_u8*)stage0, (lds_u8*)stage1, (lds_u8*)kbuf0,
                                                (lds_u8*)kbuf1, (lds_u8*)qbuf0, (lds_u8*)qbuf1, xch); break;
    default: scan_staged_wave<IO, D, 3>(p, u, sg, (lds_u8*)stage0, (lds_u8*)stage1, (lds_u8*)kbuf0,
                                                (lds_u8*)kbuf1, (lds_u8*)qbuf0, (lds_u8*)qbuf1, xch); break;
  }
}

// ==================================================================================
// Launchers
template <typename IO, int D>
static hipError_t launch_factorize_t(const FactorizeArgs<IO>& a, hipStream_t st) {
  if (a.tab.n_units == 0) return hipSuccess;
  dim3 grid(a.Hv, a.tab.n_units);
  hipLaunchKernelGGL((factorize_kernel<IO, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename IO, int D>
static hipError_t launch_scan_t(const ScanArgs<IO>& a, hipStream_t st) {
  const int64_t units = (int64_t)a.tab.n_seqs * a.Hv;
  if (units == 0) return hipSuccess;
  if constexpr (ScanStaged<IO, D>::OK) {
    using Shp = ScanStaged<IO, D>;
    const int64_t blocks = (units + 7) / 8 * 8 * Shp::NG;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((scan_staged_kernel<IO, D>), dim3((unsigned)blocks), dim3(64 * Shp::NW), 0, st, a);
  } else {
    const int64_t blocks = (units + 7) / 8 * 8 * (D / 16);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((scan_kernel<IO, D>), dim3((unsigned)blocks), dim3(64 * ScanSplit<D>::NSP), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_factorize(const FactorizeArgs<bf16_bits>& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch_factorize_t<bf16_bits, 16>(a, st);
    case 32: return launch_factorize_t<bf16_bits, 32>(a, st);
    case 64: return launch_factorize_t<bf16_bits, 64>(a, st);
    case 128: return launch_factorize_t<bf16_bits, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_factorize(const FactorizeArgs<float>& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch_factorize_t<float, 16>(a, st);
    case 32: return launch_factorize_t<float, 32>(a, st);
    case 64: return launch_factorize_t<float, 64>(a, st);
    case 128: return launch_factorize_t<float, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_scan(const ScanArgs<bf16_bits>& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch_scan_t<bf16_bits, 16>(a, st);
    case 32: return launch_scan_t<bf16_bits, 32>(a, st);
    case 64: return launch_scan_t<bf16_bits, 64>(a, st);
    case 128: return launch_scan_t<bf16_bits, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_scan(const ScanArgs<float>& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch_scan_t<float, 16>(a, st);
    case 32: return launch_scan_t<float, 32>(a, st);
    case 64: return launch_scan_t<float, 64>(a, st);
    case 128: return launch_scan_t<float, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
