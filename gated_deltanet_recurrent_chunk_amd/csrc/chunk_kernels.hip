// chunk_kernels.hip -- chunked gated delta rule on gfx950: factorize, scan, replay flush.
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
// T depends only on k, a, b, so it is computed for every chunk at once
// (factorize_kernel); the scan then walks each sequence's chunks in order with the
// state held in registers.  Rows of the state are independent of each other, so a
// sequence-head is split into 16-row slabs, one per wave.  Gates stay in log space
// and only exp(g_t - g_s) with s <= t is formed, so no factor exceeds one.
//
// Chunks are cut at every multiple of 64 tokens, of the cache block and at the call
// ends (plan.cpp); when a chunk ends on a block boundary the scan stores the state
// bits into that boundary's checkpoint page, the state the next chunk starts from
// ("Prefix caching on Gated DeltaNet hybrids", "Why hits were wrong": a full block
// keeps the recurrent state after its last token).
//
// The replay flush ("Caching less to serve more requests", "What we changed") is the
// same update for the n accepted rows of a request's input log, one block, no outputs.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace gdn {

namespace {

// Contraction-permuted LDS operand for row `row` of a row-major bf16 plane with row
// stride `ld` (elements), k-step s, lane group g.
__device__ __forceinline__ bf16x8 row_operand(const bf16_bits* plane, int ld, int row, int s, int g) {
  const bf16_bits* p = plane + row * ld + 32 * s + 4 * g;
  return lds_operand(p, p + 16);
}

// All terms of a row operand from NT planes spaced `pstride` elements apart.  LEN is
// the length of the contracted row: when it is not a multiple of 32 the last k-step
// has only 16 real elements and elements 4..7 of every lane are zero (not read).
template <int NT, int LEN = 64>
__device__ __forceinline__ void row_operand_terms(const bf16_bits* planes, int pstride, int ld, int row,
                                                  int s, int g, bf16x8 (&out)[NT]) {
  if constexpr (LEN % 32 != 0) {
    if (s == LEN / 32) {
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const bf16_bits* p = planes + i * pstride + row * ld + 32 * s + 4 * g;
        uint2 lo = *reinterpret_cast<const uint2*>(p);
        typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
        u32x4 w = {lo.x, lo.y, 0u, 0u};
        out[i] = __builtin_bit_cast(bf16x8, w);
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) out[i] = row_operand(planes + i * pstride, ld, row, s, g);
}

// 16-byte global load of VEC io elements (zeros when !pred: the row is not read).
template <typename IO>
__device__ __forceinline__ uint4 load16(const IO* p, bool pred) {
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

// ----------------------------------------------------------------------------------
// Chunk factorization shared by the prefill pre-pass and the replay flush.
//   Ks: NTI planes of CT x (D + 8) bf16 terms of the chunk's key rows (rows >= n zero).
//   g_t, b_t for lane t are given (t >= n: g_t = g_{n-1}, b_t = 0).
// Writes T = (I + A)^-1 as NTF bf16 planes (row stride tld, plane stride tps) and the
// four per-row vectors g, exp(g), b, exp(g_n - g) (vec[0..4*CT)).  One wave.
template <int CT, int D, int NTI, int NTF, int ORD>
__device__ __forceinline__ void factorize_chunk(const bf16_bits* Ks, int kps, float (*As)[CT + 4], int n, float g,
                                float bb, bf16_bits* Tout, int tps, int tld, float* vec_out,
                                float* vec_lds) {
  constexpr int KP = D + 8;
  constexpr int DT = D / 16, KSD = (DT + 1) / 2;
  constexpr int MT = CT / 16;
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
  __syncthreads();

  // A = strict lower part of diag(b) (exp(g_t - g_s)) * K K^T
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        bf16x8 a[NTI], b[NTI];
        row_operand_terms<NTI, D>(Ks, kps, KP, 16 * mt + col, s, grp, a);
        row_operand_terms<NTI, D>(Ks, kps, KP, 16 * nt + col, s, grp, b);
        mma_terms<NTI, NTI, ORD>(acc, a, b);
      }
      const int sc = 16 * nt + col;
      const float gs = vec_lds[sc];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * grp + r;
        float val = 0.f;
        if (sc < t && t < n) val = vec_lds[CT + t] * __expf(vec_lds[t] - gs) * acc[r];
        As[t][sc] = val;
      }
    }
  }
  __syncthreads();

  // Forward substitution, lane j owns column j:  T[t][j] = [t == j] - sum_{s<t} A[t][s] T[s][j]
  float Tc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < t; ++s) acc = fmaf(As[t][s], Tc[s], acc);
    Tc[t] = (t == lane ? 1.f : 0.f) - acc;
    // row t is finished before the loads of row t + 1 start: at most one row of A is
    // live in registers
    asm volatile("" : "+v"(Tc[t]) : : "memory");
  }
  if (lane < CT) {
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      bf16_bits tt[NTF];
      split_terms<NTF>(Tc[t], tt);
#pragma unroll
      for (int i = 0; i < NTF; ++i) Tout[i * tps + t * tld + lane] = tt[i];
    }
  }
}

// Store a 16-byte vector of key/query elements into NT bf16 planes at row t, columns
// j0.., and optionally into transposed planes (row = column index).
template <typename IO, int NT>
__device__ __forceinline__ void store_terms(const uint4& v, bf16_bits* planes, int pstride, int ld, int t,
                                            int j0, bf16_bits* tplanes, int tpstride, int tld) {
  constexpr int VEC = 16 / sizeof(IO);
  if constexpr (NT == 1 && sizeof(IO) == 2) {
    *reinterpret_cast<uint4*>(planes + t * ld + j0) = v;
    if (tplanes) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        uint32_t w = (&v.x)[e >> 1];
        tplanes[(j0 + e) * tld + t] = (bf16_bits)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      bf16_bits tt[NT];
      split_terms<NT>(elem<IO>(v, e), tt);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        planes[i * pstride + t * ld + j0 + e] = tt[i];
        if (tplanes) tplanes[i * tpstride + (j0 + e) * tld + t] = tt[i];
      }
    }
  }
}

}  // namespace

// ==================================================================================
// Pre-pass: one wave per (chunk, value head).
template <typename IO, int D>
__global__ __launch_bounds__(64) void factorize_kernel(FactorizeArgs<IO> p) {
  constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  constexpr int CT = kChunk;
  constexpr int KP = D + 8;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;
  __shared__ bf16_bits Ks[NTI * CT * KP];
  __shared__ float As[CT][CT + 4];
  __shared__ float vec_lds[2 * CT];

  const int c = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const ChunkDesc cd = p.chunks[c];
  const int n = cd.len;
  const int hk = h / p.group;
  const IO* kb = p.k + cd.row * p.qk_stride + (int64_t)hk * D;
  for (int idx = lane; idx < CT * PER_ROW; idx += 64) {
    const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    uint4 v = load16(kb + (int64_t)t * p.qk_stride + j0, t < n);
    store_terms<IO, NTI>(v, Ks, CT * KP, KP, t, j0, nullptr, 0, 0);
  }
  float la = 0.f, bb = 0.f;
  if (lane < n) {
    const int64_t ai = (cd.row + lane) * (int64_t)p.Hv + h;
    la = __logf(p.a[ai]);
    bb = p.b[ai];
  }
  const float g = wave_inclusive_scan(la);
  uint8_t* rec = p.factors + ((size_t)h * p.n_chunks + c) * p.factor_stride;
  bf16_bits* Tout = reinterpret_cast<bf16_bits*>(rec);
  float* vec_out = reinterpret_cast<float*>(rec + (size_t)NTF * CT * CT * 2);
  factorize_chunk<CT, D, NTI, NTF, ORD>(Ks, CT * KP, As, n, g, bb, Tout, CT * CT, CT, vec_out, vec_lds);
}

// ==================================================================================
// Scan: one workgroup per (sequence, value head, group of up to 64 value rows); one
// wave per 16-row slab.  The chunk loop keeps the slab in registers, prefetches the
// next chunk's operands into registers while computing the current one, and stages
// them through LDS.
template <typename IO, int D>
__global__ __launch_bounds__(64 * ScanShape<D>::NW) void scan_kernel(ScanArgs<IO> p) {
  constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  constexpr int NW = ScanShape<D>::NW, RW = 16 * NW, NTH = 64 * NW;
  constexpr int CT = kChunk;
  constexpr int KP = D + 8, TP = CT + 8, VP = RW + 4;
  constexpr int DT = D / 16, KSD = (DT + 1) / 2;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC, PER_VROW = RW / VEC;
  constexpr int KN = (CT * PER_ROW + NTH - 1) / NTH;
  constexpr int VN = (CT * PER_VROW + NTH - 1) / NTH;
  constexpr int TN = (NTF * CT * CT / 8 + NTH - 1) / NTH;
  constexpr int FREC_T = NTF * CT * CT * 2;  // bytes of T planes in a factor record

  __shared__ bf16_bits Ks[NTI * CT * KP];
  __shared__ bf16_bits KTs[NTI * D * TP];
  __shared__ bf16_bits Qs[NTI * CT * KP];
  __shared__ float Vs[CT * VP];
  __shared__ bf16_bits Ts[NTF * CT * TP];
  __shared__ bf16_bits Ps[NTF * CT * TP];
  __shared__ float vec[4 * CT];  // g, exp(g), b, exp(g_n - g)

  const int seq = blockIdx.x, h = blockIdx.y, rg = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int hk = h / p.group;
  const int i0 = rg * RW;               // first value row of the workgroup
  const int iw = wave * 16;             // first value row of this wave within the group
  const ScanSeq sq = p.seqs[seq];
  const size_t head_off = (size_t)h * D * D;
  const int my_row = i0 + iw + col;     // value row held by this lane

  // ---- incoming state slab: lane holds S[my_row][16 jt + 4 grp + r]
  f32x4 S[DT];
#pragma unroll
  for (int jt = 0; jt < DT; ++jt) {
    if (sq.src)
      S[jt] = *reinterpret_cast<const f32x4*>(sq.src + head_off + (size_t)my_row * D + 16 * jt + 4 * grp);
    else
      S[jt] = zero4();
  }

  // ---- prefetch registers
  uint4 kr[KN], qr[KN], vr[VN], tr[TN];
  uint4 vecr = uint4{0u, 0u, 0u, 0u};
  auto prefetch = [&](int c) {
    const ChunkDesc cd = p.chunks[c];
    const int n = cd.len;
    const IO* kb = p.k + cd.row * p.qk_stride + (int64_t)hk * D;
    const IO* qb = p.q + cd.row * p.qk_stride + (int64_t)hk * D;
    const IO* vb = p.v + cd.row * p.v_stride + (int64_t)h * D + i0;
#pragma unroll
    for (int u = 0; u < KN; ++u) {
      const int idx = tid + u * NTH;
      const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
      const bool ok = idx < CT * PER_ROW && t < n;
      kr[u] = load16(kb + (int64_t)t * p.qk_stride + j0, ok);
      qr[u] = load16(qb + (int64_t)t * p.qk_stride + j0, ok);
    }
#pragma unroll
    for (int u = 0; u < VN; ++u) {
      const int idx = tid + u * NTH;
      const int t = idx / PER_VROW, c0 = (idx % PER_VROW) * VEC;
      vr[u] = load16(vb + (int64_t)t * p.v_stride + c0, idx < CT * PER_VROW && t < n);
    }
    const uint8_t* rec = p.factors + ((size_t)h * p.n_chunks + c) * p.factor_stride;
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      const int idx = tid + u * NTH;
      tr[u] = idx < NTF * CT * CT / 8 ? reinterpret_cast<const uint4*>(rec)[idx] : uint4{0u, 0u, 0u, 0u};
    }
    if (tid < CT) vecr = reinterpret_cast<const uint4*>(rec + FREC_T)[tid];
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < KN; ++u) {
      const int idx = tid + u * NTH;
      if (idx < CT * PER_ROW) {
        const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
        store_terms<IO, NTI>(kr[u], Ks, CT * KP, KP, t, j0, KTs, D * TP, TP);
        store_terms<IO, NTI>(qr[u], Qs, CT * KP, KP, t, j0, nullptr, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < VN; ++u) {
      const int idx = tid + u * NTH;
      if (idx < CT * PER_VROW) {
        const int t = idx / PER_VROW, c0 = (idx % PER_VROW) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) Vs[t * VP + c0 + e] = elem<IO>(vr[u], e);
      }
    }
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      const int idx = tid + u * NTH;
      if (idx < NTF * CT * CT / 8) {
        const int pl = idx / (CT * CT / 8), rem = idx % (CT * CT / 8);
        const int t = rem / (CT / 8), s0 = (rem % (CT / 8)) * 8;
        *reinterpret_cast<uint4*>(Ts + pl * CT * TP + t * TP + s0) = tr[u];
      }
    }
    if (tid < CT) reinterpret_cast<uint4*>(vec)[tid] = vecr;
  };

  if (sq.chunk_begin < sq.chunk_end) prefetch(sq.chunk_begin);

  for (int c = sq.chunk_begin; c < sq.chunk_end; ++c) {
    const ChunkDesc cd = p.chunks[c];
    const int n = cd.len;
    __syncthreads();
    stage();
    __syncthreads();
    if (c + 1 < sq.chunk_end) prefetch(c + 1);

    // ---- P = mask o exp(g_t - g_s) (Q K^T), computed as P^T = K Q^T tiles (M = s, N = t)
    //      so each tile lands in LDS in the row layout the P Delta product reads.
    {
      // 10 causal tiles plus the two upper tiles the P Delta k-steps touch (all zero)
      // tile it -> (ms, nt), two bits each: ms = 0,0,1,0,1,2,0,1,2,3,1,3  nt = 0,1,1,2,2,2,3,3,3,3,0,2
      constexpr int NPT = 12;
      constexpr uint32_t MS_CODE = 0u | (0u << 2) | (1u << 4) | (0u << 6) | (1u << 8) | (2u << 10) | (0u << 12) |
                                   (1u << 14) | (2u << 16) | (3u << 18) | (1u << 20) | (3u << 22);
      constexpr uint32_t NT_CODE = 0u | (1u << 2) | (1u << 4) | (2u << 6) | (2u << 8) | (2u << 10) | (3u << 12) |
                                   (3u << 14) | (3u << 16) | (3u << 18) | (0u << 20) | (2u << 22);
      for (int it = wave; it < NPT; it += NW) {
        const int ms = (MS_CODE >> (2 * it)) & 3, nt = (NT_CODE >> (2 * it)) & 3;
        f32x4 acc = zero4();
        if (ms <= nt) {
#pragma unroll
          for (int s = 0; s < KSD; ++s) {
            bf16x8 a[NTI], b[NTI];
            row_operand_terms<NTI, D>(Ks, CT * KP, KP, 16 * ms + col, s, grp, a);
            row_operand_terms<NTI, D>(Qs, CT * KP, KP, 16 * nt + col, s, grp, b);
            mma_terms<NTI, NTI, ORD>(acc, a, b);
          }
        }
        const int t = 16 * nt + col;
        const float gt = vec[t];
        bf16_bits terms[4][NTF];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * ms + 4 * grp + r;
          float val = 0.f;
          if (s <= t && t < n) val = __expf(gt - vec[s]) * acc[r];
          split_terms<NTF>(val, terms[r]);
        }
#pragma unroll
        for (int i = 0; i < NTF; ++i) {
          uint2 w;
          w.x = (uint32_t)terms[0][i] | ((uint32_t)terms[1][i] << 16);
          w.y = (uint32_t)terms[2][i] | ((uint32_t)terms[3][i] << 16);
          *reinterpret_cast<uint2*>(Ps + i * CT * TP + t * TP + 16 * ms + 4 * grp) = w;
        }
      }
    }

    // ---- state operand terms (B operand, contraction over key channels)
    bf16x8 Sop[KSD][NTF];
#pragma unroll
    for (int s = 0; s < KSD; ++s)
      reg_operand<NTF>(S[2 * s], (2 * s + 1 < DT) ? S[2 * s + 1] : zero4(), Sop[s]);

    // ---- X = K S^T (rows t, column my_row), R = b (V - exp(g) X)
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        bf16x8 a[NTI];
        row_operand_terms<NTI, D>(Ks, CT * KP, KP, 16 * mt + col, s, grp, a);
        mma_terms<NTI, NTF, ORD>(acc, a, Sop[s]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * grp + r;
        float val = 0.f;
        if (t < n) val = vec[2 * CT + t] * (Vs[t * VP + iw + col] - vec[CT + t] * acc[r]);
        R[mt][r] = val;
      }
    }
    // ---- Delta = T R  (T lower triangular: skip the all-zero upper k-step)
    bf16x8 Rop[2][NTF];
    reg_operand<NTF>(R[0], R[1], Rop[0]);
    reg_operand<NTF>(R[2], R[3], Rop[1]);
    f32x4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dl[mt] = zero4();
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {
        bf16x8 a[NTF];
        row_operand_terms<NTF>(Ts, CT * TP, TP, 16 * mt + col, s, grp, a);
        mma_terms<NTF, NTF, ORD>(Dl[mt], a, Rop[s]);
      }
    }
    bf16x8 Dop[2][NTF];
    reg_operand<NTF>(Dl[0], Dl[1], Dop[0]);
    reg_operand<NTF>(Dl[2], Dl[3], Dop[1]);

    __syncthreads();  // P tiles from all waves are in LDS

    // ---- O = scale (exp(g) Q S^T + P Delta)
    {
      const size_t orow = (size_t)p.Hv * D;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
          bf16x8 a[NTI];
          row_operand_terms<NTI, D>(Qs, CT * KP, KP, 16 * mt + col, s, grp, a);
          mma_terms<NTI, NTF, ORD>(acc, a, Sop[s]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= vec[CT + 16 * mt + 4 * grp + r];
#pragma unroll
        for (int s = 0; s <= (mt >> 1); ++s) {
          bf16x8 a[NTF];
          row_operand_terms<NTF>(Ps, CT * TP, TP, 16 * mt + col, s, grp, a);
          mma_terms<NTF, NTF, ORD>(acc, a, Dop[s]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * grp + r;
          if (t < n) p.o[(size_t)(cd.row + t) * orow + (size_t)h * D + my_row] = p.scale * acc[r];
        }
      }
    }

    // ---- S^T <- exp(g_n) S^T + K^T (exp(g_n - g) o Delta)
    {
      f32x4 Dt[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Dt[mt][r] = vec[3 * CT + 16 * mt + 4 * grp + r] * Dl[mt][r];
      bf16x8 Dtop[2][NTF];
      reg_operand<NTF>(Dt[0], Dt[1], Dtop[0]);
      reg_operand<NTF>(Dt[2], Dt[3], Dtop[1]);
      const float egn = vec[CT + n - 1];
#pragma unroll
      for (int jt = 0; jt < DT; ++jt) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = egn * S[jt][r];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 a[NTI];
          row_operand_terms<NTI>(KTs, D * TP, TP, 16 * jt + col, s, grp, a);
          mma_terms<NTI, NTF, ORD>(acc, a, Dtop[s]);
        }
        S[jt] = acc;
      }
    }

    // ---- checkpoint: the state after this chunk, bit for bit
    if (cd.page >= 0) {
      float* dst = reinterpret_cast<float*>(p.ckpt_pool + (size_t)cd.page * p.page_bytes) + head_off +
                   (size_t)my_row * D;
#pragma unroll
      for (int jt = 0; jt < DT; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt + 4 * grp) = S[jt];
    }
  }

  {
    float* dst = sq.dst + head_off + (size_t)my_row * D;
#pragma unroll
    for (int jt = 0; jt < DT; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt + 4 * grp) = S[jt];
  }
}

// ==================================================================================
// Replay flush: one workgroup per (request, value head), one wave per 16-row slab of
// the state.  Reads the state once, factorizes the accepted rows (wave 0), applies
// them, writes the state once.
template <typename IO, int D, int CT>
__global__ __launch_bounds__(64 * (D / 16)) void flush_kernel(FlushArgs<IO> p) {
  constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  constexpr int NW = D / 16, NTH = 64 * NW;
  constexpr int KP = D + 8, TP = CT + 8, VP = D + 4;
  constexpr int DT = D / 16, KSD = (DT + 1) / 2;
  constexpr int MT = CT / 16, KST = (MT + 1) / 2;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;

  __shared__ bf16_bits Ks[NTI * CT * KP];
  __shared__ bf16_bits KTs[NTI * D * TP];
  __shared__ float Vs[CT * VP];
  __shared__ float As[CT][CT + 4];
  __shared__ bf16_bits Ts[NTF * CT * TP];
  __shared__ float vec[4 * CT];
  __shared__ float vec_tmp[2 * CT];

  const int r_ = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int slot = p.slot_ids[r_];
  const int n = p.n_accepted[r_];
  if (slot < -1 || slot >= p.n_slots || n < 0 || n > p.buf_rows) {
    if (tid == 0 && h == 0 && p.status) atomicOr(p.status, 1 << GDN_ERR_CAPACITY);
    return;
  }
  if (slot < 0 || n == 0) return;  // padding or nothing accepted: untouched

  const int hk = h / p.group;
  const int my_row = wave * 16 + col;
  float* state = p.state_pool + ((size_t)slot * p.Hv + h) * D * D;
  f32x4 S[DT];
#pragma unroll
  for (int jt = 0; jt < DT; ++jt)
    S[jt] = *reinterpret_cast<const f32x4*>(state + (size_t)my_row * D + 16 * jt + 4 * grp);

  // logged rows 0..n-1 of this slot
  const size_t row0 = (size_t)slot * p.buf_rows;
  const IO* kb = p.buf_k + row0 * p.Hqk * D + (size_t)hk * D;
  const IO* vb = p.buf_v + row0 * p.Hv * D + (size_t)h * D;
  for (int idx = tid; idx < CT * PER_ROW; idx += NTH) {
    const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    uint4 kv = load16(kb + (size_t)t * p.Hqk * D + j0, t < n);
    store_terms<IO, NTI>(kv, Ks, CT * KP, KP, t, j0, KTs, D * TP, TP);
    uint4 vv = load16(vb + (size_t)t * p.Hv * D + j0, t < n);
#pragma unroll
    for (int e = 0; e < VEC; ++e) Vs[t * VP + j0 + e] = elem<IO>(vv, e);
  }
  __syncthreads();
  if (wave == 0) {
    float la = 0.f, bb = 0.f;
    if (lane < n) {
      const size_t ai = (row0 + lane) * p.Hv + h;
      la = __logf(p.buf_a[ai]);
      bb = p.buf_b[ai];
    }
    const float g = wave_inclusive_scan(la);
    factorize_chunk<CT, D, NTI, NTF, ORD>(Ks, CT * KP, As, n, g, bb, Ts, CT * TP, TP, vec, vec_tmp);
  } else {
    // match the barriers inside factorize_chunk
    __syncthreads();
    __syncthreads();
  }
  __syncthreads();

  bf16x8 Sop[KSD][NTF];
#pragma unroll
  for (int s = 0; s < KSD; ++s) reg_operand<NTF>(S[2 * s], (2 * s + 1 < DT) ? S[2 * s + 1] : zero4(), Sop[s]);

  f32x4 R[2 * KST];
#pragma unroll
  for (int mt = 0; mt < 2 * KST; ++mt) {
    R[mt] = zero4();
    if (mt >= MT) continue;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 a[NTI];
      row_operand_terms<NTI, D>(Ks, CT * KP, KP, 16 * mt + col, s, grp, a);
      mma_terms<NTI, NTF, ORD>(acc, a, Sop[s]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * grp + r;
      float val = 0.f;
      if (t < n) val = vec[2 * CT + t] * (Vs[t * VP + my_row] - vec[CT + t] * acc[r]);
      R[mt][r] = val;
    }
  }
  bf16x8 Rop[KST][NTF];
#pragma unroll
  for (int s = 0; s < KST; ++s) reg_operand<NTF>(R[2 * s], R[2 * s + 1], Rop[s]);
  f32x4 Dt[2 * KST];
#pragma unroll
  for (int mt = 0; mt < 2 * KST; ++mt) {
    Dt[mt] = zero4();
    if (mt >= MT) continue;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s <= (mt >> 1); ++s) {
      bf16x8 a[NTF];
      row_operand_terms<NTF>(Ts, CT * TP, TP, 16 * mt + col, s, grp, a);
      mma_terms<NTF, NTF, ORD>(acc, a, Rop[s]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) Dt[mt][r] = vec[3 * CT + 16 * mt + 4 * grp + r] * acc[r];
  }
  bf16x8 Dtop[KST][NTF];
#pragma unroll
  for (int s = 0; s < KST; ++s) reg_operand<NTF>(Dt[2 * s], Dt[2 * s + 1], Dtop[s]);
  const float egn = vec[CT + n - 1];
#pragma unroll
  for (int jt = 0; jt < DT; ++jt) {
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = egn * S[jt][r];
#pragma unroll
    for (int s = 0; s < KST; ++s) {
      bf16x8 a[NTI];
      row_operand_terms<NTI>(KTs, D * TP, TP, 16 * jt + col, s, grp, a);
      mma_terms<NTI, NTF, ORD>(acc, a, Dtop[s]);
    }
    *reinterpret_cast<f32x4*>(state + (size_t)my_row * D + 16 * jt + 4 * grp) = acc;
  }
}

// ==================================================================================
// Launchers
template <typename IO, int D>
static hipError_t launch_factorize_t(const FactorizeArgs<IO>& a, int n_chunks, hipStream_t st) {
  if (n_chunks == 0) return hipSuccess;
  dim3 grid(n_chunks, a.Hv);
  hipLaunchKernelGGL((factorize_kernel<IO, D>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

template <typename IO, int D>
static hipError_t launch_scan_t(const ScanArgs<IO>& a, int n_seqs, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  constexpr int NW = ScanShape<D>::NW;
  dim3 grid(n_seqs, a.Hv, D / (16 * NW));
  hipLaunchKernelGGL((scan_kernel<IO, D>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <typename IO, int D>
static hipError_t launch_flush_t(const FlushArgs<IO>& a, int n_req, int ct, hipStream_t st) {
  if (n_req == 0) return hipSuccess;
  dim3 grid(n_req, a.Hv);
  if (ct <= 32)
    hipLaunchKernelGGL((flush_kernel<IO, D, 32>), grid, dim3(64 * (D / 16)), 0, st, a);
  else
    hipLaunchKernelGGL((flush_kernel<IO, D, 64>), grid, dim3(64 * (D / 16)), 0, st, a);
  return hipGetLastError();
}

#define GDN_DISPATCH_D(D_, CALL) \
  switch (D_) {                  \
    case 16: return CALL(16);    \
    case 32: return CALL(32);    \
    case 64: return CALL(64);    \
    case 128: return CALL(128);  \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_factorize(const FactorizeArgs<bf16_bits>& a, int D, int n_chunks, hipStream_t st) {
#define CALL(d) launch_factorize_t<bf16_bits, d>(a, n_chunks, st)
  GDN_DISPATCH_D(D, CALL)
#undef CALL
}
hipError_t launch_factorize(const FactorizeArgs<float>& a, int D, int n_chunks, hipStream_t st) {
#define CALL(d) launch_factorize_t<float, d>(a, n_chunks, st)
  switch (D) {
    case 16: return CALL(16);
    case 32: return CALL(32);
    case 64: return CALL(64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}
hipError_t launch_scan(const ScanArgs<bf16_bits>& a, int D, int n_seqs, hipStream_t st) {
#define CALL(d) launch_scan_t<bf16_bits, d>(a, n_seqs, st)
  GDN_DISPATCH_D(D, CALL)
#undef CALL
}
hipError_t launch_scan(const ScanArgs<float>& a, int D, int n_seqs, hipStream_t st) {
#define CALL(d) launch_scan_t<float, d>(a, n_seqs, st)
  switch (D) {
    case 16: return CALL(16);
    case 32: return CALL(32);
    case 64: return CALL(64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}
hipError_t launch_flush(const FlushArgs<bf16_bits>& a, int D, int n_req, int ct, hipStream_t st) {
#define CALL(d) launch_flush_t<bf16_bits, d>(a, n_req, ct, st)
  GDN_DISPATCH_D(D, CALL)
#undef CALL
}
hipError_t launch_flush(const FlushArgs<float>& a, int D, int n_req, int ct, hipStream_t st) {
#define CALL(d) launch_flush_t<float, d>(a, n_req, ct, st)
  switch (D) {
    case 16: return CALL(16);
    case 32: return CALL(32);
    case 64: return CALL(64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}

}  // namespace gdn
