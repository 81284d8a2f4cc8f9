// prefill_kernels.hip -- chunked varlen prefill of the gated delta rule on gfx950.
//
// Two kernels (the chunk algebra is stated in chunk_common.h):
//   factorize_kernel: for every (chunk, value head) at once, the state-free factors of
//     the chunk: the cumulative log decay g, T = (I + A)^-1 (the WY / UT transform of
//     the chunk), and the chunk's keys transposed.  T is written as ready-made MFMA A
//     operand fragments, K^T in the LDS image layout the scan copies by DMA.
//   scan_kernel: one workgroup per (sequence, value head, 64 value rows), one wave per
//     16-row slab of the state, walking the sequence's chunks in order with the slab in
//     registers.  Rows of the state are independent, so the slabs never exchange data.
//
// Chunks are cut at every multiple of 64 tokens, of the cache block and at the call
// ends (plan.cpp); when a chunk ends on a block boundary the scan stores the bits of
// the state into that boundary's checkpoint page, the state the next chunk starts
// from ("Prefix caching on Gated DeltaNet hybrids", "Why hits were wrong": a full block
// keeps the recurrent state after its last token), so a resume from the page computes
// exactly what the cold run computes after that point.
//
// Scan data flow per chunk (bf16 inputs, head dim 64 or 128): K, Q and K^T of chunk
// c + 1 are copied global -> LDS by LDS DMA (global_load_lds) into the second of two
// buffers while chunk c is computed; T fragments and this wave's V column come straight
// into registers one chunk ahead.  Two barriers per chunk: one after the DMA lands, one
// after the causal Q K^T tiles (shared by the four waves through LDS) are written.
#include <hip/hip_runtime.h>

#include "chunk_common.h"
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace gdn {

using namespace chunk;

namespace {

constexpr int CT = kChunk;

// The (row tile mt, k-step s) pairs of the 64 x 64 lower triangular T that the
// Delta = T R product reads (k-steps above the diagonal are all zero and skipped).
constexpr int kFragCombos = 6;
__host__ __device__ constexpr int frag_combo(int mt, int s) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + s; }

template <typename IO, int D>
struct PrefillCfg {
  static constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  static constexpr int KRB = 2 * phys_width(D);  // bytes per row of a K / Q plane
  static constexpr int KPL = CT * KRB / 2;         // elements per K / Q plane
  static constexpr int TRB = 2 * CT;               // bytes per row of a K^T / P plane
  static constexpr int KTPL = D * CT;              // elements per K^T plane
  static constexpr int PPL = CT * CT;              // elements per P plane
  // factor record: [T fragments][K^T planes][g, exp g, b, exp(g_n - g)]
  static constexpr int FRAG_BYTES = kFragCombos * NTF * 1024;
  static constexpr int KT_BYTES = NTI * KTPL * 2;
  static constexpr int VEC_OFF = FRAG_BYTES + KT_BYTES;
  static constexpr int REC_BYTES = VEC_OFF + 4 * CT * 4;
};

}  // namespace

static_assert(PrefillCfg<bf16_bits, 128>::REC_BYTES <= (int)factor_record_bytes_c(2, 1, 128), "record size");
static_assert(PrefillCfg<float, 64>::REC_BYTES <= (int)factor_record_bytes_c(3, 3, 64), "record size");

// ==================================================================================
// Pre-pass: one wave per (chunk, value head).
template <typename IO, int D>
__global__ __launch_bounds__(64) void factorize_kernel(FactorizeArgs<IO> p) {
  using Cfg = PrefillCfg<IO, D>;
  constexpr int NTI = Cfg::NTI, NTF = Cfg::NTF, ORD = Cfg::ORD;
  constexpr int KP = row_stride(D), TP = row_stride(CT);
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;
  __shared__ __attribute__((aligned(16))) bf16_bits Ks[NTI * CT * KP];
  __shared__ float As[CT][CT + 4];
  __shared__ __attribute__((aligned(16))) bf16_bits Tl[NTF * CT * TP];
  __shared__ float vec_lds[2 * CT];

  const int c = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int grp = lane >> 4, col = lane & 15;
  const ChunkDesc cd = p.chunks[c];
  const int n = cd.len;
  const int hk = h / p.group;
  if constexpr (D < 32) zero_lds(Ks, sizeof(Ks), lane, 64);
  __syncthreads();
  const IO* kb = p.k + cd.row * p.qk_stride + (int64_t)hk * D;
  for (int idx = lane; idx < CT * PER_ROW; idx += 64) {
    const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    uint4 v = load16(kb + (int64_t)t * p.qk_stride + j0, t < n);
    store_row_terms<IO, NTI>(v, Ks, CT * KP, KP, t, j0);
  }
  float la = 0.f, bb = 0.f;
  if (lane < n) {
    const int64_t ai = (cd.row + lane) * (int64_t)p.Hv + h;
    la = __logf(p.a[ai]);
    bb = p.b[ai];
  }
  const float g = wave_inclusive_scan(la);
  uint8_t* rec = p.factors + ((size_t)h * p.n_chunks + c) * p.factor_stride;
  float* vec_out = reinterpret_cast<float*>(rec + Cfg::VEC_OFF);
  factorize_chunk<CT, D, NTI, NTF, ORD>(Ks, CT * KP, As, n, g, bb, Tl, CT * TP, TP, vec_out, vec_lds);
  __syncthreads();

  // T as A-operand fragments: fragment (combo, term) holds lane l's 16 bytes at l * 16
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int s = 0; s <= (mt >> 1); ++s) {
#pragma unroll
      for (int i = 0; i < NTF; ++i) {
        const bf16x8 v = op_read(Tl + i * CT * TP, TP, 16 * mt + col, s, grp);
        *reinterpret_cast<bf16x8*>(rec + ((size_t)frag_combo(mt, s) * NTF + i) * 1024 + lane * 16) = v;
      }
    }
  }
  // K^T planes in the xor layout: row j, kappa-ordered columns t, 4 per 8-byte store
  bf16_bits* KTout = reinterpret_cast<bf16_bits*>(rec + Cfg::FRAG_BYTES);
  for (int task = lane; task < NTI * D * (CT / 4); task += 64) {
    const int i = task / (D * (CT / 4));
    const int rem = task % (D * (CT / 4));
    const int j = rem / (CT / 4), t0 = (rem % (CT / 4)) * 4;
    const bf16_bits* src = Ks + i * CT * KP + swz(j);
    const uint32_t w0 = (uint32_t)src[(t0 + 0) * KP] | ((uint32_t)src[(t0 + 1) * KP] << 16);
    const uint32_t w1 = (uint32_t)src[(t0 + 2) * KP] | ((uint32_t)src[(t0 + 3) * KP] << 16);
    *reinterpret_cast<uint2*>(KTout + i * Cfg::KTPL + xrun<Cfg::TRB>(j, swz(t0))) = uint2{w0, w1};
  }
}

// ==================================================================================
// Scan.
template <typename IO, int D>
__global__ __launch_bounds__(64 * ScanShape<D>::NW) void scan_kernel(ScanArgs<IO> p) {
  using Cfg = PrefillCfg<IO, D>;
  constexpr int NTI = Cfg::NTI, NTF = Cfg::NTF, ORD = Cfg::ORD;
  constexpr int NW = ScanShape<D>::NW, RW = 16 * NW, NTH = 64 * NW;
  constexpr int DT = D / 16, KSD = (D + 31) / 32;
  constexpr int KRB = Cfg::KRB, KPL = Cfg::KPL, TRB = Cfg::TRB, KTPL = Cfg::KTPL, PPL = Cfg::PPL;
  constexpr int ESZ = sizeof(IO);
  constexpr int VRB = RW * ESZ;          // bytes per row of the V slice (xor layout)
  constexpr int REC = Cfg::REC_BYTES;    // the factor record is copied whole
  // bf16 inputs with 128-byte or wider key rows: LDS DMA with double buffering
  constexpr bool DMA = ESZ == 2 && D >= 64;
  constexpr int NBUF = DMA ? 2 : 1;
  constexpr int VEC = 16 / ESZ;
  constexpr int PER_ROW = D / VEC, PER_VROW = RW / VEC;

  __shared__ __attribute__((aligned(16))) bf16_bits Kb[NBUF][NTI * KPL];
  __shared__ __attribute__((aligned(16))) bf16_bits Qb[NBUF][NTI * KPL];
  __shared__ __attribute__((aligned(16))) uint8_t Vb[NBUF][CT * VRB];
  __shared__ __attribute__((aligned(16))) uint8_t Rb[NBUF][REC];  // T fragments, K^T, vectors
  __shared__ __attribute__((aligned(16))) bf16_bits Ps[NTF * PPL];

  const int seq = blockIdx.x, h = blockIdx.y, rg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
  const int grp = lane >> 4, col = lane & 15;
  const int hk = h / p.group;
  const int i0 = rg * RW;               // first value row of the workgroup
  const ScanSeq sq = p.seqs[seq];
  const size_t head_off = (size_t)h * D * D;
  const int vcol = wave * 16 + col;     // this lane's column in the V slice
  const int my_row = i0 + vcol;         // value row held by this lane
  const int cb = sq.chunk_begin, ce = sq.chunk_end;

  if constexpr (D < 32) {
    // the kappa groups past a 16-wide key row are contracted: keep them zero
    zero_lds(Kb, sizeof(Kb), tid, NTH);
    zero_lds(Qb, sizeof(Qb), tid, NTH);
  }

  // ---- incoming state slab: lane holds S[my_row][16 jt + 4 grp + r]
  f32x4 S[DT];
#pragma unroll
  for (int jt = 0; jt < DT; ++jt) {
    if (sq.src)
      S[jt] = *reinterpret_cast<const f32x4*>(sq.src + head_off + (size_t)my_row * D + 16 * jt + 4 * grp);
    else
      S[jt] = zero4();
  }

  // ---- DMA source offsets (elements) of this lane, one per xor key its rows take
  constexpr int LPR = KRB / 4, RPI = 64 / LPR;          // key rows: lanes per row, rows per DMA
  constexpr int VLPR = VRB / 4, VRPI = 64 / VLPR;       // V rows
  // the xor key of a row repeats every 16 rows (xkey), so a wave striding NW * RPI rows
  // sees 16 / (NW * RPI) distinct keys
  constexpr int KCYC = DMA ? 16 / (NW * RPI) : 1;
  constexpr int VCYC = DMA ? 16 / (NW * VRPI) : 1;
  const int rsub = lane / LPR, vsub = lane / VLPR;
  uint32_t koff[KCYC], voff[VCYC];  // byte offsets from the row-group base
  if constexpr (DMA) {
    const int d = lane % LPR, vd = lane % VLPR;
#pragma unroll
    for (int k = 0; k < KCYC; ++k) {
      const int t = wave * RPI + k * NW * RPI + rsub;
      koff[k] = ESZ * (rsub * (uint32_t)p.qk_stride + unswz(8 * ((d >> 2) ^ xkey<KRB>(t)) + 2 * (d & 3)));
    }
#pragma unroll
    for (int k = 0; k < VCYC; ++k) {
      const int t = wave * VRPI + k * NW * VRPI + vsub;
      voff[k] = ESZ * (vsub * (uint32_t)p.v_stride + 8 * ((vd >> 2) ^ xkey<VRB>(t)) + 2 * (vd & 3));
    }
  }

  // ---- per-chunk operands staged in LDS: K, Q rows, the V slice, the factor record
  auto stage = [&](int c, int buf) {
    const ChunkDesc cd = uniform_chunk(p.chunks + c);
    const int n = cd.len;
    const IO* kb = p.k + cd.row * p.qk_stride + (int64_t)hk * D;
    const IO* qb = p.q + cd.row * p.qk_stride + (int64_t)hk * D;
    const IO* vb = p.v + cd.row * p.v_stride + (int64_t)h * D + i0;
    const uint8_t* rec = p.factors + ((size_t)h * p.n_chunks + c) * p.factor_stride;
    if constexpr (DMA) {
      // one dword DMA per key row (two V rows): the lane owning physical dword d of row t
      // reads the logical columns the xor / kappa layout places there.  The rows of one
      // wave cycle through KCYC (VCYC) xor keys, so the per-lane source offsets are
      // precomputed (koff, voff) and each DMA is a uniform row address plus that offset.
#pragma nounroll
      for (int k = 0; k < CT / (NW * RPI); ++k) {
        const int t0 = wave * RPI + k * NW * RPI;
        if (t0 >= n) break;
        if (t0 + RPI <= n || t0 + rsub < n) {
          const uint32_t off = koff[k % KCYC];
          lds_dma4(reinterpret_cast<const char*>(kb + (int64_t)t0 * p.qk_stride) + off, &Kb[buf][t0 * (KRB / 2)]);
          lds_dma4(reinterpret_cast<const char*>(qb + (int64_t)t0 * p.qk_stride) + off, &Qb[buf][t0 * (KRB / 2)]);
        }
      }
#pragma nounroll
      for (int k = 0; k < CT / (NW * VRPI); ++k) {
        const int t0 = wave * VRPI + k * NW * VRPI;
        if (t0 >= n) break;
        if (t0 + VRPI <= n || t0 + vsub < n)
          lds_dma4(reinterpret_cast<const char*>(vb + (int64_t)t0 * p.v_stride) + voff[k % VCYC], &Vb[buf][t0 * VRB]);
      }
#pragma nounroll
      for (int u = wave; u < REC / 1024; u += NW) lds_dma16(rec + u * 1024 + lane * 16, &Rb[buf][u * 1024]);
    } else {
      for (int idx = tid; idx < CT * PER_ROW; idx += NTH) {
        const int t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
        xstore_row_terms<IO, NTI, KRB>(load16(kb + (int64_t)t * p.qk_stride + j0, t < n), Kb[buf], KPL, t, j0);
        xstore_row_terms<IO, NTI, KRB>(load16(qb + (int64_t)t * p.qk_stride + j0, t < n), Qb[buf], KPL, t, j0);
      }
      for (int idx = tid; idx < CT * PER_VROW; idx += NTH) {
        const int t = idx / PER_VROW, pc = idx % PER_VROW;  // one 16-byte piece
        *reinterpret_cast<uint4*>(&Vb[buf][t * VRB + 16 * (pc ^ xkey<VRB>(t))]) =
            load16(vb + (int64_t)t * p.v_stride + pc * VEC, t < n);
      }
      for (int idx = tid; idx < REC / 16; idx += NTH)
        reinterpret_cast<uint4*>(Rb[buf])[idx] = reinterpret_cast<const uint4*>(rec)[idx];
    }
  };

  if constexpr (DMA) {
    if (cb < ce) stage(cb, 0);
  }

  for (int c = cb; c < ce; ++c) {
    const int buf = DMA ? ((c - cb) & 1) : 0;
    const ChunkDesc cd = uniform_chunk(p.chunks + c);
    const int n = cd.len;
    if constexpr (DMA) {
      full_barrier();  // chunk c's DMA has landed; every wave is done with chunk c - 1
      if (c + 1 < ce) stage(c + 1, buf ^ 1);
    } else {
      lds_barrier();   // every wave is done with chunk c - 1
      stage(c, 0);
      lds_barrier();
    }
    const bf16_bits* Ks = Kb[buf];
    const bf16_bits* Qs = Qb[buf];
    const uint8_t* Vs = Vb[buf];
    const bf16_bits* frag = reinterpret_cast<const bf16_bits*>(Rb[buf]);
    const bf16_bits* KTs = reinterpret_cast<const bf16_bits*>(Rb[buf] + Cfg::FRAG_BYTES);
    const float* vec = reinterpret_cast<const float*>(Rb[buf] + Cfg::VEC_OFF);

    // ---- P = mask o exp(g_t - g_s) (Q K^T), as P^T = K Q^T tiles (M = s, N = t): the
    //      C layout of a P^T tile is the A-operand layout of P.  Twelve tiles (the ten
    //      causal ones and the two upper ones the P Delta k-steps touch, all zero) are
    //      shared out over the waves and exchanged through LDS.
    {
      // tile it -> (ms, nt), two bits each: ms = 0,0,1,0,1,2,0,1,2,3,1,3  nt = 0,1,1,2,2,2,3,3,3,3,0,2
      constexpr int NPT = 12, TPW = (NPT + NW - 1) / NW;
      constexpr uint32_t MS_CODE = 0u | (0u << 2) | (1u << 4) | (0u << 6) | (1u << 8) | (2u << 10) | (0u << 12) |
                                   (1u << 14) | (2u << 16) | (3u << 18) | (1u << 20) | (3u << 22);
      constexpr uint32_t NT_CODE = 0u | (1u << 2) | (1u << 4) | (2u << 6) | (2u << 8) | (2u << 10) | (3u << 12) |
                                   (3u << 14) | (3u << 16) | (3u << 18) | (0u << 20) | (2u << 22);
      f32x4 pacc[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) pacc[u] = zero4();
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int it = wave + u * NW;
          const int ms = (MS_CODE >> (2 * it)) & 3, nt = (NT_CODE >> (2 * it)) & 3;
          if (it < NPT && ms <= nt) {
            bf16x8 a[NTI], b[NTI];
            xop_terms<KRB, NTI>(Ks, KPL, 16 * ms + col, s, grp, a);
            xop_terms<KRB, NTI>(Qs, KPL, 16 * nt + col, s, grp, b);
            mma_terms<NTI, NTI, ORD>(pacc[u], a, b);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int it = wave + u * NW;
        if (it < NPT) {
          const int ms = (MS_CODE >> (2 * it)) & 3, nt = (NT_CODE >> (2 * it)) & 3;
          const int t = 16 * nt + col;
          const float gt = vec[t];
          bf16_bits terms[4][NTF];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * ms + 4 * grp + r;
            float val = 0.f;
            if (s <= t && t < n) val = __expf(gt - vec[s]) * pacc[u][r];
            split_terms<NTF>(val, terms[r]);
          }
          const int off = xrun<TRB>(t, swz(16 * ms + 4 * grp));
#pragma unroll
          for (int i = 0; i < NTF; ++i)
            *reinterpret_cast<uint2*>(Ps + i * PPL + off) =
                uint2{(uint32_t)terms[0][i] | ((uint32_t)terms[1][i] << 16),
                      (uint32_t)terms[2][i] | ((uint32_t)terms[3][i] << 16)};
        }
      }
    }

    // ---- X = K S^T and Y = Q S^T together: eight independent accumulator chains; the
    //      state operand terms of each k-step are formed just before use
    phase_fence();
    f32x4 X[4], Y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) X[mt] = Y[mt] = zero4();
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 sop[NTF];
      reg_operand<NTF>(S[2 * s], (2 * s + 1 < DT) ? S[2 * s + 1] : zero4(), sop);
      bf16x8 ak[4][NTI], aq[4][NTI];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        xop_terms<KRB, NTI>(Ks, KPL, 16 * mt + col, s, grp, ak[mt]);
        xop_terms<KRB, NTI>(Qs, KPL, 16 * mt + col, s, grp, aq[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mma_terms<NTI, NTF, ORD>(X[mt], ak[mt], sop);
        mma_terms<NTI, NTF, ORD>(Y[mt], aq[mt], sop);
      }
      phase_fence();
    }

    // ---- R = b (V - exp(g) X), rows past n selected to zero
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * grp + r;
        const int vb = vcol * ESZ;
        const float vt = to_f32(*reinterpret_cast<const IO*>(Vs + t * VRB + 16 * ((vb >> 4) ^ xkey<VRB>(t)) + (vb & 15)));
        R[mt][r] = t < n ? vec[2 * CT + t] * (vt - vec[CT + t] * X[mt][r]) : 0.f;
      }
    bf16x8 Rop[2][NTF];
    reg_operand<NTF>(R[0], R[1], Rop[0]);
    reg_operand<NTF>(R[2], R[3], Rop[1]);
    phase_fence();

    // ---- Delta = T R  (T fragments from LDS; upper k-steps skipped)
    f32x4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Dl[mt] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 2 * s; mt < 4; ++mt) {
        bf16x8 a[NTF];
#pragma unroll
        for (int i = 0; i < NTF; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(frag + (frag_combo(mt, s) * NTF + i) * 512 + lane * 8);
        mma_terms<NTF, NTF, ORD>(Dl[mt], a, Rop[s]);
      }

    bf16x8 Dop[2][NTF];
    reg_operand<NTF>(Dl[0], Dl[1], Dop[0]);
    reg_operand<NTF>(Dl[2], Dl[3], Dop[1]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[mt][r] *= vec[CT + 16 * mt + 4 * grp + r];

    lds_barrier();  // P tiles from all waves are in LDS

    // ---- O = scale (exp(g) Q S^T + P Delta); stored before the state update so the
    //      stores drain while it runs
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 2 * s; mt < 4; ++mt) {
        bf16x8 a[NTF];
        xop_terms<TRB, NTF>(Ps, PPL, 16 * mt + col, s, grp, a);
        mma_terms<NTF, NTF, ORD>(Y[mt], a, Dop[s]);
      }
    {
      float* ob = p.o + (size_t)cd.row * p.Hv * D + (size_t)h * D + my_row;
      const size_t orow = (size_t)p.Hv * D;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * grp + r;
          if (t < n) ob[(size_t)t * orow] = p.scale * Y[mt][r];
        }
    }

    // ---- S^T <- exp(g_n) S^T + K^T (exp(g_n - g) o Delta): DT independent chains
    phase_fence();
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
      for (int jt = 0; jt < DT; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[jt][r] *= egn;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 a[DT][NTI];
#pragma unroll
        for (int jt = 0; jt < DT; ++jt) xop_terms<TRB, NTI>(KTs, KTPL, 16 * jt + col, s, grp, a[jt]);
#pragma unroll
        for (int jt = 0; jt < DT; ++jt) mma_terms<NTI, NTF, ORD>(S[jt], a[jt], Dtop[s]);
        phase_fence();
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

hipError_t launch_factorize(const FactorizeArgs<bf16_bits>& a, int D, int n_chunks, hipStream_t st) {
  switch (D) {
    case 16: return launch_factorize_t<bf16_bits, 16>(a, n_chunks, st);
    case 32: return launch_factorize_t<bf16_bits, 32>(a, n_chunks, st);
    case 64: return launch_factorize_t<bf16_bits, 64>(a, n_chunks, st);
    case 128: return launch_factorize_t<bf16_bits, 128>(a, n_chunks, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_factorize(const FactorizeArgs<float>& a, int D, int n_chunks, hipStream_t st) {
  switch (D) {
    case 16: return launch_factorize_t<float, 16>(a, n_chunks, st);
    case 32: return launch_factorize_t<float, 32>(a, n_chunks, st);
    case 64: return launch_factorize_t<float, 64>(a, n_chunks, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_scan(const ScanArgs<bf16_bits>& a, int D, int n_seqs, hipStream_t st) {
  switch (D) {
    case 16: return launch_scan_t<bf16_bits, 16>(a, n_seqs, st);
    case 32: return launch_scan_t<bf16_bits, 32>(a, n_seqs, st);
    case 64: return launch_scan_t<bf16_bits, 64>(a, n_seqs, st);
    case 128: return launch_scan_t<bf16_bits, 128>(a, n_seqs, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_scan(const ScanArgs<float>& a, int D, int n_seqs, hipStream_t st) {
  switch (D) {
    case 16: return launch_scan_t<float, 16>(a, n_seqs, st);
    case 32: return launch_scan_t<float, 32>(a, n_seqs, st);
    case 64: return launch_scan_t<float, 64>(a, n_seqs, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
