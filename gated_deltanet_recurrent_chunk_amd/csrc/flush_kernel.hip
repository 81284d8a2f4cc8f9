// flush_kernel.hip -- the ReplaySSM kernels ("Caching less to serve more requests",
// section "What we changed"): each request keeps one state plus a log of its per-token
// inputs since it.
//   flush:   folds the first n accepted rows of the log into the state as blocks of up
//            to 32 rows of the chunked gated delta rule (chunk_common.h), one launch for
//            all requests.  The state is read once and written once; rows at or past n
//            are never read.
//   replay:  the outputs of new rows appended behind the logged ones, computed from the
//            state and the log as one block of the same rule; nothing is written back.
#include <hip/hip_runtime.h>

#include "chunk_common.h"
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace gdn {

using namespace chunk;

// The gates' running log-decay of a block of nc rows: the DPP form for blocks of more
// than 16 rows, the LDS form for shorter ones (see short_req in the kernel).
__device__ __forceinline__ float flush_log_decay(float a, int nc) {
  const float la = (int)(threadIdx.x & 63) < nc ? __logf(a) : 0.f;
  return nc > 16 ? wave_inclusive_scan(la) : wave_inclusive_scan_lds(la);
}

// ==================================================================================
// Replay flush: one workgroup per (request, value head), one wave per 16-row slab of
// the state.  Reads the state once, applies the accepted rows 32 at a time as blocks of
// the chunked rule (each block factorized by wave 0, with waves 2 and 3 forming part of
// its A; the state carried in registers from block to block), writes the state once.
// The barriers order LDS only, so the state loads stay in flight through the staging of
// the first block and its factorization, and the next block's rows are requested while
// the current one is applied.
//
// One 32-row block covers the common case (a few accepted rows); its inverse is formed
// by 16-row blocks (two diagonal substitutions at once, then one off-diagonal block by
// two products), and with at most 16 rows only the first diagonal block is not the
// identity.  The kernel fits in 128 VGPRs, so two workgroups share a CU and the whole
// grid is resident at once.  (A 16-row block measured slower than this 32-row one, and a
// 64-row block, at 256 VGPRs and twice the LDS, ran in two rounds of workgroups.)  The
// state is read non-temporal and written through to device scope (store16_through).
//
// The state update reads its K^T operands from the key rows by transposing LDS reads,
// or, for requests of at most 16 rows, from a transposed copy (short_req below).
//
// Logs of more than 32 slots (TWO): a second block's factorization does not depend on
// the state, so its keys and gates are loaded with the first block's; wave 1 factorizes
// it into its own LDS while wave 0 factorizes the first.  Its values are requested once
// the first block's are staged and written, as bf16, to their own buffer before the
// barrier that ends the factorizations, so its products follow the first block's with
// no barrier between them.
template <typename IO, int D, bool TWO>
__global__ __launch_bounds__(64 * (D / 16), (sizeof(IO) == 2 && D >= 64) ? (TWO ? 2 : 4) : 1)
void flush_kernel(const int32_t* slot_ids, const int32_t* n_accepted, FlushArgs<IO> p) {
  constexpr int CT = 32;
  constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  constexpr int NW = D / 16, NTH = 64 * NW;
  constexpr int KP = row_stride(D), TP = row_stride(CT), VP = D + 4;
  constexpr int DT = D / 16, KSD = (D + 31) / 32;
  constexpr int MT = CT / 16, KST = (MT + 1) / 2;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;
  constexpr int PIECES = CT * PER_ROW, PER_THR = (PIECES + NTH - 1) / NTH;
  // TWO puts three roles on the waves: wave 0, wave 1 and the rest
  static_assert(!TWO || NW >= 3, "the two-block form needs head dim >= 64");
  // waves 2 and 3 form the second row tile of the first block's A while wave 0 forms the
  // first (measured: 17 rows 14.5 -> 13.7 us, 32 rows 14.5 -> 14.2 us)
  constexpr bool HELP = NW >= 4;
  // the same for the second block of TWO (waves 4 and 5)
  constexpr bool HELP2 = TWO && NW >= 6;

  __shared__ __attribute__((aligned(16))) bf16_bits Ks[NTI * CT * KP];
  // the first block's keys transposed (requests of at most 16 rows, see short_req)
  __shared__ __attribute__((aligned(16))) bf16_bits KTs[NTI * D * TP];
  __shared__ __attribute__((aligned(16))) float Vs[CT * VP];
  __shared__ __attribute__((aligned(16))) float As[CT][CT + 4];
  __shared__ __attribute__((aligned(16))) bf16_bits Ts[NTF * CT * TP];
  __shared__ __attribute__((aligned(16))) float vec[4 * CT];
  __shared__ float vec_tmp[2 * CT];
  // the second block's keys, factorization and gate vectors (TWO)
  constexpr int C2 = TWO ? CT : 1;
  __shared__ __attribute__((aligned(16))) bf16_bits Ks2[NTI * C2 * KP];
  // the second block's A, and its values (bf16 rows of V2P elements, padded so that rows
  // four apart fall in other banks)
  constexpr int V2P = D + 2;
  __shared__ __attribute__((aligned(16))) float As2buf[TWO ? CT * (CT + 4) : CT + 4];
  float(*const As2)[CT + 4] = reinterpret_cast<float(*)[CT + 4]>(As2buf);
  __shared__ __attribute__((aligned(16))) bf16_bits V2[TWO ? CT * V2P : 2];
  __shared__ __attribute__((aligned(16))) bf16_bits Ts2[NTF * C2 * TP];
  __shared__ __attribute__((aligned(16))) float vec2[4 * C2];
  __shared__ float vec_tmp2[2 * C2];

  // head-major grid: consecutive workgroups take consecutive heads of one request, so
  // they sweep that request's contiguous state block in address order
  const int h = blockIdx.x, r_ = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  // slot_ids and n_accepted (also in p) come first in the argument list: preloaded into
  // SGPRs at launch where the build asks for it; both words are fetched before either is
  // tested (one round trip, not two)
  int slot = slot_ids[r_];
  int n = n_accepted[r_];
  asm volatile("" : "+s"(slot), "+s"(n));
  const bool bad = (slot < -1) | (slot >= p.n_slots) | (n < 0) | (n > p.buf_rows);
  if (bad) {
    if (tid == 0 && h == 0 && p.status) atomicOr(p.status, 1 << GDN_ERR_CAPACITY);
    return;
  }
  if (slot < 0 || n == 0) return;  // padding or nothing accepted: untouched

  const int hk = h / p.group;
  const int my_row = wave * 16 + col;
  // Requests of at most 16 rows take two slower-looking steps before the factorization:
  // all waves copy the keys transposed (the state update reads K^T from that copy) and
  // the gates' prefix sum runs through LDS.  Longer requests read K^T from the key rows by
  // transposing reads and take the DPP prefix sum.  Measured both ways on both forms of
  // the kernel: the short forms made requests of at most 16 rows 0.3-1.1 us faster and
  // longer ones 0.2-0.8 us slower.  Per-workgroup timestamps show the difference in the
  // load and store phases, not in the changed steps: the first workgroups' state stores,
  // issued earlier, compete with the state reads of the rest.
  const bool short_req = n <= 16;
  float* state = p.state_pool + ((size_t)slot * p.Hv + h) * D * D;
  if constexpr (D < 32) zero_lds(Ks, sizeof(Ks), tid, NTH);  // padding columns, never written
  if constexpr (D < 32 && TWO) zero_lds(Ks2, sizeof(Ks2), tid, NTH);

  // rows c0 .. c0 + nc - 1 of the slot's log: the gates (wave 0) first, since the
  // factorization waits for them, then keys and values
  const size_t row0 = (size_t)slot * p.buf_rows;
  const IO* kb = p.buf_k + row0 * p.Hqk * D + (size_t)hk * D;
  const IO* vb = p.buf_v + row0 * p.Hv * D + (size_t)h * D;
  float a_row = 0.f, bb = 0.f;
  uint4 kv[PER_THR], vv[PER_THR];
  auto load_rows = [&](int c0, int nc) {
    a_row = 0.f;
    bb = 0.f;
    if (wave == 0 && lane < nc) {
      const size_t ai = (row0 + c0 + lane) * p.Hv + h;
      a_row = p.buf_a[ai];
      bb = p.buf_b[ai];
    }
#pragma unroll
    for (int i = 0; i < PER_THR; ++i) {
      const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
      kv[i] = load16(kb + (size_t)(c0 + t) * p.Hqk * D + j0, idx < PIECES && t < nc);
      vv[i] = load16(vb + (size_t)(c0 + t) * p.Hv * D + j0, idx < PIECES && t < nc);
    }
  };
  load_rows(0, n < CT ? n : CT);
  // TWO: the second block's keys (all waves) and gates (wave 1), with the first block's
  const int n2 = TWO && n > CT ? n - CT : 0;
  uint4 kv2[TWO ? PER_THR : 1];
  float a2_row = 0.f, b2 = 0.f;
  if constexpr (TWO) {
    if (n2 > 0) {
    if (wave == 1 && lane < n2) {
      const size_t ai = (row0 + CT + lane) * p.Hv + h;
      a2_row = p.buf_a[ai];
      b2 = p.buf_b[ai];
    }
#pragma unroll
    for (int i = 0; i < PER_THR; ++i) {
      const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
      kv2[i] = load16(kb + (size_t)(CT + t) * p.Hqk * D + j0, idx < PIECES && t < n2);
    }
    }
  }
  auto load_values = [&](int c0, int nc) {
#pragma unroll
    for (int i = 0; i < PER_THR; ++i) {
      const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
      vv[i] = load16(vb + (size_t)(c0 + t) * p.Hv * D + j0, idx < PIECES && t < nc);
    }
  };
  // then the state: loads complete in issue order, so waiting for the rows (to stage
  // them) leaves the state loads in flight until the products need them
  f32x4 S[DT];
#pragma unroll
  for (int jt = 0; jt < DT; ++jt)
    S[jt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(state + (size_t)my_row * D + 16 * jt + 4 * grp));

  // A operand of K^T (state tile jt, k-step s over the block's rows) from a key-row plane,
  // by transposing LDS reads: in each 16-lane group, ds_read_b64_tr_b16 gives lane i, as
  // its element e, the 16-bit value at lane 4 e + i / 4's address plus i % 4 elements.
  // Lane 4 e + c of group grp names row 32 s + 16 h + 4 grp + e (read h = 0, 1) at the
  // run of four key columns 16 jt + 4 c (contiguous in the swizzled order), so lane
  // (col, grp) receives K[32 s + 16 h + 4 grp + e][16 jt + col]: elements 4 h + e of the
  // operand under the contraction order kappa.
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));
  typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
  auto kt_operand = [&](const bf16_bits* plane, int jt, int s) {
    const int e = (lane >> 2) & 3, c4 = lane & 3;
    u32x2_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_bits* a = plane + (32 * s + 16 * h + 4 * grp + e) * KP + swz(16 * jt + 4 * c4);
      w[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (__attribute__((address_space(3))) v4s*)a));
    }
    return __builtin_bit_cast(bf16x8, u32x4_t{w[0][0], w[0][1], w[1][0], w[1][1]});
  };

  // one block of rows c0 .. c0 + nc - 1; written out twice below rather than as a loop,
  // which would hoist every LDS address of the products out of it and hold them all in
  // registers
  auto apply_block = [&](const int c0, const int nc, auto pre_) {
    // PRE: the second block of TWO, factorized with the first; its keys are in Ks2
    constexpr bool PRE = decltype(pre_)::value;
    const bf16_bits* Kb = PRE ? Ks2 : Ks;
    const bf16_bits* Tb = PRE ? Ts2 : Ts;
    const float* vb_ = PRE ? vec2 : vec;
    // the previous block's readers are done with the LDS (first block: the zero fill,
    // d < 32, precedes the row stores).  PRE reads only what the first block's barrier
    // after the factorizations published (its keys, factors, gate vectors and values),
    // and nothing the first block's products write: no barrier.
    if constexpr (!PRE) lds_barrier();
    if constexpr (!PRE) {
#pragma unroll
      for (int i = 0; i < PER_THR; ++i) {
        const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
        if (idx < PIECES) {
          store_row_terms<IO, NTI>(kv[i], Ks, CT * KP, KP, t, j0);
          if constexpr (TWO) {
            if (n2 > 0) store_row_terms<IO, NTI>(kv2[i], Ks2, CT * KP, KP, t, j0);
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) Vs[t * VP + j0 + e] = elem<IO>(vv[i], e);
        }
      }
      const float a_cur = a_row, b_cur = bb;
      // TWO: the second block's values, into the registers just staged from
      if constexpr (TWO) {
        if (n2 > 0) load_values(CT, n2);
      }
      lds_barrier();
      if (short_req) transpose_keys<CT, D, NTI>(Ks, KP, KTs, D * TP, TP, tid, NTH);
      if (wave == 0) {
        const float g = flush_log_decay(a_cur, nc);
        factorize_chunk<CT, D, NTI, NTF, ORD, false, HELP>(Ks, CT * KP, As, nc, g, b_cur, Ts, CT * TP, TP,
                                                                   vec, vec_tmp);
      } else if (TWO && wave == 1 && n2 > 0) {
        // the second block, at the same time (its prefix sum in DPP moves at any length:
        // every wave waits for it at the first barrier)
        const float g = wave_inclusive_scan(lane < n2 ? __logf(a2_row) : 0.f);
        factorize_chunk<CT, D, NTI, NTF, ORD, false, HELP2>(Ks2, CT * KP, As2, n2, g, b2, Ts2, CT * TP, TP, vec2,
                                                               vec_tmp2);
      } else {
        // match the barriers inside factorize_chunk; in between, waves 2 and 3 form the
        // tiles (1, 0) and (1, 1) of the first block's A (more than 16 rows), and waves 4
        // and 5 those of the second block's (TWO, more than 16 rows there)
        lds_barrier();
        if (HELP && nc > 16 && (wave == 2 || wave == 3))
          form_a_tile<CT, D, NTI, ORD>(Ks, CT * KP, As, nc, 1, wave - 2, vec_tmp);
        if (HELP2 && n2 > 16 && (wave == 4 || wave == 5))
          form_a_tile<CT, D, NTI, ORD>(Ks2, CT * KP, As2, n2, 1, wave - 4, vec_tmp2);
        lds_barrier();
      }
      if constexpr (TWO) {
        // the second block's values (requested with the first block's staging), published
        // by the barrier below
        if (n2 > 0) {
#pragma unroll
          for (int i = 0; i < PER_THR; ++i) {
            const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
            if (idx < PIECES) {
              const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(V2 + t * V2P + j0 + 2 * e) = w[e];
            }
          }
        }
      }
      lds_barrier();
      if constexpr (!TWO) {
        // the next block's rows (n <= 2 CT), requested after the factorization, whose
        // registers they would otherwise add to, and in flight during the products
        if (c0 + CT < n) load_rows(c0 + CT, n - c0 - CT);
      }
    }

    // X = K S^T, R = b (V - e^g X), Dt = e^(g_n - g) T R, S^T <- e^(g_n) S^T + K^T Dt
    bf16x8 Sop[KSD][NTF];
#pragma unroll
    for (int s = 0; s < KSD; ++s) reg_operand<NTF>(S[2 * s], (2 * s + 1 < DT) ? S[2 * s + 1] : zero4(), Sop[s]);
    f32x4 R[2 * KST];
#pragma unroll
    for (int mt = 0; mt < 2 * KST; ++mt) {
      R[mt] = zero4();
      if (mt >= MT || 16 * mt >= nc) continue;  // rows t >= nc: R = 0
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        bf16x8 a[NTI];
        op_terms<NTI>(Kb, CT * KP, KP, 16 * mt + col, s, grp, a);
        mma_terms<NTI, NTF, ORD>(acc, a, Sop[s]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * grp + r;
        float val = 0.f;
        if (t < nc) {
          const float vt = PRE ? bf16_to_f32(V2[t * V2P + my_row]) : Vs[t * VP + my_row];
          val = vb_[2 * CT + t] * (vt - vb_[CT + t] * acc[r]);
        }
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
      if (mt >= MT || 16 * mt >= nc) continue;  // rows t >= nc: identity rows of T, R = 0
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {
        bf16x8 a[NTF];
        op_terms<NTF>(Tb, CT * TP, TP, 16 * mt + col, s, grp, a);
        mma_terms<NTF, NTF, ORD>(acc, a, Rop[s]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Dt[mt][r] = vb_[3 * CT + 16 * mt + 4 * grp + r] * acc[r];
    }
    bf16x8 Dtop[KST][NTF];
#pragma unroll
    for (int s = 0; s < KST; ++s) reg_operand<NTF>(Dt[2 * s], Dt[2 * s + 1], Dtop[s]);
    const float egn = vb_[CT + nc - 1];
#pragma unroll
    for (int jt = 0; jt < DT; ++jt) {
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = egn * S[jt][r];
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        bf16x8 a[NTI];
        if (!PRE && short_req) {
          op_terms<NTI>(KTs, D * TP, TP, 16 * jt + col, s, grp, a);
        } else {
#pragma unroll
          for (int i = 0; i < NTI; ++i) a[i] = kt_operand(Kb + i * CT * KP, jt, s);
        }
        mma_terms<NTI, NTF, ORD>(acc, a, Dtop[s]);
      }
      S[jt] = acc;
    }
  };
  static_assert(kMaxBufRows <= 2 * CT, "a log holds at most two blocks");
  apply_block(0, n < CT ? n : CT, std::false_type{});
  if (n > CT) apply_block(CT, n - CT, std::integral_constant<bool, TWO>{});
#pragma unroll
  for (int jt = 0; jt < DT; ++jt) store16_through(state + (size_t)my_row * D + 16 * jt + 4 * grp, S[jt]);
}

// ==================================================================================
// Replay outputs: one workgroup per (request, value head), one wave per 16-row slab of
// the state.  With L = m + n rows (m logged, n new), S_0 the slot's state, g the running
// log-decay and T = (I + A)^-1 from the rows' keys and gates (wave 0), the block form of
// the rule gives
//   Delta = T diag(b) (V - diag(e^g) K S_0^T)            (the rows' corrected updates)
//   O     = scale (diag(e^g) Q S_0^T + P Delta),  P[t][s] = e^(g_t - g_s) q_t.k_s, s <= t
// whose row t is scale * S_t q_t, the output after row t.  Rows t < m carry no query:
// their outputs are zero and not stored.
template <typename IO, int D, int CT>
__global__ __launch_bounds__(64 * (D / 16)) void replay_kernel(ReplayArgs<IO> p) {
  constexpr int NTI = Prec<IO>::NTI, NTF = Prec<IO>::NTF, ORD = Prec<IO>::ORD;
  constexpr int NW = D / 16, NTH = 64 * NW;
  constexpr int KP = row_stride(D), TP = row_stride(CT), VP = D + 4;
  constexpr int DT = D / 16, KSD = (D + 31) / 32;
  constexpr int MT = CT / 16, KST = (MT + 1) / 2;
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int PER_ROW = D / VEC;
  // P tiles formed: (mt, nt) with nt <= mt | 1, which covers every tile the output
  // products read (tiles above the diagonal come out zero)
  constexpr int NPT = MT == 4 ? 12 : MT == 2 ? 4 : 1;

  __shared__ __attribute__((aligned(16))) bf16_bits Ks[NTI * CT * KP];
  __shared__ __attribute__((aligned(16))) bf16_bits Qs[NTI * CT * KP];
  __shared__ __attribute__((aligned(16))) float Vs[CT * VP];
  __shared__ __attribute__((aligned(16))) float As[CT][CT + 4];
  __shared__ __attribute__((aligned(16))) bf16_bits Ts[NTF * CT * TP];
  __shared__ __attribute__((aligned(16))) bf16_bits Ps[NTF * CT * TP];
  __shared__ __attribute__((aligned(16))) float vec[4 * CT];
  __shared__ float vec_tmp[2 * CT];

  // head-major grid, as for the flush
  const int h = blockIdx.x, r_ = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;
  // the three words are fetched before any is tested (one round trip)
  int slot = p.slot_ids[r_];
  int m = p.n_logged[r_], n = p.n_new[r_];
  asm volatile("" : "+s"(slot), "+s"(m), "+s"(n));
  const bool bad = (slot < -1) | (slot >= p.n_slots) | (m < 0) | (n < 0) | (m + n > p.buf_rows) | (n > p.max_new);
  if (bad) {
    if (tid == 0 && h == 0 && p.status) atomicOr(p.status, 1 << GDN_ERR_CAPACITY);
    return;
  }
  if (slot < 0 || n == 0) return;  // padding or no new rows: nothing written
  const int L = m + n;

  const int hk = h / p.group;
  const int my_row = wave * 16 + col;
  const float* state = p.state_pool + ((size_t)slot * p.Hv + h) * D * D;
  if constexpr (D < 32) {
    zero_lds(Ks, sizeof(Ks), tid, NTH);
    zero_lds(Qs, sizeof(Qs), tid, NTH);
  }

  // log rows 0 .. L-1 of this slot (keys, values) and the queries of the new rows; the
  // state is requested only once the factorization no longer waits for this wave (see
  // below)
  constexpr int PIECES = CT * PER_ROW, PER_THR = (PIECES + NTH - 1) / NTH;
  const size_t row0 = (size_t)slot * p.buf_rows;
  // the rows' gates (wave 0) go first: the factorization waits for them
  float a_row = 0.f, bb = 0.f;
  if (wave == 0 && lane < L) {
    const size_t ai = (row0 + lane) * p.Hv + h;
    a_row = p.buf_a[ai];
    bb = p.buf_b[ai];
  }
  const IO* kb = p.buf_k + row0 * p.Hqk * D + (size_t)hk * D;
  const IO* vb = p.buf_v + row0 * p.Hv * D + (size_t)h * D;
  const IO* qb = p.q_new + (size_t)r_ * p.max_new * p.Hqk * D + (size_t)hk * D;
  uint4 kv[PER_THR], qv[PER_THR], vv[PER_THR];
#pragma unroll
  for (int i = 0; i < PER_THR; ++i) {
    const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    const bool in = idx < PIECES;
    kv[i] = load16(kb + (size_t)t * p.Hqk * D + j0, in && t < L);
    qv[i] = load16(qb + (size_t)(t >= m ? t - m : 0) * p.Hqk * D + j0, in && t >= m && t < L);
    vv[i] = load16(vb + (size_t)t * p.Hv * D + j0, in && t < L);
  }
  f32x4 S[DT];
  lds_barrier();  // the zero fills (d < 32) precede the row stores
#pragma unroll
  for (int i = 0; i < PER_THR; ++i) {
    const int idx = tid + NTH * i, t = idx / PER_ROW, j0 = (idx % PER_ROW) * VEC;
    if (idx < PIECES) {
      store_row_terms<IO, NTI>(kv[i], Ks, CT * KP, KP, t, j0);
      store_row_terms<IO, NTI>(qv[i], Qs, CT * KP, KP, t, j0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) Vs[t * VP + j0 + e] = elem<IO>(vv[i], e);
    }
  }
  lds_barrier();
  // P tiles, as NTF bf16 term planes (row t, column s): they need the gates only, so the
  // waves other than wave 0 form them while wave 0 factorizes (between the barrier that
  // publishes the gate vectors and the next one); with one wave, after the factorization
  auto p_tiles = [&](int first, int step) {
  for (int ti = first; ti < NPT; ti += step) {
    const int mt = MT == 4 ? (ti < 2 ? 0 : ti < 4 ? 1 : ti < 8 ? 2 : 3) : MT == 2 ? ti >> 1 : 0;
    const int nt = MT == 4 ? (ti < 4 ? ti & 1 : (ti - 4) & 3) : MT == 2 ? ti & 1 : 0;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 a[NTI], b[NTI];
      op_terms<NTI>(Qs, CT * KP, KP, 16 * mt + col, s, grp, a);
      op_terms<NTI>(Ks, CT * KP, KP, 16 * nt + col, s, grp, b);
      mma_terms<NTI, NTI, ORD>(acc, a, b);
    }
    const int sc = 16 * nt + col;
    const float gs = vec[sc];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * grp + r;
      // the exponent g_t - g_s is <= 0 on the causal side kept by the select
      float dec = __expf(vec[t] - gs);
      asm volatile("" : "+v"(dec));
      const float val = (sc <= t && t < L) ? dec * acc[r] : 0.f;
      bf16_bits tt[NTF];
      split_terms<NTF>(val, tt);
#pragma unroll
      for (int q = 0; q < NTF; ++q) Ps[q * CT * TP + t * TP + swz(sc)] = tt[q];
    }
  }
  };
  // The state (64 KiB per workgroup at d = 128) is requested by each wave once its part
  // of the factorization is done: wave 0 after the factorization, the others after
  // their P tiles.  Requested at the start instead, the second workgroup of a CU waited
  // for its rows and its waves stalled issuing loads while the first workgroup's state
  // streamed in (measured: 14.6 us, the second workgroups finishing ~4 us after the
  // first; 11.6 us with the requests placed here and the factorization's wave-local
  // second barrier).
  auto load_state = [&]() {
#pragma unroll
    for (int jt = 0; jt < DT; ++jt)
      S[jt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(state + (size_t)my_row * D + 16 * jt + 4 * grp));
  };
  if (wave == 0) {
    const float g = wave_inclusive_scan(lane < L ? __logf(a_row) : 0.f);
    factorize_chunk<CT, D, NTI, NTF, ORD, true>(Ks, CT * KP, As, L, g, bb, Ts, CT * TP, TP, vec,
                                                                  vec_tmp);
    if constexpr (NW == 1) {
      lds_barrier();
      p_tiles(0, 1);
    }
    load_state();
  } else {
    // match the barrier inside factorize_chunk that publishes the gate vectors
    lds_barrier();
    p_tiles(wave - 1, NW - 1);
    load_state();
  }
  lds_barrier();

  // X = K S_0^T and Y = Q S_0^T for this wave's slab
  bf16x8 Sop[KSD][NTF];
#pragma unroll
  for (int s = 0; s < KSD; ++s) reg_operand<NTF>(S[2 * s], (2 * s + 1 < DT) ? S[2 * s + 1] : zero4(), Sop[s]);
  f32x4 R[2 * KST], Y[2 * KST];
#pragma unroll
  for (int mt = 0; mt < 2 * KST; ++mt) {
    R[mt] = zero4();
    Y[mt] = zero4();
    if (mt >= MT) continue;
    f32x4 acc = zero4(), accy = zero4();
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      bf16x8 a[NTI], aq[NTI];
      op_terms<NTI>(Ks, CT * KP, KP, 16 * mt + col, s, grp, a);
      op_terms<NTI>(Qs, CT * KP, KP, 16 * mt + col, s, grp, aq);
      mma_terms<NTI, NTF, ORD>(acc, a, Sop[s]);
      mma_terms<NTI, NTF, ORD>(accy, aq, Sop[s]);
    }
    Y[mt] = accy;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * grp + r;
      float val = 0.f;
      if (t < L) val = vec[2 * CT + t] * (Vs[t * VP + my_row] - vec[CT + t] * acc[r]);
      R[mt][r] = val;
    }
  }
  // Delta = T R
  bf16x8 Rop[KST][NTF];
#pragma unroll
  for (int s = 0; s < KST; ++s) reg_operand<NTF>(R[2 * s], R[2 * s + 1], Rop[s]);
  f32x4 Dl[2 * KST];
#pragma unroll
  for (int mt = 0; mt < 2 * KST; ++mt) {
    Dl[mt] = zero4();
    if (mt >= MT) continue;
#pragma unroll
    for (int s = 0; s <= (mt >> 1); ++s) {
      bf16x8 a[NTF];
      op_terms<NTF>(Ts, CT * TP, TP, 16 * mt + col, s, grp, a);
      mma_terms<NTF, NTF, ORD>(Dl[mt], a, Rop[s]);
    }
  }
  // O = scale (e^g Y + P Delta); rows m .. L-1 stored
  bf16x8 Dop[KST][NTF];
#pragma unroll
  for (int s = 0; s < KST; ++s) reg_operand<NTF>(Dl[2 * s], Dl[2 * s + 1], Dop[s]);
  float* ob = p.o + (size_t)r_ * p.max_new * p.Hv * D + (size_t)h * D + my_row;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = vec[CT + 16 * mt + 4 * grp + r] * Y[mt][r];
#pragma unroll
    for (int s = 0; s <= (mt >> 1); ++s) {
      bf16x8 a[NTF];
      op_terms<NTF>(Ps, CT * TP, TP, 16 * mt + col, s, grp, a);
      mma_terms<NTF, NTF, ORD>(acc, a, Dop[s]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * grp + r;
      if (t >= m && t < L) ob[(size_t)(t - m) * p.Hv * D] = p.scale * acc[r];
    }
  }
}

template <typename IO, int D>
static hipError_t launch_replay_t(const ReplayArgs<IO>& a, int n_req, int ct, hipStream_t st) {
  if (n_req == 0) return hipSuccess;
  dim3 grid(a.Hv, n_req);
  if (ct <= 32) {
    hipLaunchKernelGGL((replay_kernel<IO, D, 32>), grid, dim3(64 * (D / 16)), 0, st, a);
  } else {
    // a 64-row block of fp32 rows at head dim 128 does not fit a CU's LDS (refused by
    // gdn_replay_forward before the launch)
    if constexpr (sizeof(IO) == 4 && D >= 128) return hipErrorInvalidValue;
    else hipLaunchKernelGGL((replay_kernel<IO, D, 64>), grid, dim3(64 * (D / 16)), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs<bf16_bits>& a, int D, int n_req, int ct, hipStream_t st) {
  switch (D) {
    case 16: return launch_replay_t<bf16_bits, 16>(a, n_req, ct, st);
    case 32: return launch_replay_t<bf16_bits, 32>(a, n_req, ct, st);
    case 64: return launch_replay_t<bf16_bits, 64>(a, n_req, ct, st);
    case 128: return launch_replay_t<bf16_bits, 128>(a, n_req, ct, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_replay(const ReplayArgs<float>& a, int D, int n_req, int ct, hipStream_t st) {
  switch (D) {
    case 16: return launch_replay_t<float, 16>(a, n_req, ct, st);
    case 32: return launch_replay_t<float, 32>(a, n_req, ct, st);
    case 64: return launch_replay_t<float, 64>(a, n_req, ct, st);
    case 128: return launch_replay_t<float, 128>(a, n_req, ct, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename IO, int D>
static hipError_t launch_flush_t(const FlushArgs<IO>& a, int n_req, hipStream_t st) {
  if (n_req == 0) return hipSuccess;
  dim3 grid(a.Hv, n_req);
  // a log of more than one 32-row block takes the form that factorizes both at once
  // (head dim >= 64: it needs three waves; bf16: two such workgroups still share a CU)
  if constexpr (D >= 64 && sizeof(IO) == 2) {
    if (a.buf_rows > 32) {
      hipLaunchKernelGGL((flush_kernel<IO, D, true>), grid, dim3(64 * (D / 16)), 0, st, a.slot_ids, a.n_accepted,
                         a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((flush_kernel<IO, D, false>), grid, dim3(64 * (D / 16)), 0, st, a.slot_ids, a.n_accepted, a);
  return hipGetLastError();
}

hipError_t launch_flush(const FlushArgs<bf16_bits>& a, int D, int n_req, hipStream_t st) {
  switch (D) {
    case 16: return launch_flush_t<bf16_bits, 16>(a, n_req, st);
    case 32: return launch_flush_t<bf16_bits, 32>(a, n_req, st);
    case 64: return launch_flush_t<bf16_bits, 64>(a, n_req, st);
    case 128: return launch_flush_t<bf16_bits, 128>(a, n_req, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_flush(const FlushArgs<float>& a, int D, int n_req, hipStream_t st) {
  switch (D) {
    case 16: return launch_flush_t<float, 16>(a, n_req, st);
    case 32: return launch_flush_t<float, 32>(a, n_req, st);
    case 64: return launch_flush_t<float, 64>(a, n_req, st);
    case 128: return launch_flush_t<float, 128>(a, n_req, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
