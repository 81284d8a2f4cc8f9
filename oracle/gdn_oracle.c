/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle for the Gated DeltaNet state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * cpu_baseline leg may load this library.  The GPU library never links it, and it
 * shares no code, header, table or helper with the GPU library.
 *
 * Every function is the definition written out, token by token, in fp64:
 *
 *   Recurrence (the gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta
 *   Networks: Improving Mamba2 with Delta Rule", ICLR 2025), per value head h with
 *   state S (d_v x d_k, row i = value channel, column j = key channel):
 *       S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *       o_t = scale * S_t q_t
 *   written out as the three steps below (decay, read the old value at k_t, write
 *   the correction), which is the same map expanded.
 *   The per-head fp32 state of 128 x 128 and the short conv window as the rest of
 *   the state follow "Prefix caching on Gated DeltaNet hybrids", section "Why hits
 *   were wrong", and "Hybrid linear attention (gated DeltaNet)", section "Why this
 *   family is different".
 *
 *   Checkpoints: a full block keeps the state after its last token ("Prefix caching
 *   on Gated DeltaNet hybrids", "Why hits were wrong"), so for absolute start
 *   position p0 and L tokens, the state is recorded after every token whose
 *   absolute end position is a positive multiple of `block`, the call end included.
 *
 *   Conv: a depthwise causal conv of width W over each channel, the last tap on the
 *   current token, optional SiLU, with the W-1 previous raw inputs carried as the
 *   conv part of the state.
 *
 *   Prefix accounting ("The cache block that is not a cache setting", "What that
 *   costs, exactly"): cached = (floor(shared/block) - 1) * block, never below 0.
 *
 * Parallelism: OpenMP over independent value heads (recurrence) or channels (conv);
 * each unit is computed by one thread in token order, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of absolute block boundaries p*block (p >= 1) in (p0, p0 + L]. */
int64_t gdn_oracle_count_boundaries(int64_t p0, int64_t L, int64_t block) {
  if (block <= 0 || L <= 0) return 0;
  return (p0 + L) / block - p0 / block;
}

/* One token of the gated delta rule on one head, in place on S (dv x dk, row-major).
 * If o != NULL, writes o[i] = scale * (S_t q)[i] with the updated state. */
static void delta_rule_token(double* S, int dk, int dv, const double* q, const double* k,
                             const double* v, double a, double b, double scale, double* o) {
  for (int i = 0; i < dv; ++i) {
    double* row = S + (size_t)i * dk;
    /* decay: S <- a S */
    for (int j = 0; j < dk; ++j) row[j] = a * row[j];
    /* value the decayed memory returns for key k: u_i = (a S_{t-1} k)_i */
    double u = 0.0;
    for (int j = 0; j < dk; ++j) u += row[j] * k[j];
    /* write: S <- S + b (v - u) k^T */
    double w = b * (v[i] - u);
    for (int j = 0; j < dk; ++j) row[j] += w * k[j];
    if (o) {
      double r = 0.0;
      for (int j = 0; j < dk; ++j) r += row[j] * q[j];
      o[i] = scale * r;
    }
  }
}

/*
 * Gated delta rule over L tokens of one sequence, all heads.
 *   q, k : [L][Hqk][dk]      v : [L][Hv][dv]      a, b : [L][Hv]
 *   S0   : [Hv][dv][dk] or NULL for a zero start state (never read when NULL)
 *   o    : [L][Hv][dv] or NULL (no outputs, e.g. a replay flush)
 *   S_out: [Hv][dv][dk] final state (may equal S0)
 *   ckpt : [n_ckpt][Hv][dv][dk] or NULL, n_ckpt = gdn_oracle_count_boundaries(p0, L, block)
 * Value head h reads query/key head h / (Hv / Hqk).
 * Returns 0, or -1 on bad shapes.
 */
int gdn_oracle_recurrence(int64_t L, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                          const double* q, const double* k, const double* v, const double* a,
                          const double* b, double scale, const double* S0, int64_t p0,
                          int64_t block, double* o, double* S_out, double* ckpt,
                          int32_t n_threads) {
  if (L < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0) return -1;
  const int group = Hv / Hqk;
  const size_t state_elems = (size_t)dv * dk;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < Hv; ++h) {
    const int hk = h / group;
    double* S = (double*)malloc(state_elems * sizeof(double));
    if (S0)
      memcpy(S, S0 + (size_t)h * state_elems, state_elems * sizeof(double));
    else
      memset(S, 0, state_elems * sizeof(double));
    int64_t next_ckpt = 0;
    for (int64_t t = 0; t < L; ++t) {
      const double* qt = q ? q + ((size_t)t * Hqk + hk) * dk : NULL;
      const double* kt = k + ((size_t)t * Hqk + hk) * dk;
      const double* vt = v + ((size_t)t * Hv + h) * dv;
      const double at = a[(size_t)t * Hv + h];
      const double bt = b[(size_t)t * Hv + h];
      double* ot = (o && qt) ? o + ((size_t)t * Hv + h) * dv : NULL;
      delta_rule_token(S, dk, dv, qt, kt, vt, at, bt, scale, ot);
      const int64_t pos_after = p0 + t + 1; /* absolute tokens consumed */
      if (block > 0 && pos_after % block == 0) {
        if (ckpt)
          memcpy(ckpt + ((size_t)next_ckpt * Hv + h) * state_elems, S,
                 state_elems * sizeof(double));
        ++next_ckpt;
      }
    }
    memcpy(S_out + (size_t)h * state_elems, S, state_elems * sizeof(double));
    free(S);
  }
  return 0;
}

/*
 * Depthwise causal conv of width W over L tokens of one sequence.
 *   x        : [L][C] raw inputs        w : [C][W], w[c][W-1] multiplies the current token
 *   tail_in  : [W-1][C] the W-1 raw inputs before the first token (oldest first),
 *              or NULL for zeros (never read when NULL)
 *   act      : 0 = none, 1 = SiLU (x * sigmoid(x)) applied to the conv sum
 *   y        : [L][C]
 *   tail_out : [W-1][C] the last W-1 raw inputs of the extended sequence
 *   ckpt_tails: [n_ckpt][W-1][C] or NULL: the W-1 raw inputs before each absolute
 *              block boundary in (p0, p0 + L]
 */
int gdn_oracle_conv(int64_t L, int32_t C, int32_t W, const double* x, const double* w,
                    const double* tail_in, int32_t act, int64_t p0, int64_t block, double* y,
                    double* tail_out, double* ckpt_tails, int32_t n_threads) {
  if (L < 0 || C <= 0 || W < 1) return -1;
  const int H = W - 1; /* history rows */
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(static)
  for (int c = 0; c < C; ++c) {
    /* extended sequence xe[i], i = -H .. L-1; xe[i] = tail_in[H + i] for i < 0 */
    double* xe = (double*)malloc((size_t)(L + H) * sizeof(double));
    for (int i = 0; i < H; ++i) xe[i] = tail_in ? tail_in[(size_t)i * C + c] : 0.0;
    for (int64_t t = 0; t < L; ++t) xe[H + t] = x[(size_t)t * C + c];
    for (int64_t t = 0; t < L; ++t) {
      double s = 0.0;
      for (int j = 0; j < W; ++j) s += w[(size_t)c * W + j] * xe[t + j]; /* xe index t+j = token t-H+j */
      if (act == 1) s = s / (1.0 + exp(-s));
      y[(size_t)t * C + c] = s;
    }
    for (int i = 0; i < H; ++i) tail_out[(size_t)i * C + c] = xe[L + i];
    if (ckpt_tails && block > 0) {
      int64_t n = 0;
      for (int64_t t = 0; t < L; ++t) {
        if ((p0 + t + 1) % block == 0) {
          /* rows before the boundary: tokens t-H+1 .. t, i.e. xe[t+1 .. t+H] */
          for (int i = 0; i < H; ++i)
            ckpt_tails[((size_t)n * H + i) * C + c] = xe[t + 1 + i];
          ++n;
        }
      }
    }
    free(xe);
  }
  return 0;
}

/* Prefix tokens served from cache for a shared prefix of `shared` tokens: whole blocks
 * only, the last full block left open, never below zero. */
int64_t gdn_oracle_cached_prefix_tokens(int64_t shared, int64_t block) {
  if (block <= 0 || shared <= 0) return 0;
  int64_t full = shared / block;
  return full >= 1 ? (full - 1) * block : 0;
}

/* A prefill chunk budget floored to a block boundary. */
int64_t gdn_oracle_floor_chunk(int64_t budget, int64_t block) {
  if (block <= 0 || budget <= 0) return budget > 0 ? budget : 0;
  return (budget / block) * block;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
