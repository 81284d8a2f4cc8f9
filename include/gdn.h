/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet recurrent-state update for AMD MI355X (gfx950).
 *
 * The operation.  Per value head, a state S of d x d fp32 (row i = value channel,
 * column j = key channel) follows the gated delta rule (Yang, Kautz & Hatamizadeh,
 * "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025):
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = scale * S_t q_t
 *
 * with a_t in (0, 1] (the decay gate) and b_t in [0, 1] (the write strength).  A
 * layer holds one such state per value head plus a short causal conv window over
 * the packed q|k|v channels.  The state shape (48 heads x 128 x 128 fp32 per layer
 * on the 27B models, 32 heads on the 4B ones) and the conv window being part of the
 * state come from "Prefix caching on Gated DeltaNet hybrids" (section "Why hits were
 * wrong") and "Hybrid linear attention (gated DeltaNet)" (section "Why this family is
 * different").
 *
 * Conventions for every call:
 *   - Pointers marked [host] are host memory read before the call returns; all other
 *     pointers are device memory of the current HIP device, except a gdn_staging
 *     buffer (pinned host memory, below).  The caller owns all memory; libgdn allocates
 *     and frees nothing and keeps no state between calls, so calls on different streams
 *     never wait for one another.  (gdn_chunk_prefill_noalloc is the one exception: it
 *     keeps its scratch array's device address, once per device.)
 *   - A call's small tables (one entry per sequence, one page id per crossed block
 *     boundary) travel in the kernel arguments when the batch has at most
 *     GDN_INLINE_SEQS sequences and GDN_INLINE_PAGES boundaries.  Past that, the call
 *     writes them into the caller's gdn_staging buffer and copies them from there into
 *     its workspace on `stream`; the caller must leave that buffer untouched until the
 *     stream has passed the call (as for any asynchronous copy from host memory), and
 *     gdn_*_staging_bytes gives the size (0 when none is needed).
 *   - Work is enqueued on `stream` and runs asynchronously.  Argument validation is
 *     synchronous and happens before anything is enqueued: on any error the call
 *     returns a non-zero gdn_status, enqueues nothing and modifies no memory (fail
 *     closed, as "Prefix caching on Gated DeltaNet hybrids", section "The in-page
 *     layout", requires of a partial-block copy or an off-boundary resume).
 *   - Token-major packed layouts: q, k are [tokens][n_qk_heads][d]; v and o are
 *     [tokens][n_v_heads][d]; a, b are [tokens][n_v_heads] fp32.  Value head h reads
 *     query/key head h / (n_v_heads / n_qk_heads).
 *   - A state is fp32 [n_v_heads][d][d], row-major (value channel major).
 *   - Masked or unused rows are excluded by selection, never by multiplying with a
 *     mask, so NaN bit patterns in rows a call must not read cannot reach a result
 *     ("Prefix caching on Gated DeltaNet hybrids", "The in-page layout", defect 1).
 *   - Domain.  The results hold the stated accuracy (relative L2 1e-3 with bf16 inputs,
 *     1e-5 with fp32 inputs) for a_t in (0, 1] and b_t in [0, 1] with b_t |k_t|^2 <= 2:
 *     the range in which the update S (I - b k k^T) does not grow the state (unit keys,
 *     as the packed core's post-conv step makes them, are always in it).  Outside it
 *     the state grows geometrically and so do fp32 rounding errors.  A state decayed
 *     below 2^-126 (the smallest normal fp32, e.g. by a = 2^-126) is held as an fp32
 *     subnormal or zero, without relative precision.
 *
 * Determinism.  For one sequence, given its inputs, its start position, the bits of
 * its state source and the layer descriptor, every output, checkpoint and final state
 * is bit-identical whatever the other sequences of the call are, however many there
 * are and in which order, and however the sequence is split across calls, provided
 * each split falls on a multiple of 64 tokens or of the block.  This is what makes a
 * resume from a checkpoint equal a cold run ("The prefix cache changed the answer",
 * section "The fix: one line").  Decode versus prefill, and a replay flush versus
 * token-by-token updates, agree within rounding but not bitwise.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_ARG = 1,        /* a required pointer is NULL */
  GDN_ERR_BAD_SHAPE = 2,       /* head counts, head_dim, conv width or strides not supported */
  GDN_ERR_BAD_DTYPE = 3,       /* unknown dtype or activation code */
  GDN_ERR_BAD_VARLEN = 4,      /* cu_seqlens not starting at 0 / decreasing, negative start_pos */
  GDN_ERR_OFF_BOUNDARY = 5,    /* state source inconsistent with start_pos (see gdn_src) */
  GDN_ERR_PAGE_TOO_SMALL = 6,  /* page_bytes < gdn_checkpoint_bytes, or misaligned pool */
  GDN_ERR_BAD_PAGE = 7,        /* page id outside [-1, n_pages) or a page used twice */
  GDN_ERR_CAPACITY = 8,        /* a count exceeds what the call supports (rows, slots) */
  GDN_ERR_WORKSPACE = 9,       /* workspace NULL, too small or misaligned */
  GDN_ERR_HIP = 10,            /* a HIP runtime call failed while enqueueing */
  GDN_ERR_BAD_SOURCE = 11,     /* unknown state source kind */
  GDN_ERR_STAGING = 12         /* the tables need a staging buffer: missing or too small */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_act { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_act;
/* Flag OR-ed into gdn_layer.conv_act: after the activation, every q and k head of a
 * conv output row (channels [0, 2 * n_qk_heads * head_dim), head_dim values each) is
 * scaled to unit L2 norm, y <- y * (sum y^2 + 1e-6)^(-1/2): the post-conv step of the
 * packed core ("Hybrid linear attention (gated DeltaNet)", "Packed-core traces"), done
 * inside the conv pass.  Value channels and the stored tails are unaffected. */
#define GDN_CONV_QK_L2NORM 0x100

/* Layer descriptor.  head_dim is d_k = d_v and must be 16, 32, 64 or 128.
 * n_v_heads must be a positive multiple of n_qk_heads: invalid dimensions and head
 * counts that do not divide are refused, as "Hybrid linear attention (gated
 * DeltaNet)", section "Packed-core traces", requires.  conv_width must be 4.
 * io_dtype is the type of q, k, v and of the conv input, output, weights and tails.
 * The conv activation is applied after the conv sum. */
typedef struct gdn_layer {
  int32_t n_qk_heads;
  int32_t n_v_heads;
  int32_t head_dim;
  int32_t conv_width;
  int32_t io_dtype;  /* gdn_dtype */
  int32_t conv_act;  /* gdn_act */
  float scale;       /* output scale, e.g. 1.0 or 1/sqrt(d) */
} gdn_layer;

/* Variable-length batch, all [host].  Sequence s owns packed rows
 * [cu_seqlens[s], cu_seqlens[s+1]); cu_seqlens[0] == 0 and it never decreases (a
 * sequence may have zero rows).  start_pos[s] >= 0 is the absolute position, counted
 * from the start of that sequence, of its first row in this call. */
typedef struct gdn_varlen {
  int32_t n_seqs;
  const int64_t* cu_seqlens; /* [host] n_seqs + 1 */
  const int64_t* start_pos;  /* [host] n_seqs */
} gdn_varlen;

/* Where a sequence's incoming state (or conv tail) comes from.
 *   GDN_SRC_ZERO:       all zeros; requires start_pos == 0; no memory is read.
 *   GDN_SRC_SLOT:       `src` points at the state (or tail) itself; requires start_pos > 0.
 *   GDN_SRC_CHECKPOINT: `src` points at a checkpoint page (layout below); requires
 *                       start_pos > 0 and start_pos % block == 0: a resume off a block
 *                       boundary is refused ("Prefix caching on Gated DeltaNet
 *                       hybrids", "The in-page layout": fail closed), since a state can
 *                       only be restored where one was saved ("The cache block that is
 *                       not a cache setting", "Why a hybrid cannot use a 64-token page"). */
typedef enum gdn_src { GDN_SRC_ZERO = 0, GDN_SRC_SLOT = 1, GDN_SRC_CHECKPOINT = 2 } gdn_src;

/* Per-sequence state reference, [host] array of n_seqs.  `dst` receives the state (or
 * tail) after the sequence's last row; it may equal `src` for an in-place update but
 * must not overlap another sequence's src or dst. */
typedef struct gdn_state_ref {
  int32_t src_kind; /* gdn_src */
  const void* src;  /* device */
  void* dst;        /* device */
} gdn_state_ref;

/* Checkpoint pages.  A page holds, from its start: the fp32 state
 * [n_v_heads][d][d] (gdn_state_bytes), then the conv tail [conv_width-1][channels] in
 * io_dtype (gdn_conv_tail_bytes).  "Prefix caching on Gated DeltaNet hybrids" ("Why
 * hits were wrong", "The in-page layout") stores such checkpoints inside attention
 * pages of block * bytes-per-token; any page_bytes >= gdn_checkpoint_bytes works.
 * A checkpoint is written when a sequence's absolute position reaches a positive
 * multiple of `block` (the call's last row included): it holds the state after
 * exactly that many tokens, i.e. the state that closes the block (same page and
 * section: a complete block carries the recurrent state reached at its end).
 * Positions stay below 2^30 (GDN_ERR_CAPACITY).  page_ids lists one page per crossed boundary,
 * sequences in order and boundaries in order (gdn_count_boundaries gives the count
 * per sequence); -1 means "do not store this one".  block == 0 disables
 * checkpoints; the pool and page_ids are then not read. */
typedef struct gdn_ckpt {
  void* pool;                /* device, 256-byte aligned */
  int64_t page_bytes;        /* multiple of 256 */
  int64_t n_pages;
  int32_t block;             /* tokens per cache block, 0 .. 2^24 */
  const int32_t* page_ids;   /* [host] */
} gdn_ckpt;

/* Host staging for the per-call tables of a batch larger than the kernel arguments
 * carry (more than GDN_INLINE_SEQS sequences or GDN_INLINE_PAGES crossed boundaries).
 * `host` is caller-owned host memory of at least gdn_*_staging_bytes bytes, pinned
 * (hipHostMalloc, or a torch tensor with pin_memory=True) so that the copy from it is
 * asynchronous; the call writes the tables into it and enqueues one copy into the
 * table region of the workspace.  Keep it untouched until the stream has passed the
 * call.  May be NULL when the staging size is 0. */
#define GDN_INLINE_SEQS 8
#define GDN_INLINE_PAGES 256
typedef struct gdn_staging {
  void* host;
  size_t bytes;
} gdn_staging;

/* ---------------------------------------------------------------- sizes and helpers */

int32_t gdn_abi_version(void);
const char* gdn_status_string(gdn_status status);

/* Bytes of one fp32 state: n_v_heads * d * d * 4 (3 MiB at 48 heads of 128 x 128, the
 * figure of "Prefix caching on Gated DeltaNet hybrids", "Why hits were wrong").  -1 if
 * the layer is invalid. */
int64_t gdn_state_bytes(const gdn_layer* layer);
/* Bytes of one conv tail: (conv_width - 1) * (2 n_qk_heads + n_v_heads) d * sizeof(io),
 * the conv part of the state (same page and section; "Hybrid linear attention (gated
 * DeltaNet)", "Why this family is different"). */
int64_t gdn_conv_tail_bytes(const gdn_layer* layer);
/* State plus conv tail, rounded up to 256 bytes: the minimum page_bytes (the
 * per-layer checkpoint that "Prefix caching on Gated DeltaNet hybrids", "Why hits
 * were wrong", stores in an attention page). */
int64_t gdn_checkpoint_bytes(const gdn_layer* layer);
/* Number of conv channels (2 n_qk_heads + n_v_heads) * d: the packed q | k | v rows the
 * conv runs over ("Hybrid linear attention (gated DeltaNet)", "Packed-core traces"). */
int64_t gdn_conv_channels(const gdn_layer* layer);

/* Tokens served from cache for a shared prefix: whole blocks only, the last full
 * block left open, so max(0, (floor(shared / block) - 1) * block) ("The cache block
 * that is not a cache setting", section "What that costs, exactly").  0 if block <= 0. */
int64_t gdn_cached_prefix_tokens(int64_t shared, int64_t block);
/* A prefill chunk budget floored to a block boundary, floor(budget / block) * block
 * ("Hybrid linear attention (gated DeltaNet)", "Why this family is different", item 3).
 * Returns budget when block <= 0. */
int64_t gdn_floor_chunk(int64_t budget, int64_t block);
/* Number of block boundaries p * block, p >= 1, in (start_pos, start_pos + n_tokens]. */
int64_t gdn_count_boundaries(int64_t start_pos, int64_t n_tokens, int64_t block);
/* Cache block size that lets one attention page hold one state:
 * alignment * cdiv(state_bytes, alignment * attn_bytes_per_token) ("Hybrid linear
 * attention (gated DeltaNet)", "Why this family is different", item 2).  -1 on bad input. */
int64_t gdn_block_size_for_state(int64_t state_bytes, int64_t attn_bytes_per_token,
                                 int64_t alignment);

/* Workspace bytes gdn_chunk_prefill needs for this batch and block: room for the
 * staged tables, then one record of chunk factors per (chunk, value head) -- the
 * state-free half of the chunked form of the rule (the WY / UT transform of
 * "Gated Delta Networks", Yang, Kautz & Hatamizadeh, ICLR 2025).  -1 if invalid. */
int64_t gdn_prefill_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen,
                                    int32_t block);
/* Bytes of pinned host staging a prefill of this batch and block needs; 0 when its
 * tables fit the kernel arguments.  -1 if invalid. */
int64_t gdn_prefill_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen,
                                  int32_t block);
/* Workspace bytes gdn_conv_update needs (the staged tables only; 0 when they fit the
 * kernel arguments, and the workspace may then be NULL).  -1 if invalid. */
int64_t gdn_conv_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen,
                                 int32_t block);
/* Bytes of pinned host staging a conv of this batch needs; 0 when none.  -1 if invalid. */
int64_t gdn_conv_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen,
                               int32_t block);

/* ---------------------------------------------------------------- the hot path */

/* Short causal conv update over a varlen batch ("Hybrid linear attention (gated
 * DeltaNet)", section "The part that is easy to get wrong": gdn_conv_prefill /
 * gdn_conv_decode).
 *   x  row t at x + t * x_stride: C io_dtype values, C = gdn_conv_channels (the packed
 *      q | k | v channels); x_stride >= C elements, x_stride * io bytes a multiple of 16
 *      (C for dense rows, the packed qkvz row width to read the in-projection in place)
 *   w  [C][conv_width] io_dtype; w[c][conv_width-1] multiplies the current token
 *   y  [tokens][C] io_dtype: act(sum_j w[c][j] * x[t - (W-1) + j][c]), fp32 sums,
 *      rounded to io_dtype with round-to-nearest-even
 *   tails [host] n_seqs refs to [W-1][C] io_dtype tails (oldest row first): the rows
 *      before each sequence's first token (ZERO: none), and the last W-1 rows after
 *      it.  A CHECKPOINT source is a page base; the tail is read from its tail region.
 *   ckpt: at every crossed block boundary, the W-1 raw rows before it are written
 *      to the tail region of that boundary's page.
 * x and y must not overlap.  Errors: see gdn_status. */
gdn_status gdn_conv_update(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                           const void* x, int64_t x_stride, const void* w, const gdn_state_ref* tails,
                           const gdn_ckpt* ckpt, void* y, void* workspace,
                           size_t workspace_bytes, const gdn_staging* staging);

/* The conv's decode regime ("Hybrid linear attention (gated DeltaNet)", "The part that
 * is easy to get wrong": gdn_conv_decode beside gdn_conv_prefill): one new row per
 * request, whose previous conv_width - 1 rows sit in slot slot_ids[r] of a tail pool.
 * For each request r with its row t = rows[r] (rows NULL: t = r):
 *   y[t][c] = act(w[c][0] tail[0][c] + w[c][1] tail[1][c] + w[c][2] tail[2][c] + w[c][3] x[t][c])
 * (the GDN_CONV_QK_L2NORM flag normalises the q and k heads as in gdn_conv_update), and
 * the slot becomes (tail[1], tail[2], x[t]).
 *   x: row t at x + t * x_stride (x_stride as in gdn_conv_update); y [n_rows][C]
 *   io_dtype (the packed rows of a batch; C = gdn_conv_channels);
 *   w [C][conv_width]; tail_pool [n_slots][conv_width - 1][C] io_dtype, updated in place;
 *   slot_ids, rows [n_req] int32 (device).  Slot -1 reads and writes nothing; a slot
 *   outside [-1, n_slots) or a row outside [0, n_rows) leaves the request untouched and
 *   sets GDN_ERR_CAPACITY in *status (device int32, may be NULL).  Two requests must not
 *   share a slot.  No checkpoint tail is written: after a token that ends a block, the
 *   slot holds exactly that block's tail. */
gdn_status gdn_conv_decode(const gdn_layer* layer, hipStream_t stream, int32_t n_req, int64_t n_rows,
                           const void* x, int64_t x_stride, const void* w, void* tail_pool,
                           int64_t n_slots, const int32_t* slot_ids, const int32_t* rows, void* y,
                           int32_t* status);

/* Chunked varlen prefill of the gated delta rule with block checkpoints ("Hybrid
 * linear attention (gated DeltaNet)", "The part that is easy to get wrong":
 * gdn_prefill; checkpoints and resume as in "Prefix caching on Gated DeltaNet hybrids",
 * "Why hits were wrong").
 *   q, k  [tokens][qk_stride] io_dtype, head h at offset h*d; qk_stride >= n_qk_heads*d
 *         (pass n_qk_heads*d for dense tensors).  The recurrence reads them as given
 *         (no normalisation).
 *   v     [tokens][v_stride] io_dtype, v_stride >= n_v_heads*d.
 *   a, b  [tokens][n_v_heads] fp32.  a in (0, 1], b in [0, 1].
 *   states [host] n_seqs state refs (ZERO, SLOT or CHECKPOINT); dst gets the final state.
 *   ckpt  block checkpoints (state region of each page).
 *   o     [tokens][n_v_heads][d] fp32.
 *   workspace >= gdn_prefill_workspace_bytes(layer, varlen, ckpt->block), 256-byte aligned.
 * Each sequence is cut into chunks at every multiple of 64 tokens, at every multiple
 * of the block and at the call's ends, positions counted from the sequence start, so
 * every crossed block boundary ends a chunk ("The prefix cache changed the answer",
 * "The fix: one line").  q, k, v, a, b, o and the workspace must not overlap. */
gdn_status gdn_chunk_prefill(const gdn_layer* layer, hipStream_t stream,
                             const gdn_varlen* varlen, const void* q, const void* k,
                             const void* v, int64_t qk_stride, int64_t v_stride, const float* a,
                             const float* b, const gdn_state_ref* states, const gdn_ckpt* ckpt,
                             float* o, void* workspace, size_t workspace_bytes,
                             const gdn_staging* staging);

/* gdn_chunk_prefill for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation with the
 * same results, bit for bit, but no workspace or staging argument.  Its chunk factors go
 * to a fixed device array of GDN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU
 * (held from the library's load on that GPU until the process ends); the caller still
 * passes the inputs and outputs.  A batch whose workspace (gdn_prefill_workspace_bytes)
 * exceeds that size, or whose tables do not fit the kernel arguments (more than
 * GDN_INLINE_SEQS sequences or GDN_INLINE_PAGES boundaries), is refused with
 * GDN_ERR_CAPACITY and nothing is enqueued.  64 MiB holds the records of about 2,600
 * (chunk, value head) pairs: a 1,792-token step of a 48-head layer needs under 40 MiB.
 * All calls on one GPU share its array: calls that overlap in time on one GPU (two
 * streams, two threads) race on it, so order them.  It calls no allocating routine; its
 * first call on a device looks up the array's device address once (hipGetSymbolAddress)
 * and keeps it. */
#define GDN_NOALLOC_SCRATCH_BYTES (64 << 20)
gdn_status gdn_chunk_prefill_noalloc(const gdn_layer* layer, hipStream_t stream,
                                     const gdn_varlen* varlen, const void* q, const void* k,
                                     const void* v, int64_t qk_stride, int64_t v_stride,
                                     const float* a, const float* b, const gdn_state_ref* states,
                                     const gdn_ckpt* ckpt, float* o);

/* The two stages of gdn_chunk_prefill, for callers that schedule or time them apart.
 * gdn_prefill_factorize computes, for every chunk and value head, the state-free
 * chunk factors into the workspace: the gate vectors from the cumulative log-decay,
 * the inverse of the unit lower triangular key-interaction matrix (the WY / UT
 * transform of the chunk), the causal decayed query-key scores and the keys
 * transposed.  gdn_prefill_scan then walks each sequence chunk by chunk and applies
 * them to the state.  The scan must run on the same stream after a factorize with the
 * same layer, varlen, q, k, a, b, ckpt->block and workspace.  Together they do exactly
 * what gdn_chunk_prefill does.  Each stages its own tables when the batch needs it
 * (two calls in a row need two staging buffers, or a wait between them).  Strides: qk_stride * io bytes, v_stride * io bytes and
 * n_v_heads * d * 4 must each stay below 2^31 / 64 (GDN_ERR_BAD_SHAPE otherwise; the
 * same holds for gdn_chunk_prefill). */
gdn_status gdn_prefill_factorize(const gdn_layer* layer, hipStream_t stream,
                                 const gdn_varlen* varlen, const void* q, const void* k,
                                 int64_t qk_stride, const float* a, const float* b, int32_t block,
                                 void* workspace, size_t workspace_bytes,
                                 const gdn_staging* staging);
gdn_status gdn_prefill_scan(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                            const void* q, const void* k, const void* v, int64_t qk_stride,
                            int64_t v_stride, const gdn_state_ref* states, const gdn_ckpt* ckpt,
                            float* o, void* workspace, size_t workspace_bytes,
                            const gdn_staging* staging);

/* One decode token per request ("Hybrid linear attention (gated DeltaNet)", "The part
 * that is easy to get wrong": gdn_decode).  Request r updates the state in slot
 * slot_ids[r] of state_pool [n_slots][n_v_heads][d][d] in place and writes
 * o[r] = scale * S_new q.
 *   q, k [n_req][n_qk_heads][d], v [n_req][n_v_heads][d] io_dtype; a, b [n_req][n_v_heads].
 *   slot_ids [n_req] int32 (device): -1 marks padding: that request reads and writes
 *   nothing, its o row included ("Prefix caching on Gated DeltaNet hybrids", "The
 *   in-page layout", defect 2).  A slot id outside [-1, n_slots) is not touched either
 *   and sets GDN_ERR_CAPACITY in *status.  Two requests must not share a slot.
 *   status: device int32, may be NULL; data-dependent errors are OR-ed into it. */
gdn_status gdn_decode_step(const gdn_layer* layer, hipStream_t stream, int32_t n_req,
                           const void* q, const void* k, const void* v, const float* a,
                           const float* b, float* state_pool, int64_t n_slots,
                           const int32_t* slot_ids, float* o, int32_t* status);

/* The decode tokens of a mixed batch ("Hybrid linear attention (gated DeltaNet)", "The
 * part that is easy to get wrong": in the mixed regime gdn_decode_mixed runs beside the
 * prefill kernels).  As gdn_decode_step, but request r's token is row rows[r] of packed
 * token arrays that the batch's prefill sequences share (their rows go to
 * gdn_chunk_prefill, the decode rows here; the conv covers all of them as sequences):
 *   q, k: row t at q + t * qk_stride ([n_qk_heads][d] at the row's start); v: row t at
 *   v + t * v_stride; a, b [n_rows][n_v_heads] fp32; o [n_rows][n_v_heads][d] fp32.
 *   rows [n_req] int32 (device).  A row outside [0, n_rows) for a request with a slot
 *   writes nothing for it and sets GDN_ERR_CAPACITY in *status.  Slot rules as for
 *   gdn_decode_step. */
gdn_status gdn_decode_mixed(const gdn_layer* layer, hipStream_t stream, int32_t n_req, int64_t n_rows,
                            const void* q, const void* k, const void* v, int64_t qk_stride,
                            int64_t v_stride, const float* a, const float* b, float* state_pool,
                            int64_t n_slots, const int32_t* slot_ids, const int32_t* rows, float* o,
                            int32_t* status);

/* ReplaySSM flush ("Caching less to serve more requests", section "What we changed"):
 * each request keeps one state plus a log of per-token inputs since it; the flush
 * folds the first n_accepted[r] logged rows of request r into its state as blocked
 * updates of up to 32 rows each, in one launch for all requests.  The state in slot slot_ids[r] of
 * state_pool [n_slots][n_v_heads][d][d] is read once and written once; rows at or
 * past n_accepted[r] are never read (a rollback is just a smaller n_accepted).
 *   buf_k [n_slots][buf_rows][n_qk_heads][d], buf_v [n_slots][buf_rows][n_v_heads][d]
 *   io_dtype; buf_a, buf_b [n_slots][buf_rows][n_v_heads] fp32: the log of each slot.
 *   buf_rows <= 64 (the pages use 32).  n_accepted [n_req] int32 (device): requests
 *   with 0 rows or slot -1 are left untouched; n_accepted outside [0, buf_rows] or a
 *   slot outside [-1, n_slots) leaves the request untouched and sets GDN_ERR_CAPACITY
 *   in *status (device int32, may be NULL).  Two requests must not share a slot. */
gdn_status gdn_replay_flush(const gdn_layer* layer, hipStream_t stream, int32_t n_req,
                            float* state_pool, int64_t n_slots, const int32_t* slot_ids,
                            const void* buf_k, const void* buf_v, const float* buf_a,
                            const float* buf_b, int32_t buf_rows, const int32_t* n_accepted,
                            int32_t* status);

/* Gates of the packed core ("Hybrid linear attention (gated DeltaNet)", "Packed-core
 * traces": the core owns dt_bias and a float32 A_log and takes the "ba" projection).
 * For each token t and value head h, in fp32:
 *   b[t][h] = sigmoid(ba[t][h]),
 *   a[t][h] = exp(-exp(A_log[h]) * softplus(ba[t][Hv + h] + dt_bias[h])),
 * a kept at or above the smallest normal float (its log is the prefill's log-decay).
 *   ba: token t at ba + t * ba_stride (ba_stride >= 2 * n_v_heads elements), io_dtype;
 *   A_log [n_v_heads] fp32; dt_bias [n_v_heads] io_dtype; a, b [n_tokens][n_v_heads]
 *   fp32, the decay and write strength gdn_chunk_prefill and gdn_decode_step take. */
gdn_status gdn_gates(const gdn_layer* layer, hipStream_t stream, int64_t n_tokens, const void* ba,
                     int64_t ba_stride, const float* A_log, const void* dt_bias, float* a, float* b);

/* Gated RMSNorm of the output rows (the packed core's output is "gated-normalized value
 * rows", with one norm scale replicated over the heads; same page and section).  For
 * each token t, value head h and channel j:
 *   out[t][h][j] = o[t][h][j] * (mean_j o[t][h][j]^2 + eps)^(-1/2) * weight[j] * silu(z[t][h][j]).
 *   o [n_tokens][n_v_heads][d] fp32 (the prefill or decode output); z: token t at
 *   z + t * z_stride, [n_v_heads][d] io_dtype (z_stride a multiple of 8 elements, at
 *   least n_v_heads * d); weight [d] io_dtype; out [n_tokens][n_v_heads][d] io_dtype.
 *   o, z, weight, out 16-byte aligned; eps >= 0. */
gdn_status gdn_gated_norm(const gdn_layer* layer, hipStream_t stream, int64_t n_tokens, const float* o,
                          const void* z, int64_t z_stride, const void* weight, float eps, void* out);

/* The packed core over a varlen batch ("Hybrid linear attention (gated DeltaNet)",
 * "Packed-core traces": its input is the packed qkvz rows plus the "ba" projection, its
 * output the gated-normalized value rows; it owns the conv taps, dt_bias, the fp32 A_log
 * and the norm scale).  One call enqueues, on `stream`:
 *   gdn_conv_update over the q | k | v channels of each packed row (the layer's
 *   activation and q/k norm flags apply) -> gdn_gates over ba -> gdn_chunk_prefill on
 *   q, k, v read in place from the conv's rows -> gdn_gated_norm with z read in place
 *   from the packed rows;
 * each stage exactly as that call defines it.  Everything is checked before the first
 * stage is enqueued.
 *   qkvz: row t at qkvz + t * qkvz_stride holds [q (n_qk_heads*d) | k (n_qk_heads*d) |
 *     v (n_v_heads*d) | z (n_v_heads*d)] io_dtype; qkvz_stride >= C + n_v_heads*d
 *     (C = gdn_conv_channels), qkvz_stride * io bytes a multiple of 16, qkvz 16-byte
 *     aligned.  (The pages give no layout inside the packed row; this one is the plain
 *     concatenation in the order of the name.)
 *   ba: row t at ba + t * ba_stride, [b (n_v_heads) | a (n_v_heads)] io_dtype.
 *   conv_w [C][conv_width], A_log [n_v_heads] fp32, dt_bias [n_v_heads] and
 *     norm_weight [d] io_dtype; eps as in gdn_gated_norm.
 *   tails, states [host]: per sequence, the conv tail and the state references of
 *     gdn_conv_update and gdn_chunk_prefill; ckpt: as there (each crossed boundary's
 *     page receives both the state and the tail).
 *   out [tokens][n_v_heads][d] io_dtype.
 *   workspace: gdn_core_prefill_workspace_bytes (256-byte aligned; it holds the stage
 *     outputs), staging: gdn_core_prefill_staging_bytes (may be NULL when 0). */
int64_t gdn_core_prefill_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block);
int64_t gdn_core_prefill_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block);
gdn_status gdn_core_prefill(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                            const void* qkvz, int64_t qkvz_stride, const void* ba, int64_t ba_stride,
                            const void* conv_w, const float* A_log, const void* dt_bias,
                            const void* norm_weight, float eps, const gdn_state_ref* tails,
                            const gdn_state_ref* states, const gdn_ckpt* ckpt, void* out,
                            void* workspace, size_t workspace_bytes, const gdn_staging* staging);

/* ReplaySSM verification outputs ("Caching less to serve more requests", section "What
 * we changed": each request keeps one state and a log of the per-token inputs since it,
 * and a layer's output is computed from the two).  Request r has m = n_logged[r] rows
 * in the log of slot slot_ids[r] and n = n_new[r] new rows written behind them by the
 * caller (log rows m .. m + n - 1).  The gated delta rule runs from the slot's state
 * over log rows 0 .. m + n - 1, and o[r][i] = scale * S_{m+i} q_new[r][i] for i < n,
 * with S_t the state after log row t.  Nothing is written to the state or the log: a
 * later gdn_replay_flush accepts rows, a smaller count rolls them back.
 *   state_pool, buf_k, buf_v, buf_a, buf_b, buf_rows (<= 64) as for gdn_replay_flush;
 *   with fp32 inputs at d = 128, buf_rows <= 32 (GDN_ERR_CAPACITY otherwise).
 *   q_new [n_req][max_new][n_qk_heads][d] io_dtype; o [n_req][max_new][n_v_heads][d]
 *   fp32, rows at or past n_new[r] not written.  n_logged, n_new [n_req] int32
 *   (device).  Slot -1 or n = 0 writes nothing.  m < 0, n < 0, m + n > buf_rows,
 *   n > max_new or a slot outside [-1, n_slots) writes nothing for that request and
 *   sets GDN_ERR_CAPACITY in *status (device int32, may be NULL).  All device pointers;
 *   libgdn allocates nothing. */
gdn_status gdn_replay_forward(const gdn_layer* layer, hipStream_t stream, int32_t n_req,
                              const float* state_pool, int64_t n_slots, const int32_t* slot_ids,
                              const void* buf_k, const void* buf_v, const float* buf_a,
                              const float* buf_b, int32_t buf_rows, const int32_t* n_logged,
                              const int32_t* n_new, const void* q_new, int32_t max_new, float* o,
                              int32_t* status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
