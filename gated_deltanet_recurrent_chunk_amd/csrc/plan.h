// plan.h -- host-side validation and planning for libgdn (no HIP calls, no device code).
//
// Everything a call checks before it enqueues work lives here, together with the
// chunk-grid rule and the layout of the small tables that the host uploads for the
// kernels.  Kept free of HIP so that it is plain C++ that can be reasoned about and
// exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/gdn.h"

namespace gdn {

constexpr int kChunk = 64;          // rows per prefill chunk (the MFMA tile height x 4)
constexpr int kConvTile = 16;       // rows per conv tile
constexpr int kMaxBufRows = 64;     // replay-flush log rows per request
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Functions both the host planner and the kernels evaluate (the kernels derive every
// chunk and tile of a sequence from its table entry with them; the host sizes the
// workspace and validates with the same code).
#ifdef __HIP__
#define GDN_HD __host__ __device__
#else
#define GDN_HD
#endif

// A 64-bit address from its two 32-bit halves, as a kernel rebuilds a wave-uniform
// pointer after moving each half through readfirstlane (which returns a signed int).
// Both halves are widened as unsigned: a sign-extended low half would fill the high
// word with ones whenever bit 31 of the address is set.
GDN_HD inline uint64_t join_address(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | (uint64_t)lo; }

// ------------------------------------------------------------------ call tables
// The only per-call table of the prefill and conv kernels: one entry per sequence and
// the page id of every crossed block boundary.  Chunks and tiles are not tabulated;
// each kernel derives them from the entry (chunk_start, next_cut, tile rows below).
struct SeqEntry {
  const void* src;  // incoming state or conv tail; nullptr = zero rows, never read
  void* dst;        // final state or new conv tail
  int64_t row0;     // first packed row
  int32_t p0;       // absolute position of the first row
  int32_t len;      // rows
  int32_t unit0;    // global index of the sequence's first chunk (prefill) or tile (conv)
  int32_t n_units;  // its chunks or tiles
  int32_t page0;    // index of its first crossed block boundary in the page list
  int32_t pad;
};
static_assert(sizeof(SeqEntry) == 48, "SeqEntry layout");

// Tables up to this size travel in the kernel arguments; larger ones are copied from a
// caller-owned pinned staging buffer into the caller's workspace (gdn.h).
constexpr int kInlineSeqs = 8;
constexpr int kInlinePages = 256;
// Positions stay below 2^30, so that 32-bit chunk arithmetic never overflows.
constexpr int64_t kMaxPosition = (int64_t)1 << 30;

struct CallTable {
  const SeqEntry* seqs;     // staged copy in device memory, or nullptr: inl_seqs
  const int32_t* pages;     // staged copy, or nullptr: inl_pages
  const int32_t* unit_seq;  // staged: the sequence of every unit; nullptr when inline
  int32_t n_seqs, n_pages, n_units, block;
  uint32_t lcm;             // lcm(kChunk, block), 0 without blocks
  uint32_t pad[3];
  SeqEntry inl_seqs[kInlineSeqs];
  int32_t inl_pages[kInlinePages];
};

// The chunk grid of one sequence: cuts at every multiple of kChunk and of the block
// (positions counted from the sequence start) strictly inside (p0, p0 + len), plus
// both ends.  All positions are below kMaxPosition.
GDN_HD inline uint32_t grid_lcm(uint32_t block) {
  if (block == 0) return 0;
  uint32_t a = block, b = kChunk;
  while (b) {
    const uint32_t t = a % b;
    a = b;
    b = t;
  }
  return block / a * kChunk;
}
// Number of cuts in (p0, x], for p0 <= x.
GDN_HD inline uint32_t cuts_upto(uint32_t p0, uint32_t x, uint32_t block, uint32_t lcm) {
  uint32_t n = x / kChunk - p0 / kChunk;
  if (block) n += (x / block - p0 / block) - (x / lcm - p0 / lcm);
  return n;
}
// Chunks of a sequence of len rows starting at p0.
GDN_HD inline uint32_t chunk_count(uint32_t p0, uint32_t len, uint32_t block, uint32_t lcm) {
  return len ? cuts_upto(p0, p0 + len - 1, block, lcm) + 1 : 0;
}
// Start position of chunk j < chunk_count: the j-th cut after p0 (chunk 0 starts at p0).
GDN_HD inline uint32_t chunk_start(uint32_t p0, uint32_t j, uint32_t block, uint32_t lcm) {
  if (j == 0) return p0;
  const uint32_t first = p0 / kChunk;
  // the multiples of kChunk alone give j cuts in (p0, (first + j) kChunk]
  uint32_t hi = (first + j) * kChunk;
  if (block % kChunk == 0) return hi;  // every block boundary is a multiple of kChunk
  uint32_t lo = p0 + 1;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (cuts_upto(p0, mid, block, lcm) >= j)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}
// The cut after position x, capped at end.
GDN_HD inline uint32_t next_cut(uint32_t x, uint32_t end, uint32_t block) {
  uint32_t n = (x / kChunk + 1) * kChunk;
  if (block) {
    const uint32_t nb = (x / block + 1) * block;
    if (nb < n) n = nb;
  }
  return n < end ? n : end;
}
// Ordinal (0-based) of the block boundary at position P, p0 < P, within a sequence
// starting at p0.
GDN_HD inline uint32_t boundary_ordinal(uint32_t p0, uint32_t P, uint32_t block) {
  return P / block - p0 / block - 1;
}
// Conv tiles of a sequence: kConvTile rows each; an empty sequence has one empty tile
// (it passes its tail through).
GDN_HD inline uint32_t tile_count(uint32_t len) { return len ? (len + kConvTile - 1) / kConvTile : 1; }

// ------------------------------------------------------------------ layer facts
struct LayerInfo {
  int Hqk, Hv, D, W;
  int io;           // gdn_dtype
  int act;
  float scale;
  int64_t channels;
  size_t io_bytes;
  int64_t state_bytes;
  int64_t tail_bytes;
  int64_t ckpt_bytes;
  int ntf;          // bf16 terms carried by fp32 operands in matrix products
  int nti;          // bf16 terms carried by an input operand (1 for bf16 inputs)
};

gdn_status check_layer(const gdn_layer* layer, LayerInfo* out);

// ------------------------------------------------------------------ varlen / sources
struct SeqSpan {
  int64_t row0, len, p0;
};
gdn_status check_varlen(const gdn_varlen* v, std::vector<SeqSpan>* spans);
// Every state reference must be consistent with its start position (and the block for a
// checkpoint source).
gdn_status check_sources(const gdn_state_ref* refs, const std::vector<SeqSpan>& spans,
                         int32_t block);
// Checkpoint pool checks; fills the flat page-id list (one per crossed boundary).
gdn_status check_ckpt(const gdn_ckpt* ckpt, const LayerInfo& L, const std::vector<SeqSpan>& spans,
                      std::vector<int32_t>* pages, std::vector<int32_t>* page_begin);

// ------------------------------------------------------------------ chunk grid
// Cut points of one sequence: every multiple of kChunk and of `block` strictly inside
// (p0, p0 + len), plus both ends; positions are absolute within the sequence.
void chunk_grid(int64_t p0, int64_t len, int32_t block, std::vector<int64_t>* cuts);
int64_t count_boundaries(int64_t p0, int64_t len, int64_t block);

// A planned prefill or conv call: the table entries (src / dst filled by the caller of
// the planner), the flat page list, and the workspace layout.  The workspace holds
// the staged table (when the table does not fit the kernel arguments), then, for the
// prefill, one factor record per (chunk, value head).
struct CallPlan {
  std::vector<SeqEntry> seqs;
  std::vector<int32_t> pages;
  int32_t n_units = 0, block = 0;
  uint32_t lcm = 0;
  bool staged = false;                 // table exceeds the kernel-argument capacity
  size_t table_bytes = 0;              // staged table: entries, pages, unit -> sequence map
  size_t off_pages = 0, off_unit_seq = 0;
  size_t off_factors = 0, factor_stride = 0, total_bytes = 0;
};
// Plans a prefill (units = chunks) or conv (units = tiles) call.  pages may be null (no
// page ids needed: the factorize stage).  Fails with GDN_ERR_CAPACITY past the
// position, unit or page limits.
gdn_status plan_call(const LayerInfo& L, const std::vector<SeqSpan>& spans, int32_t block,
                     const std::vector<int32_t>* pages, const std::vector<int32_t>* page_begin,
                     bool prefill, CallPlan* plan);
// Host image of the staged table (plan->table_bytes bytes).
void staged_table(const CallPlan& plan, uint8_t* out);
// The kernel-argument form of the table: inline arrays, or pointers into the staged
// copy at workspace `ws`.
void fill_call_table(const CallPlan& plan, const void* ws, CallTable* t);

// Bytes of the per-(chunk, value head) factor record written by the prefill pre-pass.
// Every matrix in it is stored as ready-made MFMA A-operand fragments of 1 KiB (16
// bytes per lane of a 64-lane wave), ntf (or nti) bf16 terms each:
//   T = (I + A)^-1: 6 fragments x ntf (the (row tile, k-step) pairs of its lower triangle)
//   P = scale * exp(g_t - g_s) q_t.k_s (s <= t): 6 x ntf, same pairs
//   K^T: (d / 16) row tiles x 2 k-steps x nti, except for bf16 inputs with d >= 64,
//        whose scan forms K^T from the key rows it stages
// then four fp32 row vectors of kChunk and one fp32 chunk scalar (16 bytes).
constexpr size_t factor_record_bytes_c(int ntf, int nti, int d) {
  const bool kt = !(nti == 1 && d >= 64);
  return ((size_t)12 * ntf * 1024 + (kt ? (size_t)(d / 16) * 2 * nti * 1024 : 0) + 4 * kChunk * 4 + 16 + kAlign - 1) /
         kAlign * kAlign;
}
inline size_t factor_record_bytes(int ntf, int nti, int d) { return factor_record_bytes_c(ntf, nti, d); }

}  // namespace gdn
