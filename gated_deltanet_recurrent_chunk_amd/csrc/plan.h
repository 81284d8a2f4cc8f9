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

// ------------------------------------------------------------------ device tables
// One prefill chunk: packed rows [row, row + len) of one sequence; after it, the state
// is stored to checkpoint page `page` (or not, when page < 0).
struct ChunkDesc {
  int64_t row;
  int32_t len;
  int32_t page;
};
static_assert(sizeof(ChunkDesc) == 16, "ChunkDesc layout");

// One prefill sequence as the scan sees it.
struct ScanSeq {
  const float* src;  // incoming state, nullptr = zero state (never read)
  float* dst;        // final state
  int32_t chunk_begin, chunk_end;
  int32_t pad0, pad1;
};
static_assert(sizeof(ScanSeq) == 32, "ScanSeq layout");

// One conv sequence.
struct ConvSeq {
  const void* src_tail;  // nullptr = zero rows (never read)
  void* dst_tail;
  int64_t row0;          // first packed row
  int64_t p0;            // absolute position of the first row
  int64_t len;
  int32_t page_begin;    // index of its first crossed boundary in the page-id table
  int32_t pad;
};
static_assert(sizeof(ConvSeq) == 48, "ConvSeq layout");

// One conv tile: packed rows [row, row + len) of sequence `seq`.
struct ConvTile {
  int64_t row;
  int32_t len;
  int32_t seq;
};
static_assert(sizeof(ConvTile) == 16, "ConvTile layout");

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

struct PrefillPlan {
  std::vector<ChunkDesc> chunks;
  std::vector<int32_t> seq_chunk_begin;  // n_seqs + 1
  size_t off_chunks, off_seqs, off_factors, factor_stride, total_bytes;
};
// pages may be null (factorize stage: no page ids needed); page entries are then -1.
void plan_prefill(const LayerInfo& L, const std::vector<SeqSpan>& spans, int32_t block,
                  const std::vector<int32_t>* pages, const std::vector<int32_t>* page_begin,
                  PrefillPlan* plan);

struct ConvPlan {
  std::vector<ConvTile> tiles;
  size_t off_seqs, off_tiles, off_pages, total_bytes;
};
void plan_conv(const std::vector<SeqSpan>& spans, size_t n_pages, ConvPlan* plan);

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
