// plan.cpp -- host-side validation and planning for libgdn (no HIP calls).
#include "plan.h"

#include <algorithm>
#include <cstring>
#include <unordered_set>

namespace gdn {

gdn_status check_layer(const gdn_layer* layer, LayerInfo* out) {
  if (!layer) return GDN_ERR_NULL_ARG;
  const gdn_layer& l = *layer;
  if (l.io_dtype != GDN_F32 && l.io_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  const int32_t act = l.conv_act & ~GDN_CONV_QK_L2NORM;
  if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_ERR_BAD_DTYPE;
  if (l.n_qk_heads <= 0 || l.n_v_heads <= 0) return GDN_ERR_BAD_SHAPE;
  // value heads share query/key heads in equal groups; a count that does not divide is
  // refused ("Hybrid linear attention (gated DeltaNet)", "Packed-core traces")
  if (l.n_v_heads % l.n_qk_heads != 0) return GDN_ERR_BAD_SHAPE;
  if (l.head_dim != 16 && l.head_dim != 32 && l.head_dim != 64 && l.head_dim != 128)
    return GDN_ERR_BAD_SHAPE;
  if (l.conv_width != 4) return GDN_ERR_BAD_SHAPE;
  if (l.n_v_heads > 4096 || l.n_qk_heads > 4096) return GDN_ERR_BAD_SHAPE;
  if (!(l.scale == l.scale)) return GDN_ERR_BAD_SHAPE;  // NaN scale
  if (out) {
    LayerInfo& L = *out;
    L.Hqk = l.n_qk_heads;
    L.Hv = l.n_v_heads;
    L.D = l.head_dim;
    L.W = l.conv_width;
    L.io = l.io_dtype;
    L.act = l.conv_act;
    L.scale = l.scale;
    L.io_bytes = l.io_dtype == GDN_BF16 ? 2 : 4;
    L.channels = (int64_t)(2 * l.n_qk_heads + l.n_v_heads) * l.head_dim;
    L.state_bytes = (int64_t)l.n_v_heads * l.head_dim * l.head_dim * 4;
    L.tail_bytes = (int64_t)(l.conv_width - 1) * L.channels * (int64_t)L.io_bytes;
    L.ckpt_bytes = (int64_t)align_up((size_t)(L.state_bytes + L.tail_bytes));
    // bf16 inputs: fp32 operands as two bf16 terms; fp32 inputs: three terms
    L.ntf = l.io_dtype == GDN_BF16 ? 2 : 3;
    L.nti = l.io_dtype == GDN_BF16 ? 1 : 3;
  }
  return GDN_OK;
}

gdn_status check_varlen(const gdn_varlen* v, std::vector<SeqSpan>* spans) {
  if (!v) return GDN_ERR_NULL_ARG;
  if (v->n_seqs < 0) return GDN_ERR_BAD_VARLEN;
  if (v->n_seqs > 0 && (!v->cu_seqlens || !v->start_pos)) return GDN_ERR_NULL_ARG;
  spans->clear();
  if (v->n_seqs == 0) return GDN_OK;
  if (v->cu_seqlens[0] != 0) return GDN_ERR_BAD_VARLEN;
  for (int s = 0; s < v->n_seqs; ++s) {
    int64_t r0 = v->cu_seqlens[s], r1 = v->cu_seqlens[s + 1];
    if (r1 < r0) return GDN_ERR_BAD_VARLEN;
    if (v->start_pos[s] < 0) return GDN_ERR_BAD_VARLEN;
    if (r1 - r0 > ((int64_t)1 << 40) || v->start_pos[s] > ((int64_t)1 << 50))
      return GDN_ERR_BAD_VARLEN;
    spans->push_back({r0, r1 - r0, v->start_pos[s]});
  }
  return GDN_OK;
}

gdn_status check_sources(const gdn_state_ref* refs, const std::vector<SeqSpan>& spans,
                         int32_t block) {
  if (spans.empty()) return GDN_OK;
  if (!refs) return GDN_ERR_NULL_ARG;
  for (size_t s = 0; s < spans.size(); ++s) {
    const gdn_state_ref& r = refs[s];
    if (!r.dst) return GDN_ERR_NULL_ARG;
    switch (r.src_kind) {
      case GDN_SRC_ZERO:
        // a fresh sequence starts at position 0; anything else would silently drop
        // the history ("Prefix caching on Gated DeltaNet hybrids", "Why hits were wrong")
        if (spans[s].p0 != 0) return GDN_ERR_OFF_BOUNDARY;
        break;
      case GDN_SRC_SLOT:
        if (!r.src) return GDN_ERR_NULL_ARG;
        if (spans[s].p0 == 0) return GDN_ERR_OFF_BOUNDARY;
        break;
      case GDN_SRC_CHECKPOINT:
        if (!r.src) return GDN_ERR_NULL_ARG;
        // a checkpoint exists only at a block boundary: resuming anywhere else is refused
        // ("Prefix caching on Gated DeltaNet hybrids", "The in-page layout": fail closed)
        if (block <= 0 || spans[s].p0 <= 0 || spans[s].p0 % block != 0)
          return GDN_ERR_OFF_BOUNDARY;
        if (((uintptr_t)r.src) % kAlign != 0) return GDN_ERR_PAGE_TOO_SMALL;
        break;
      default:
        return GDN_ERR_BAD_SOURCE;
    }
  }
  return GDN_OK;
}

int64_t count_boundaries(int64_t p0, int64_t len, int64_t block) {
  if (block <= 0 || len <= 0) return 0;
  return (p0 + len) / block - p0 / block;
}

gdn_status check_ckpt(const gdn_ckpt* ckpt, const LayerInfo& L, const std::vector<SeqSpan>& spans,
                      std::vector<int32_t>* pages, std::vector<int32_t>* page_begin) {
  pages->clear();
  page_begin->assign(spans.size() + 1, 0);
  if (!ckpt) return GDN_ERR_NULL_ARG;
  if (ckpt->block < 0) return GDN_ERR_BAD_SHAPE;
  if (ckpt->block == 0) return GDN_OK;
  int64_t total = 0;
  for (size_t s = 0; s < spans.size(); ++s) {
    (*page_begin)[s] = (int32_t)total;
    total += count_boundaries(spans[s].p0, spans[s].len, ckpt->block);
  }
  (*page_begin)[spans.size()] = (int32_t)total;
  if (total == 0) return GDN_OK;
  if (total > (1 << 30)) return GDN_ERR_CAPACITY;
  if (!ckpt->pool || !ckpt->page_ids) return GDN_ERR_NULL_ARG;
  if (ckpt->page_bytes < L.ckpt_bytes) return GDN_ERR_PAGE_TOO_SMALL;
  if (ckpt->page_bytes % (int64_t)kAlign != 0 || ((uintptr_t)ckpt->pool) % kAlign != 0)
    return GDN_ERR_PAGE_TOO_SMALL;
  if (ckpt->n_pages <= 0) return GDN_ERR_BAD_PAGE;
  std::unordered_set<int32_t> seen;
  pages->resize((size_t)total);
  for (int64_t i = 0; i < total; ++i) {
    int32_t p = ckpt->page_ids[i];
    if (p < -1 || (int64_t)p >= ckpt->n_pages) return GDN_ERR_BAD_PAGE;
    if (p >= 0 && !seen.insert(p).second) return GDN_ERR_BAD_PAGE;  // two boundaries, one page
    (*pages)[(size_t)i] = p;
  }
  return GDN_OK;
}

void chunk_grid(int64_t p0, int64_t len, int32_t block, std::vector<int64_t>* cuts) {
  cuts->clear();
  if (len <= 0) return;
  const int64_t end = p0 + len;
  cuts->push_back(p0);
  int64_t x = p0;
  while (true) {
    // next multiple of the chunk size and of the block strictly after x
    int64_t nc = (x / kChunk + 1) * kChunk;
    int64_t nxt = nc;
    if (block > 0) nxt = std::min(nxt, (x / block + 1) * (int64_t)block);
    if (nxt >= end) break;
    cuts->push_back(nxt);
    x = nxt;
  }
  cuts->push_back(end);
}

gdn_status plan_call(const LayerInfo& L, const std::vector<SeqSpan>& spans, int32_t block,
                     const std::vector<int32_t>* pages, const std::vector<int32_t>* page_begin,
                     bool prefill, CallPlan* plan) {
  if (block < 0 || block > (1 << 24)) return GDN_ERR_CAPACITY;
  plan->block = block;
  plan->lcm = grid_lcm((uint32_t)block);
  plan->seqs.assign(spans.size(), SeqEntry{});
  // one page per crossed boundary; without page ids (the factorize stage) the list holds
  // -1s, so that both prefill stages lay out the workspace the same way
  int64_t n_bound = 0;
  for (const SeqSpan& sp : spans) n_bound += count_boundaries(sp.p0, sp.len, block);
  if (n_bound > (1 << 30)) return GDN_ERR_CAPACITY;
  if (pages && (int64_t)pages->size() != n_bound) return GDN_ERR_BAD_PAGE;
  plan->pages = pages ? *pages : std::vector<int32_t>((size_t)n_bound, -1);
  int64_t units = 0, bound = 0;
  for (size_t s = 0; s < spans.size(); ++s) {
    const SeqSpan& sp = spans[s];
    if (sp.p0 + sp.len >= kMaxPosition || sp.row0 + sp.len > ((int64_t)1 << 40)) return GDN_ERR_CAPACITY;
    SeqEntry& e = plan->seqs[s];
    e.row0 = sp.row0;
    e.p0 = (int32_t)sp.p0;
    e.len = (int32_t)sp.len;
    e.unit0 = (int32_t)units;
    e.n_units = (int32_t)(prefill ? chunk_count((uint32_t)sp.p0, (uint32_t)sp.len, (uint32_t)block, plan->lcm)
                                  : tile_count((uint32_t)sp.len));
    e.page0 = page_begin ? (*page_begin)[s] : (int32_t)bound;
    bound += count_boundaries(sp.p0, sp.len, block);
    units += e.n_units;
    if (units > INT32_MAX / 2) return GDN_ERR_CAPACITY;
  }
  plan->n_units = (int32_t)units;
  plan->staged = spans.size() > (size_t)kInlineSeqs || plan->pages.size() > (size_t)kInlinePages;
  plan->off_pages = align_up(spans.size() * sizeof(SeqEntry));
  plan->off_unit_seq = plan->off_pages + align_up(plan->pages.size() * sizeof(int32_t));
  plan->table_bytes = plan->staged ? plan->off_unit_seq + align_up((size_t)units * sizeof(int32_t)) : 0;
  // the workspace always reserves the staged table's room, so that its size does not
  // depend on how the table travels
  const size_t table_room = plan->off_unit_seq + align_up((size_t)units * sizeof(int32_t));
  plan->off_factors = table_room;
  plan->factor_stride = prefill ? factor_record_bytes(L.ntf, L.nti, L.D) : 0;
  plan->total_bytes = plan->off_factors + plan->factor_stride * (size_t)units * (size_t)L.Hv;
  if (plan->total_bytes == 0) plan->total_bytes = kAlign;
  return GDN_OK;
}

void staged_table(const CallPlan& plan, uint8_t* out) {
  std::memset(out, 0, plan.table_bytes);
  std::memcpy(out, plan.seqs.data(), plan.seqs.size() * sizeof(SeqEntry));
  if (!plan.pages.empty()) std::memcpy(out + plan.off_pages, plan.pages.data(), plan.pages.size() * sizeof(int32_t));
  int32_t* us = reinterpret_cast<int32_t*>(out + plan.off_unit_seq);
  for (size_t s = 0; s < plan.seqs.size(); ++s)
    for (int32_t u = 0; u < plan.seqs[s].n_units; ++u) us[plan.seqs[s].unit0 + u] = (int32_t)s;
}

void fill_call_table(const CallPlan& plan, const void* ws, CallTable* t) {
  std::memset(t, 0, sizeof(CallTable));
  t->n_seqs = (int32_t)plan.seqs.size();
  t->n_pages = (int32_t)plan.pages.size();
  t->n_units = plan.n_units;
  t->block = plan.block;
  t->lcm = plan.lcm;
  if (plan.staged) {
    const uint8_t* w = static_cast<const uint8_t*>(ws);
    t->seqs = reinterpret_cast<const SeqEntry*>(w);
    t->pages = reinterpret_cast<const int32_t*>(w + plan.off_pages);
    t->unit_seq = reinterpret_cast<const int32_t*>(w + plan.off_unit_seq);
  } else {
    if (!plan.seqs.empty()) std::memcpy(t->inl_seqs, plan.seqs.data(), plan.seqs.size() * sizeof(SeqEntry));
    if (!plan.pages.empty()) std::memcpy(t->inl_pages, plan.pages.data(), plan.pages.size() * sizeof(int32_t));
  }
}

}  // namespace gdn
