// gdn_api.cpp -- the extern "C" entry points of libgdn (see include/gdn.h).
//
// Each call validates everything it can on the host (plan.cpp) before anything is
// enqueued, uploads the small per-call tables (chunk grid, per-sequence pointers,
// checkpoint page ids) into the caller's workspace, and launches the kernels.
//
// Table uploads go through one pinned host staging ring per process (allocated on
// first use and kept): a table is copied into the ring and an asynchronous copy is
// enqueued on the caller's stream, followed by an event; a ring region is reused only
// after the event that last covered it has completed.  This keeps every call
// asynchronous with respect to the host.  The events skip the system-scope fence: they
// only tell the host that a copy has finished reading the ring, and the fence's cache
// writeback and invalidation would delay the kernel that follows and start it with cold
// caches.  Completed events are kept and reused.
#include <hip/hip_runtime.h>

#include <cstring>
#include <deque>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "kernels.h"
#include "plan.h"

using namespace gdn;

namespace {

constexpr size_t kRingBytes = (size_t)32 << 20;

struct StagingRing {
  std::mutex mu;
  uint8_t* base = nullptr;
  size_t head = 0;
  struct Seg {
    size_t off, len;
    hipEvent_t ev;
  };
  std::deque<Seg> live;
  std::vector<hipEvent_t> spare;
};
StagingRing g_ring;

hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_ring.mu);
  if (bytes > kRingBytes) {
    // larger than the whole ring: a plain copy that completes before the call returns
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(stream);
  }
  if (!g_ring.base) {
    void* p = nullptr;
    hipError_t e = hipHostMalloc(&p, kRingBytes, hipHostMallocPortable);
    if (e != hipSuccess) return e;
    g_ring.base = static_cast<uint8_t*>(p);
    g_ring.head = 0;
  }
  size_t off = align_up(g_ring.head);
  if (off + bytes > kRingBytes) off = 0;
  for (auto it = g_ring.live.begin(); it != g_ring.live.end();) {
    const bool overlap = !(it->off + it->len <= off || off + bytes <= it->off);
    if (overlap) {
      hipError_t e = hipEventSynchronize(it->ev);
      if (e != hipSuccess) return e;
    } else if (hipEventQuery(it->ev) != hipSuccess) {
      ++it;
      continue;
    }
    g_ring.spare.push_back(it->ev);
    it = g_ring.live.erase(it);
  }
  std::memcpy(g_ring.base + off, src, bytes);
  hipError_t e = hipMemcpyAsync(dst, g_ring.base + off, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  hipEvent_t ev;
  if (!g_ring.spare.empty()) {
    ev = g_ring.spare.back();
    g_ring.spare.pop_back();
  } else {
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) return e;
  }
  e = hipEventRecord(ev, stream);
  if (e != hipSuccess) {
    g_ring.spare.push_back(ev);
    return e;
  }
  g_ring.live.push_back({off, bytes, ev});
  g_ring.head = off + bytes;
  return hipSuccess;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p) % a == 0; }

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Checks shared by the prefill stages.
gdn_status check_qkv(const LayerInfo& L, const void* q, const void* k, const void* v, int64_t qk_stride,
                     int64_t v_stride, bool need_q, bool need_v) {
  const int64_t vec = 16 / (int64_t)L.io_bytes;
  if (!k || (need_q && !q) || (need_v && !v)) return GDN_ERR_NULL_ARG;
  if (!aligned(k, 16) || (need_q && !aligned(q, 16)) || (need_v && !aligned(v, 16))) return GDN_ERR_BAD_SHAPE;
  if (qk_stride < (int64_t)L.Hqk * L.D || qk_stride % vec != 0) return GDN_ERR_BAD_SHAPE;
  if (need_v && (v_stride < (int64_t)L.Hv * L.D || v_stride % vec != 0)) return GDN_ERR_BAD_SHAPE;
  // fp32 inputs enter the matrix products as three bf16 terms; the registers of the
  // chunk kernels hold them for head_dim <= 64
  if (L.io == GDN_F32 && L.D > 64) return GDN_ERR_BAD_SHAPE;
  // the scan addresses one chunk of rows with 32-bit byte offsets
  const int64_t lim = (int64_t)INT32_MAX / kChunk;
  if (qk_stride * (int64_t)L.io_bytes > lim || (need_v && v_stride * (int64_t)L.io_bytes > lim) ||
      (int64_t)L.Hv * L.D * 4 > lim)
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

struct PrefillPrep {
  LayerInfo L;
  std::vector<SeqSpan> spans;
  std::vector<int32_t> pages, page_begin;
  PrefillPlan plan;
};

gdn_status prep_prefill(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block, const gdn_ckpt* ckpt,
                        PrefillPrep* P) {
  gdn_status s = check_layer(layer, &P->L);
  if (s != GDN_OK) return s;
  s = check_varlen(varlen, &P->spans);
  if (s != GDN_OK) return s;
  if (block < 0) return GDN_ERR_BAD_SHAPE;
  if (ckpt) {
    s = check_ckpt(ckpt, P->L, P->spans, &P->pages, &P->page_begin);
    if (s != GDN_OK) return s;
  }
  plan_prefill(P->L, P->spans, block, ckpt ? &P->pages : nullptr, ckpt ? &P->page_begin : nullptr, &P->plan);
  if (P->plan.chunks.size() > (size_t)INT32_MAX) return GDN_ERR_CAPACITY;
  return GDN_OK;
}

gdn_status check_workspace(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return GDN_ERR_WORKSPACE;
  if (!aligned(ws, kAlign) || ws_bytes < need) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

template <typename IO>
gdn_status do_factorize(const PrefillPrep& P, hipStream_t stream, const void* q, const void* k, int64_t qk_stride,
                        const float* a, const float* b, void* ws) {
  FactorizeArgs<IO> fa;
  fa.chunks = reinterpret_cast<const ChunkDesc*>(static_cast<uint8_t*>(ws) + P.plan.off_chunks);
  fa.q = static_cast<const IO*>(q);
  fa.k = static_cast<const IO*>(k);
  fa.qk_stride = qk_stride;
  fa.a = a;
  fa.b = b;
  fa.factors = static_cast<uint8_t*>(ws) + P.plan.off_factors;
  fa.factor_stride = P.plan.factor_stride;
  fa.n_chunks = (int32_t)P.plan.chunks.size();
  fa.Hv = P.L.Hv;
  fa.group = P.L.Hv / P.L.Hqk;
  fa.scale = P.L.scale;
  return hip_status(launch_factorize(fa, P.L.D, fa.n_chunks, stream));
}

template <typename IO>
gdn_status do_scan(const PrefillPrep& P, hipStream_t stream, const void* q, const void* k, const void* v,
                   int64_t qk_stride, int64_t v_stride, const gdn_ckpt* ckpt, float* o, void* ws) {
  ScanArgs<IO> sa;
  uint8_t* w = static_cast<uint8_t*>(ws);
  sa.chunks = reinterpret_cast<const ChunkDesc*>(w + P.plan.off_chunks);
  sa.seqs = reinterpret_cast<const ScanSeq*>(w + P.plan.off_seqs);
  sa.q = static_cast<const IO*>(q);
  sa.k = static_cast<const IO*>(k);
  sa.v = static_cast<const IO*>(v);
  sa.qk_stride = qk_stride;
  sa.v_stride = v_stride;
  sa.factors = w + P.plan.off_factors;
  sa.factor_stride = P.plan.factor_stride;
  sa.n_chunks = (int32_t)P.plan.chunks.size();
  sa.n_seqs = (int32_t)P.spans.size();
  sa.Hv = P.L.Hv;
  sa.group = P.L.Hv / P.L.Hqk;
  sa.o = o;
  sa.ckpt_pool = static_cast<uint8_t*>(ckpt->pool);
  sa.page_bytes = (size_t)ckpt->page_bytes;
  return hip_status(launch_scan(sa, P.L.D, stream));
}

// Host image of the chunk table and, when states != null, of the sequence table.
std::vector<uint8_t> prefill_tables(const PrefillPrep& P, const gdn_state_ref* states, bool with_seqs) {
  const size_t bytes = with_seqs ? P.plan.off_factors : P.plan.off_seqs;
  std::vector<uint8_t> buf(bytes, 0);
  if (!P.plan.chunks.empty())
    std::memcpy(buf.data() + P.plan.off_chunks, P.plan.chunks.data(), P.plan.chunks.size() * sizeof(ChunkDesc));
  if (with_seqs) {
    ScanSeq* sq = reinterpret_cast<ScanSeq*>(buf.data() + P.plan.off_seqs);
    for (size_t s = 0; s < P.spans.size(); ++s) {
      const gdn_state_ref& r = states[s];
      sq[s].src = r.src_kind == GDN_SRC_ZERO ? nullptr : static_cast<const float*>(r.src);
      sq[s].dst = static_cast<float*>(r.dst);
      sq[s].chunk_begin = P.plan.seq_chunk_begin[s];
      sq[s].chunk_end = P.plan.seq_chunk_begin[s + 1];
      sq[s].pad0 = sq[s].pad1 = 0;
    }
  }
  return buf;
}

gdn_status check_states(const PrefillPrep& P, const gdn_state_ref* states, int32_t block) {
  gdn_status s = check_sources(states, P.spans, block);
  if (s != GDN_OK) return s;
  for (size_t i = 0; i < P.spans.size(); ++i) {
    if (states[i].src_kind != GDN_SRC_ZERO && !aligned(states[i].src, 16)) return GDN_ERR_BAD_SHAPE;
    if (!aligned(states[i].dst, 16)) return GDN_ERR_BAD_SHAPE;
  }
  return GDN_OK;
}

// Decode launch shared by the dense and the mixed-batch entry points.
gdn_status decode_rows(const LayerInfo& L, hipStream_t stream, int32_t n_req, int64_t n_rows, const void* q,
                       const void* k, const void* v, int64_t qk_stride, int64_t v_stride, const float* a,
                       const float* b, float* state_pool, int64_t n_slots, const int32_t* slot_ids,
                       const int32_t* rows, float* o, int32_t* status) {
  auto fill = [&](auto& da, auto tag) {
    using IO = decltype(tag);
    da.q = static_cast<const IO*>(q);
    da.k = static_cast<const IO*>(k);
    da.v = static_cast<const IO*>(v);
    da.a = a;
    da.b = b;
    da.state_pool = state_pool;
    da.slot_ids = slot_ids;
    da.o = o;
    da.status = status;
    da.n_slots = n_slots;
    da.Hqk = L.Hqk;
    da.Hv = L.Hv;
    da.group = L.Hv / L.Hqk;
    da.scale = L.scale;
    da.rows = rows;
    da.n_rows = n_rows;
    da.qk_stride = qk_stride;
    da.v_stride = v_stride;
  };
  if (L.io == GDN_BF16) {
    DecodeArgs<bf16_bits> da;
    fill(da, bf16_bits{});
    return hip_status(launch_decode(da, L.D, n_req, stream));
  }
  DecodeArgs<float> da;
  fill(da, float{});
  return hip_status(launch_decode(da, L.D, n_req, stream));
}

}  // namespace

extern "C" {

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_ARG: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "unsupported shape, stride or alignment";
    case GDN_ERR_BAD_DTYPE: return "unknown dtype or activation";
    case GDN_ERR_BAD_VARLEN: return "bad cu_seqlens or start_pos";
    case GDN_ERR_OFF_BOUNDARY: return "state source inconsistent with the start position";
    case GDN_ERR_PAGE_TOO_SMALL: return "checkpoint page too small or misaligned";
    case GDN_ERR_BAD_PAGE: return "checkpoint page id out of range or reused";
    case GDN_ERR_CAPACITY: return "count exceeds what the call supports";
    case GDN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case GDN_ERR_HIP: return "HIP runtime error";
    case GDN_ERR_BAD_SOURCE: return "unknown state source kind";
  }
  return "unknown status";
}

int64_t gdn_state_bytes(const gdn_layer* layer) {
  LayerInfo L;
  return check_layer(layer, &L) == GDN_OK ? L.state_bytes : -1;
}
int64_t gdn_conv_tail_bytes(const gdn_layer* layer) {
  LayerInfo L;
  return check_layer(layer, &L) == GDN_OK ? L.tail_bytes : -1;
}
int64_t gdn_checkpoint_bytes(const gdn_layer* layer) {
  LayerInfo L;
  return check_layer(layer, &L) == GDN_OK ? L.ckpt_bytes : -1;
}
int64_t gdn_conv_channels(const gdn_layer* layer) {
  LayerInfo L;
  return check_layer(layer, &L) == GDN_OK ? L.channels : -1;
}

int64_t gdn_cached_prefix_tokens(int64_t shared, int64_t block) {
  if (block <= 0 || shared <= 0) return 0;
  const int64_t full = shared / block;
  return full >= 1 ? (full - 1) * block : 0;
}
int64_t gdn_floor_chunk(int64_t budget, int64_t block) {
  if (budget <= 0) return 0;
  if (block <= 0) return budget;
  return budget / block * block;
}
int64_t gdn_count_boundaries(int64_t start_pos, int64_t n_tokens, int64_t block) {
  if (start_pos < 0) return 0;
  return count_boundaries(start_pos, n_tokens, block);
}
int64_t gdn_block_size_for_state(int64_t state_bytes, int64_t attn_bytes_per_token, int64_t alignment) {
  if (state_bytes <= 0 || attn_bytes_per_token <= 0 || alignment <= 0) return -1;
  const int64_t per_align = alignment * attn_bytes_per_token;
  return alignment * ((state_bytes + per_align - 1) / per_align);
}

int64_t gdn_prefill_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  PrefillPrep P;
  if (prep_prefill(layer, varlen, block, nullptr, &P) != GDN_OK) return -1;
  return (int64_t)P.plan.total_bytes;
}

int64_t gdn_conv_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  LayerInfo L;
  std::vector<SeqSpan> spans;
  if (check_layer(layer, &L) != GDN_OK || check_varlen(varlen, &spans) != GDN_OK || block < 0) return -1;
  size_t n_pages = 0;
  for (auto& sp : spans) n_pages += (size_t)count_boundaries(sp.p0, sp.len, block);
  ConvPlan plan;
  plan_conv(spans, n_pages, &plan);
  return (int64_t)plan.total_bytes;
}

gdn_status gdn_prefill_factorize(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                                 const void* q, const void* k, int64_t qk_stride, const float* a, const float* b,
                                 int32_t block, void* workspace, size_t workspace_bytes) {
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, block, nullptr, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, nullptr, qk_stride, 0, true, false);
  if (s != GDN_OK) return s;
  if (!P.plan.chunks.empty() && (!a || !b)) return GDN_ERR_NULL_ARG;
  s = check_workspace(workspace, workspace_bytes, P.plan.total_bytes);
  if (s != GDN_OK) return s;
  std::vector<uint8_t> tab = prefill_tables(P, nullptr, false);
  s = hip_status(upload(workspace, tab.data(), tab.size(), stream));
  if (s != GDN_OK) return s;
  return P.L.io == GDN_BF16 ? do_factorize<bf16_bits>(P, stream, q, k, qk_stride, a, b, workspace)
                            : do_factorize<float>(P, stream, q, k, qk_stride, a, b, workspace);
}

gdn_status gdn_prefill_scan(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* q,
                            const void* k, const void* v, int64_t qk_stride, int64_t v_stride,
                            const gdn_state_ref* states, const gdn_ckpt* ckpt, float* o, void* workspace,
                            size_t workspace_bytes) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, ckpt->block, ckpt, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, v, qk_stride, v_stride, true, true);
  if (s != GDN_OK) return s;
  if (!o && !P.plan.chunks.empty()) return GDN_ERR_NULL_ARG;
  s = check_states(P, states, ckpt->block);
  if (s != GDN_OK) return s;
  s = check_workspace(workspace, workspace_bytes, P.plan.total_bytes);
  if (s != GDN_OK) return s;
  std::vector<uint8_t> tab = prefill_tables(P, states, true);
  s = hip_status(upload(workspace, tab.data(), tab.size(), stream));
  if (s != GDN_OK) return s;
  return P.L.io == GDN_BF16 ? do_scan<bf16_bits>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace)
                            : do_scan<float>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace);
}

gdn_status gdn_chunk_prefill(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* q,
                             const void* k, const void* v, int64_t qk_stride, int64_t v_stride, const float* a,
                             const float* b, const gdn_state_ref* states, const gdn_ckpt* ckpt, float* o,
                             void* workspace, size_t workspace_bytes) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, ckpt->block, ckpt, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, v, qk_stride, v_stride, true, true);
  if (s != GDN_OK) return s;
  if (!P.plan.chunks.empty() && (!a || !b || !o)) return GDN_ERR_NULL_ARG;
  s = check_states(P, states, ckpt->block);
  if (s != GDN_OK) return s;
  s = check_workspace(workspace, workspace_bytes, P.plan.total_bytes);
  if (s != GDN_OK) return s;
  std::vector<uint8_t> tab = prefill_tables(P, states, true);
  s = hip_status(upload(workspace, tab.data(), tab.size(), stream));
  if (s != GDN_OK) return s;
  if (P.L.io == GDN_BF16) {
    s = do_factorize<bf16_bits>(P, stream, q, k, qk_stride, a, b, workspace);
    if (s != GDN_OK) return s;
    return do_scan<bf16_bits>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace);
  }
  s = do_factorize<float>(P, stream, q, k, qk_stride, a, b, workspace);
  if (s != GDN_OK) return s;
  return do_scan<float>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace);
}

gdn_status gdn_conv_update(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* x,
                           const void* w, const gdn_state_ref* tails, const gdn_ckpt* ckpt, void* y,
                           void* workspace, size_t workspace_bytes) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  std::vector<SeqSpan> spans;
  s = check_varlen(varlen, &spans);
  if (s != GDN_OK) return s;
  if (!ckpt) return GDN_ERR_NULL_ARG;
  std::vector<int32_t> pages, page_begin;
  s = check_ckpt(ckpt, L, spans, &pages, &page_begin);
  if (s != GDN_OK) return s;
  s = check_sources(tails, spans, ckpt->block);
  if (s != GDN_OK) return s;
  int64_t total_rows = spans.empty() ? 0 : spans.back().row0 + spans.back().len;
  if (total_rows > 0 && (!x || !y)) return GDN_ERR_NULL_ARG;
  if (!w && !spans.empty()) return GDN_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 16)) return GDN_ERR_BAD_SHAPE;
  for (size_t i = 0; i < spans.size(); ++i) {
    if (tails[i].src_kind != GDN_SRC_ZERO && !aligned(tails[i].src, 16)) return GDN_ERR_BAD_SHAPE;
    if (!aligned(tails[i].dst, 16)) return GDN_ERR_BAD_SHAPE;
  }
  ConvPlan plan;
  plan_conv(spans, pages.size(), &plan);
  const std::vector<ConvTile>& tiles = plan.tiles;
  const size_t off_tiles = plan.off_tiles, off_pages = plan.off_pages, need = plan.total_bytes;
  if (tiles.size() > (size_t)INT32_MAX) return GDN_ERR_CAPACITY;
  s = check_workspace(workspace, workspace_bytes, need);
  if (s != GDN_OK) return s;
  if (tiles.empty()) return GDN_OK;
  std::vector<uint8_t> buf(need, 0);
  ConvSeq* cs = reinterpret_cast<ConvSeq*>(buf.data());
  for (size_t i = 0; i < spans.size(); ++i) {
    const gdn_state_ref& r = tails[i];
    const uint8_t* src = static_cast<const uint8_t*>(r.src);
    if (r.src_kind == GDN_SRC_ZERO) src = nullptr;
    if (r.src_kind == GDN_SRC_CHECKPOINT) src += L.state_bytes;  // tail region of the page
    cs[i].src_tail = src;
    cs[i].dst_tail = r.dst;
    cs[i].row0 = spans[i].row0;
    cs[i].p0 = spans[i].p0;
    cs[i].len = spans[i].len;
    cs[i].page_begin = page_begin[i];
    cs[i].pad = 0;
  }
  std::memcpy(buf.data() + off_tiles, tiles.data(), tiles.size() * sizeof(ConvTile));
  if (!pages.empty()) std::memcpy(buf.data() + off_pages, pages.data(), pages.size() * sizeof(int32_t));
  s = hip_status(upload(workspace, buf.data(), buf.size(), stream));
  if (s != GDN_OK) return s;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (L.io == GDN_BF16) {
    ConvArgs<bf16_bits> ca;
    ca.seqs = reinterpret_cast<const ConvSeq*>(ws);
    ca.tiles = reinterpret_cast<const ConvTile*>(ws + off_tiles);
    ca.pages = reinterpret_cast<const int32_t*>(ws + off_pages);
    ca.x = static_cast<const bf16_bits*>(x);
    ca.w = static_cast<const bf16_bits*>(w);
    ca.y = static_cast<bf16_bits*>(y);
    ca.ckpt_pool = static_cast<uint8_t*>(ckpt->pool);
    ca.page_bytes = (size_t)ckpt->page_bytes;
    ca.tail_offset = (size_t)L.state_bytes;
    ca.channels = L.channels;
    ca.qk_channels = 2 * (int64_t)L.Hqk * L.D;
    ca.head_dim = L.D;
    ca.block = ckpt->block;
    ca.act = L.act;
    return hip_status(launch_conv(ca, (int)tiles.size(), stream));
  }
  ConvArgs<float> ca;
  ca.seqs = reinterpret_cast<const ConvSeq*>(ws);
  ca.tiles = reinterpret_cast<const ConvTile*>(ws + off_tiles);
  ca.pages = reinterpret_cast<const int32_t*>(ws + off_pages);
  ca.x = static_cast<const float*>(x);
  ca.w = static_cast<const float*>(w);
  ca.y = static_cast<float*>(y);
  ca.ckpt_pool = static_cast<uint8_t*>(ckpt->pool);
  ca.page_bytes = (size_t)ckpt->page_bytes;
  ca.tail_offset = (size_t)L.state_bytes;
  ca.channels = L.channels;
  ca.qk_channels = 2 * (int64_t)L.Hqk * L.D;
  ca.head_dim = L.D;
  ca.block = ckpt->block;
  ca.act = L.act;
  return hip_status(launch_conv(ca, (int)tiles.size(), stream));
}

gdn_status gdn_decode_step(const gdn_layer* layer, hipStream_t stream, int32_t n_req, const void* q, const void* k,
                           const void* v, const float* a, const float* b, float* state_pool, int64_t n_slots,
                           const int32_t* slot_ids, float* o, int32_t* status) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_req < 0 || n_slots < 0) return GDN_ERR_BAD_SHAPE;
  if (n_req == 0) return GDN_OK;
  if (!q || !k || !v || !a || !b || !state_pool || !slot_ids || !o) return GDN_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state_pool, 16)) return GDN_ERR_BAD_SHAPE;
  if (L.io == GDN_F32 && (!aligned(q, 16) || !aligned(k, 16))) return GDN_ERR_BAD_SHAPE;
  if (n_req > 65535) return GDN_ERR_CAPACITY;
  return decode_rows(L, stream, n_req, n_req, q, k, v, (int64_t)L.Hqk * L.D, (int64_t)L.Hv * L.D, a, b,
                     state_pool, n_slots, slot_ids, nullptr, o, status);
}

gdn_status gdn_decode_mixed(const gdn_layer* layer, hipStream_t stream, int32_t n_req, int64_t n_rows,
                            const void* q, const void* k, const void* v, int64_t qk_stride, int64_t v_stride,
                            const float* a, const float* b, float* state_pool, int64_t n_slots,
                            const int32_t* slot_ids, const int32_t* rows, float* o, int32_t* status) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_req < 0 || n_slots < 0 || n_rows < 0) return GDN_ERR_BAD_SHAPE;
  if (n_req == 0) return GDN_OK;
  if (!q || !k || !v || !a || !b || !state_pool || !slot_ids || !rows || !o) return GDN_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state_pool, 16)) return GDN_ERR_BAD_SHAPE;
  if (qk_stride < (int64_t)L.Hqk * L.D || v_stride < (int64_t)L.Hv * L.D) return GDN_ERR_BAD_SHAPE;
  if (n_req > 65535) return GDN_ERR_CAPACITY;
  return decode_rows(L, stream, n_req, n_rows, q, k, v, qk_stride, v_stride, a, b, state_pool, n_slots, slot_ids,
                     rows, o, status);
}

gdn_status gdn_replay_flush(const gdn_layer* layer, hipStream_t stream, int32_t n_req, float* state_pool,
                            int64_t n_slots, const int32_t* slot_ids, const void* buf_k, const void* buf_v,
                            const float* buf_a, const float* buf_b, int32_t buf_rows, const int32_t* n_accepted,
                            int32_t* status) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_req < 0 || n_slots < 0) return GDN_ERR_BAD_SHAPE;
  if (buf_rows < 1 || buf_rows > kMaxBufRows) return GDN_ERR_CAPACITY;
  if (L.io == GDN_F32 && L.D > 64) return GDN_ERR_BAD_SHAPE;
  if (n_req == 0) return GDN_OK;
  if (!state_pool || !slot_ids || !buf_k || !buf_v || !buf_a || !buf_b || !n_accepted) return GDN_ERR_NULL_ARG;
  if (!aligned(state_pool, 16) || !aligned(buf_k, 16) || !aligned(buf_v, 16)) return GDN_ERR_BAD_SHAPE;
  if (n_req > 65535) return GDN_ERR_CAPACITY;
  if (L.io == GDN_BF16) {
    FlushArgs<bf16_bits> fa{state_pool, slot_ids, n_accepted, static_cast<const bf16_bits*>(buf_k),
                            static_cast<const bf16_bits*>(buf_v), buf_a, buf_b, status, n_slots, buf_rows, L.Hqk,
                            L.Hv, L.Hv / L.Hqk};
    return hip_status(launch_flush(fa, L.D, n_req, stream));
  }
  FlushArgs<float> fa{state_pool, slot_ids, n_accepted, static_cast<const float*>(buf_k),
                      static_cast<const float*>(buf_v), buf_a, buf_b, status, n_slots, buf_rows, L.Hqk, L.Hv,
                      L.Hv / L.Hqk};
  return hip_status(launch_flush(fa, L.D, n_req, stream));
}

gdn_status gdn_gates(const gdn_layer* layer, hipStream_t stream, int64_t n_tokens, const void* ba,
                     int64_t ba_stride, const float* A_log, const void* dt_bias, float* a, float* b) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_tokens < 0 || ba_stride < 2 * (int64_t)L.Hv) return GDN_ERR_BAD_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  if (!ba || !A_log || !dt_bias || !a || !b) return GDN_ERR_NULL_ARG;
  if (L.io == GDN_BF16) {
    GateArgs<bf16_bits> ga{static_cast<const bf16_bits*>(ba), A_log, static_cast<const bf16_bits*>(dt_bias), a, b,
                           n_tokens, ba_stride, L.Hv};
    return hip_status(launch_gates(ga, stream));
  }
  GateArgs<float> ga{static_cast<const float*>(ba), A_log, static_cast<const float*>(dt_bias), a, b, n_tokens,
                     ba_stride, L.Hv};
  return hip_status(launch_gates(ga, stream));
}

gdn_status gdn_gated_norm(const gdn_layer* layer, hipStream_t stream, int64_t n_tokens, const float* o,
                          const void* z, int64_t z_stride, const void* weight, float eps, void* out) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  // z rows are read 16 bytes at a time: a stride of whole 8-element groups
  if (n_tokens < 0 || z_stride < (int64_t)L.Hv * L.D || z_stride % 8 != 0 || !(eps >= 0.f)) return GDN_ERR_BAD_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  if (!o || !z || !weight || !out) return GDN_ERR_NULL_ARG;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(weight, 16) || !aligned(out, 16)) return GDN_ERR_BAD_SHAPE;
  if (L.io == GDN_BF16) {
    NormArgs<bf16_bits> na{o, static_cast<const bf16_bits*>(z), static_cast<const bf16_bits*>(weight),
                           static_cast<bf16_bits*>(out), n_tokens * L.Hv, z_stride, L.Hv, eps};
    return hip_status(launch_gated_norm(na, L.D, stream));
  }
  NormArgs<float> na{o, static_cast<const float*>(z), static_cast<const float*>(weight), static_cast<float*>(out),
                     n_tokens * L.Hv, z_stride, L.Hv, eps};
  return hip_status(launch_gated_norm(na, L.D, stream));
}

gdn_status gdn_replay_forward(const gdn_layer* layer, hipStream_t stream, int32_t n_req, const float* state_pool,
                              int64_t n_slots, const int32_t* slot_ids, const void* buf_k, const void* buf_v,
                              const float* buf_a, const float* buf_b, int32_t buf_rows, const int32_t* n_logged,
                              const int32_t* n_new, const void* q_new, int32_t max_new, float* o, int32_t* status) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_req < 0 || n_slots < 0 || max_new < 0) return GDN_ERR_BAD_SHAPE;
  if (buf_rows < 1 || buf_rows > kMaxBufRows) return GDN_ERR_CAPACITY;
  if (L.io == GDN_F32 && L.D > 64) return GDN_ERR_BAD_SHAPE;
  if (n_req == 0 || max_new == 0) return GDN_OK;
  if (!state_pool || !slot_ids || !buf_k || !buf_v || !buf_a || !buf_b || !n_logged || !n_new || !q_new || !o)
    return GDN_ERR_NULL_ARG;
  if (!aligned(state_pool, 16) || !aligned(buf_k, 16) || !aligned(buf_v, 16) || !aligned(q_new, 16))
    return GDN_ERR_BAD_SHAPE;
  if (n_req > 65535) return GDN_ERR_CAPACITY;
  const int ct = buf_rows <= 32 ? 32 : 64;
  auto fill = [&](auto& ra, auto tag) {
    using IO = decltype(tag);
    ra.state_pool = state_pool;
    ra.slot_ids = slot_ids;
    ra.n_logged = n_logged;
    ra.n_new = n_new;
    ra.buf_k = static_cast<const IO*>(buf_k);
    ra.buf_v = static_cast<const IO*>(buf_v);
    ra.buf_a = buf_a;
    ra.buf_b = buf_b;
    ra.q_new = static_cast<const IO*>(q_new);
    ra.o = o;
    ra.status = status;
    ra.n_slots = n_slots;
    ra.buf_rows = buf_rows;
    ra.max_new = max_new;
    ra.Hqk = L.Hqk;
    ra.Hv = L.Hv;
    ra.group = L.Hv / L.Hqk;
    ra.scale = L.scale;
  };
  if (L.io == GDN_BF16) {
    ReplayArgs<bf16_bits> ra;
    fill(ra, bf16_bits{});
    return hip_status(launch_replay(ra, L.D, n_req, ct, stream));
  }
  ReplayArgs<float> ra;
  fill(ra, float{});
  return hip_status(launch_replay(ra, L.D, n_req, ct, stream));
}

}  // extern "C"
