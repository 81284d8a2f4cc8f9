// gdn_api.cpp -- the extern "C" entry points of libgdn (see include/gdn.h).
//
// Each call validates everything it can on the host (plan.cpp) before anything is
// enqueued, then launches its kernels.  The prefill and conv kernels take the call's
// table -- one entry per sequence plus the checkpoint page ids -- inside their kernel
// arguments; a table too large for that is written into the caller's pinned staging
// buffer and copied from there into the caller's workspace on the call's stream.  The
// library holds no memory and no state between calls, so calls on different streams
// never wait for each other.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <vector>

#include "../../include/gdn.h"
#include "kernels.h"
#include "plan.h"

using namespace gdn;

// Device scratch of gdn_chunk_prefill_noalloc (the factor records of one call), for
// callers that cannot allocate: one array per device, held from the library's load on
// that device until the process ends.  Host code never uses this name as an address:
// it is a host-side stand-in, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each device, looked up once per device (with that
// device current) on the entry point's first call there.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

gdn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return GDN_OK;
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
  CallPlan plan;
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
  return plan_call(P->L, P->spans, block, ckpt ? &P->pages : nullptr, ckpt ? &P->page_begin : nullptr, true,
                   &P->plan);
}

gdn_status check_workspace(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return GDN_ERR_WORKSPACE;
  if (!aligned(ws, kAlign) || ws_bytes < need) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

gdn_status check_staging(const CallPlan& plan, const gdn_staging* staging) {
  if (!plan.staged) return GDN_OK;
  if (!staging || !staging->host || staging->bytes < plan.table_bytes) return GDN_ERR_STAGING;
  return GDN_OK;
}

// A staged table: written into the caller's staging buffer, then copied on the stream
// into the table region at the start of the workspace.  The caller keeps the staging
// buffer untouched until the stream has passed this copy.
gdn_status stage_table(const CallPlan& plan, const gdn_staging* staging, void* ws, hipStream_t stream) {
  if (!plan.staged) return GDN_OK;
  staged_table(plan, static_cast<uint8_t*>(staging->host));
  return hip_status(hipMemcpyAsync(ws, staging->host, plan.table_bytes, hipMemcpyHostToDevice, stream));
}

template <typename IO>
gdn_status do_factorize(const PrefillPrep& P, hipStream_t stream, const void* q, const void* k, int64_t qk_stride,
                        const float* a, const float* b, void* ws) {
  FactorizeArgs<IO> fa;
  fill_call_table(P.plan, ws, &fa.tab);
  fa.q = static_cast<const IO*>(q);
  fa.k = static_cast<const IO*>(k);
  fa.qk_stride = qk_stride;
  fa.a = a;
  fa.b = b;
  fa.factors = static_cast<uint8_t*>(ws) + P.plan.off_factors;
  fa.factor_stride = P.plan.factor_stride;
  fa.Hv = P.L.Hv;
  fa.group = P.L.Hv / P.L.Hqk;
  fa.scale = P.L.scale;
  return hip_status(launch_factorize(fa, P.L.D, stream));
}

template <typename IO>
gdn_status do_scan(const PrefillPrep& P, hipStream_t stream, const void* q, const void* k, const void* v,
                   int64_t qk_stride, int64_t v_stride, const gdn_ckpt* ckpt, float* o, void* ws) {
  ScanArgs<IO> sa;
  fill_call_table(P.plan, ws, &sa.tab);
  sa.q = static_cast<const IO*>(q);
  sa.k = static_cast<const IO*>(k);
  sa.v = static_cast<const IO*>(v);
  sa.qk_stride = qk_stride;
  sa.v_stride = v_stride;
  sa.factors = static_cast<uint8_t*>(ws) + P.plan.off_factors;
  sa.factor_stride = P.plan.factor_stride;
  sa.Hv = P.L.Hv;
  sa.group = P.L.Hv / P.L.Hqk;
  sa.o = o;
  sa.ckpt_pool = static_cast<uint8_t*>(ckpt->pool);
  sa.page_bytes = (size_t)ckpt->page_bytes;
  return hip_status(launch_scan(sa, P.L.D, stream));
}

// The state references of the scan go into the table entries.
void set_state_refs(PrefillPrep* P, const gdn_state_ref* states) {
  for (size_t s = 0; s < P->spans.size(); ++s) {
    const gdn_state_ref& r = states[s];
    P->plan.seqs[s].src = r.src_kind == GDN_SRC_ZERO ? nullptr : r.src;
    P->plan.seqs[s].dst = r.dst;
  }
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


// A whole prefill call checked before anything is enqueued (gdn_chunk_prefill and the
// prefill stage of gdn_core_prefill).
gdn_status prep_prefill_call(const gdn_layer* layer, const gdn_varlen* varlen, const void* q, const void* k,
                             const void* v, int64_t qk_stride, int64_t v_stride, const float* a, const float* b,
                             const gdn_state_ref* states, const gdn_ckpt* ckpt, const float* o,
                             const void* workspace, size_t workspace_bytes, const gdn_staging* staging,
                             PrefillPrep* P) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  gdn_status s = prep_prefill(layer, varlen, ckpt->block, ckpt, P);
  if (s != GDN_OK) return s;
  s = check_qkv(P->L, q, k, v, qk_stride, v_stride, true, true);
  if (s != GDN_OK) return s;
  if (P->plan.n_units > 0 && (!a || !b || !o)) return GDN_ERR_NULL_ARG;
  s = check_states(*P, states, ckpt->block);
  if (s != GDN_OK) return s;
  s = check_workspace(const_cast<void*>(workspace), workspace_bytes, P->plan.total_bytes);
  if (s != GDN_OK) return s;
  s = check_staging(P->plan, staging);
  if (s != GDN_OK) return s;
  set_state_refs(P, states);
  return GDN_OK;
}

gdn_status launch_prefill_call(const PrefillPrep& P, hipStream_t stream, const void* q, const void* k,
                               const void* v, int64_t qk_stride, int64_t v_stride, const float* a, const float* b,
                               const gdn_ckpt* ckpt, float* o, void* workspace, const gdn_staging* staging) {
  gdn_status s = stage_table(P.plan, staging, workspace, stream);
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

// A conv call checked before anything is enqueued (gdn_conv_update and the conv stage
// of gdn_core_prefill): the plan's entries carry the tail sources and destinations.
struct ConvCall {
  LayerInfo L;
  std::vector<SeqSpan> spans;
  CallPlan plan;
};

gdn_status prep_conv(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block, const gdn_ckpt* ckpt,
                     LayerInfo* L, std::vector<SeqSpan>* spans, CallPlan* plan) {
  gdn_status s = check_layer(layer, L);
  if (s != GDN_OK) return s;
  s = check_varlen(varlen, spans);
  if (s != GDN_OK) return s;
  if (block < 0) return GDN_ERR_BAD_SHAPE;
  std::vector<int32_t> pages, page_begin;
  if (ckpt) {
    s = check_ckpt(ckpt, *L, *spans, &pages, &page_begin);
    if (s != GDN_OK) return s;
  }
  return plan_call(*L, *spans, block, ckpt ? &pages : nullptr, ckpt ? &page_begin : nullptr, false, plan);
}

gdn_status prep_conv_call(const gdn_layer* layer, const gdn_varlen* varlen, const void* x, int64_t x_stride,
                          const void* w, const gdn_state_ref* tails, const gdn_ckpt* ckpt, const void* y,
                          const void* workspace, size_t workspace_bytes, const gdn_staging* staging, ConvCall* c) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  gdn_status s = prep_conv(layer, varlen, ckpt->block, ckpt, &c->L, &c->spans, &c->plan);
  if (s != GDN_OK) return s;
  const LayerInfo& L = c->L;
  s = check_sources(tails, c->spans, ckpt->block);
  if (s != GDN_OK) return s;
  const int64_t total_rows = c->spans.empty() ? 0 : c->spans.back().row0 + c->spans.back().len;
  if (total_rows > 0 && (!x || !y)) return GDN_ERR_NULL_ARG;
  if (!w && !c->spans.empty()) return GDN_ERR_NULL_ARG;
  // rows are read 16 bytes at a time: a stride of whole 16-byte groups
  if (x_stride < L.channels || (x_stride * (int64_t)L.io_bytes) % 16 != 0) return GDN_ERR_BAD_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 16)) return GDN_ERR_BAD_SHAPE;
  for (size_t i = 0; i < c->spans.size(); ++i) {
    if (tails[i].src_kind != GDN_SRC_ZERO && !aligned(tails[i].src, 16)) return GDN_ERR_BAD_SHAPE;
    if (!aligned(tails[i].dst, 16)) return GDN_ERR_BAD_SHAPE;
  }
  if (c->plan.staged) {
    s = check_workspace(const_cast<void*>(workspace), workspace_bytes, c->plan.table_bytes);
    if (s != GDN_OK) return s;
  }
  s = check_staging(c->plan, staging);
  if (s != GDN_OK) return s;
  for (size_t i = 0; i < c->spans.size(); ++i) {
    const gdn_state_ref& r = tails[i];
    const uint8_t* src = static_cast<const uint8_t*>(r.src);
    if (r.src_kind == GDN_SRC_ZERO) src = nullptr;
    if (r.src_kind == GDN_SRC_CHECKPOINT) src += L.state_bytes;  // tail region of the page
    c->plan.seqs[i].src = src;
    c->plan.seqs[i].dst = r.dst;
  }
  return GDN_OK;
}

gdn_status launch_conv_call(const ConvCall& c, hipStream_t stream, const void* x, int64_t x_stride, const void* w,
                            const gdn_ckpt* ckpt, void* y, void* workspace, const gdn_staging* staging) {
  if (c.plan.n_units == 0) return GDN_OK;
  gdn_status s = stage_table(c.plan, staging, workspace, stream);
  if (s != GDN_OK) return s;
  const LayerInfo& L = c.L;
  auto fill = [&](auto& ca, auto tag) {
    using IO = decltype(tag);
    fill_call_table(c.plan, workspace, &ca.tab);
    ca.x = static_cast<const IO*>(x);
    ca.x_stride = x_stride;
    ca.w = static_cast<const IO*>(w);
    ca.y = static_cast<IO*>(y);
    ca.ckpt_pool = static_cast<uint8_t*>(ckpt->pool);
    ca.page_bytes = (size_t)ckpt->page_bytes;
    ca.tail_offset = (size_t)L.state_bytes;
    ca.channels = L.channels;
    ca.qk_channels = 2 * (int64_t)L.Hqk * L.D;
    ca.head_dim = L.D;
    ca.act = L.act;
  };
  if (L.io == GDN_BF16) {
    ConvArgs<bf16_bits> ca;
    fill(ca, bf16_bits{});
    return hip_status(launch_conv(ca, stream));
  }
  ConvArgs<float> ca;
  fill(ca, float{});
  return hip_status(launch_conv(ca, stream));
}

// The gates and the gated norm: checks, then launches.
gdn_status check_gates(const LayerInfo& L, int64_t n_tokens, const void* ba, int64_t ba_stride, const float* A_log,
                       const void* dt_bias, const float* a, const float* b) {
  if (n_tokens < 0 || ba_stride < 2 * (int64_t)L.Hv) return GDN_ERR_BAD_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  if (!ba || !A_log || !dt_bias || !a || !b) return GDN_ERR_NULL_ARG;
  return GDN_OK;
}

gdn_status launch_gates_call(const LayerInfo& L, hipStream_t stream, int64_t n_tokens, const void* ba,
                             int64_t ba_stride, const float* A_log, const void* dt_bias, float* a, float* b) {
  if (n_tokens == 0) return GDN_OK;
  if (L.io == GDN_BF16) {
    GateArgs<bf16_bits> ga{static_cast<const bf16_bits*>(ba), A_log, static_cast<const bf16_bits*>(dt_bias), a, b,
                           n_tokens, ba_stride, L.Hv};
    return hip_status(launch_gates(ga, stream));
  }
  GateArgs<float> ga{static_cast<const float*>(ba), A_log, static_cast<const float*>(dt_bias), a, b, n_tokens,
                     ba_stride, L.Hv};
  return hip_status(launch_gates(ga, stream));
}

gdn_status check_gated_norm(const LayerInfo& L, int64_t n_tokens, const float* o, const void* z, int64_t z_stride,
                            const void* weight, float eps, const void* out) {
  // z rows are read 16 bytes at a time: a stride of whole 8-element groups
  if (n_tokens < 0 || z_stride < (int64_t)L.Hv * L.D || z_stride % 8 != 0 || !(eps >= 0.f)) return GDN_ERR_BAD_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  if (!o || !z || !weight || !out) return GDN_ERR_NULL_ARG;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(weight, 16) || !aligned(out, 16)) return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

gdn_status launch_gated_norm_call(const LayerInfo& L, hipStream_t stream, int64_t n_tokens, const float* o,
                                  const void* z, int64_t z_stride, const void* weight, float eps, void* out) {
  if (n_tokens == 0) return GDN_OK;
  if (L.io == GDN_BF16) {
    NormArgs<bf16_bits> na{o, static_cast<const bf16_bits*>(z), static_cast<const bf16_bits*>(weight),
                           static_cast<bf16_bits*>(out), n_tokens * L.Hv, z_stride, L.Hv, eps};
    return hip_status(launch_gated_norm(na, L.D, stream));
  }
  NormArgs<float> na{o, static_cast<const float*>(z), static_cast<const float*>(weight), static_cast<float*>(out),
                     n_tokens * L.Hv, z_stride, L.Hv, eps};
  return hip_status(launch_gated_norm(na, L.D, stream));
}

// Workspace and staging layout of gdn_core_prefill: the conv's staged table, the
// prefill's workspace (its staged table, then the factor records), then the stage
// outputs y [tokens][C] io, a and b [tokens][Hv] fp32, o [tokens][Hv][d] fp32, each
// region 256-byte aligned.  Staging: the conv's table, then the prefill's.
struct CoreLayout {
  ConvCall conv;
  PrefillPrep pre;
  int64_t tokens = 0;
  size_t off_prefill = 0, off_y = 0, off_a = 0, off_b = 0, off_o = 0, total = 0;
  size_t stage_prefill = 0, stage_total = 0;
};

gdn_status core_layout(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block, const gdn_ckpt* ckpt,
                       CoreLayout* c) {
  gdn_status s = prep_conv(layer, varlen, block, ckpt, &c->conv.L, &c->conv.spans, &c->conv.plan);
  if (s != GDN_OK) return s;
  s = prep_prefill(layer, varlen, block, ckpt, &c->pre);
  if (s != GDN_OK) return s;
  const LayerInfo& L = c->conv.L;
  c->tokens = c->conv.spans.empty() ? 0 : c->conv.spans.back().row0 + c->conv.spans.back().len;
  const size_t T = (size_t)c->tokens;
  c->off_prefill = align_up(c->conv.plan.staged ? c->conv.plan.table_bytes : 0);
  c->off_y = align_up(c->off_prefill + c->pre.plan.total_bytes);
  c->off_a = align_up(c->off_y + T * (size_t)L.channels * L.io_bytes);
  c->off_b = align_up(c->off_a + T * (size_t)L.Hv * 4);
  c->off_o = align_up(c->off_b + T * (size_t)L.Hv * 4);
  c->total = align_up(c->off_o + T * (size_t)L.Hv * L.D * 4);
  c->stage_prefill = align_up(c->conv.plan.staged ? c->conv.plan.table_bytes : 0);
  c->stage_total = c->pre.plan.staged || c->conv.plan.staged ? c->stage_prefill + c->pre.plan.table_bytes : 0;
  return GDN_OK;
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
    case GDN_ERR_STAGING: return "the call's tables need a pinned host staging buffer (missing or too small)";
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

int64_t gdn_prefill_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  PrefillPrep P;
  if (prep_prefill(layer, varlen, block, nullptr, &P) != GDN_OK) return -1;
  return (int64_t)P.plan.table_bytes;
}


int64_t gdn_conv_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  LayerInfo L;
  std::vector<SeqSpan> spans;
  CallPlan plan;
  if (prep_conv(layer, varlen, block, nullptr, &L, &spans, &plan) != GDN_OK) return -1;
  return (int64_t)plan.table_bytes;
}

int64_t gdn_conv_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  return gdn_conv_workspace_bytes(layer, varlen, block);
}

gdn_status gdn_prefill_factorize(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                                 const void* q, const void* k, int64_t qk_stride, const float* a, const float* b,
                                 int32_t block, void* workspace, size_t workspace_bytes,
                                 const gdn_staging* staging) {
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, block, nullptr, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, nullptr, qk_stride, 0, true, false);
  if (s != GDN_OK) return s;
  if (P.plan.n_units > 0 && (!a || !b)) return GDN_ERR_NULL_ARG;
  s = check_workspace(workspace, workspace_bytes, P.plan.total_bytes);
  if (s != GDN_OK) return s;
  s = check_staging(P.plan, staging);
  if (s != GDN_OK) return s;
  s = stage_table(P.plan, staging, workspace, stream);
  if (s != GDN_OK) return s;
  return P.L.io == GDN_BF16 ? do_factorize<bf16_bits>(P, stream, q, k, qk_stride, a, b, workspace)
                            : do_factorize<float>(P, stream, q, k, qk_stride, a, b, workspace);
}

gdn_status gdn_prefill_scan(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* q,
                            const void* k, const void* v, int64_t qk_stride, int64_t v_stride,
                            const gdn_state_ref* states, const gdn_ckpt* ckpt, float* o, void* workspace,
                            size_t workspace_bytes, const gdn_staging* staging) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, ckpt->block, ckpt, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, v, qk_stride, v_stride, true, true);
  if (s != GDN_OK) return s;
  if (!o && P.plan.n_units > 0) return GDN_ERR_NULL_ARG;
  s = check_states(P, states, ckpt->block);
  if (s != GDN_OK) return s;
  s = check_workspace(workspace, workspace_bytes, P.plan.total_bytes);
  if (s != GDN_OK) return s;
  s = check_staging(P.plan, staging);
  if (s != GDN_OK) return s;
  set_state_refs(&P, states);
  s = stage_table(P.plan, staging, workspace, stream);
  if (s != GDN_OK) return s;
  return P.L.io == GDN_BF16 ? do_scan<bf16_bits>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace)
                            : do_scan<float>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, workspace);
}

gdn_status gdn_chunk_prefill(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* q,
                             const void* k, const void* v, int64_t qk_stride, int64_t v_stride, const float* a,
                             const float* b, const gdn_state_ref* states, const gdn_ckpt* ckpt, float* o,
                             void* workspace, size_t workspace_bytes, const gdn_staging* staging) {
  PrefillPrep P;
  gdn_status s = prep_prefill_call(layer, varlen, q, k, v, qk_stride, v_stride, a, b, states, ckpt, o, workspace,
                                   workspace_bytes, staging, &P);
  if (s != GDN_OK) return s;
  return launch_prefill_call(P, stream, q, k, v, qk_stride, v_stride, a, b, ckpt, o, workspace, staging);
}

gdn_status gdn_chunk_prefill_noalloc(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen,
                                     const void* q, const void* k, const void* v, int64_t qk_stride, int64_t v_stride,
                                     const float* a, const float* b, const gdn_state_ref* states,
                                     const gdn_ckpt* ckpt, float* o) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  PrefillPrep P;
  gdn_status s = prep_prefill(layer, varlen, ckpt->block, ckpt, &P);
  if (s != GDN_OK) return s;
  s = check_qkv(P.L, q, k, v, qk_stride, v_stride, true, true);
  if (s != GDN_OK) return s;
  if (P.plan.n_units > 0 && (!a || !b || !o)) return GDN_ERR_NULL_ARG;
  s = check_states(P, states, ckpt->block);
  if (s != GDN_OK) return s;
  // the scratch holds the records; the tables must travel in the kernel arguments
  if (P.plan.staged || P.plan.total_bytes > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_CAPACITY;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != GDN_OK) return s;
  set_state_refs(&P, states);
  if (P.L.io == GDN_BF16) {
    s = do_factorize<bf16_bits>(P, stream, q, k, qk_stride, a, b, ws);
    if (s != GDN_OK) return s;
    return do_scan<bf16_bits>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, ws);
  }
  s = do_factorize<float>(P, stream, q, k, qk_stride, a, b, ws);
  if (s != GDN_OK) return s;
  return do_scan<float>(P, stream, q, k, v, qk_stride, v_stride, ckpt, o, ws);
}

gdn_status gdn_conv_update(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* x,
                           int64_t x_stride, const void* w, const gdn_state_ref* tails, const gdn_ckpt* ckpt,
                           void* y, void* workspace, size_t workspace_bytes, const gdn_staging* staging) {
  ConvCall c;
  gdn_status s = prep_conv_call(layer, varlen, x, x_stride, w, tails, ckpt, y, workspace, workspace_bytes, staging,
                                &c);
  if (s != GDN_OK) return s;
  return launch_conv_call(c, stream, x, x_stride, w, ckpt, y, workspace, staging);
}

gdn_status gdn_conv_decode(const gdn_layer* layer, hipStream_t stream, int32_t n_req, int64_t n_rows,
                           const void* x, int64_t x_stride, const void* w, void* tail_pool, int64_t n_slots,
                           const int32_t* slot_ids, const int32_t* rows, void* y, int32_t* status) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  if (n_req < 0 || n_slots < 0 || n_rows < 0) return GDN_ERR_BAD_SHAPE;
  if (x_stride < L.channels || (x_stride * (int64_t)L.io_bytes) % 16 != 0) return GDN_ERR_BAD_SHAPE;
  if (n_req == 0) return GDN_OK;
  if (!x || !w || !tail_pool || !slot_ids || !y) return GDN_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(tail_pool, 16) || !aligned(y, 16)) return GDN_ERR_BAD_SHAPE;
  if (n_req > 65535) return GDN_ERR_CAPACITY;
  auto fill = [&](auto& ca, auto tag) {
    using IO = decltype(tag);
    ca.x = static_cast<const IO*>(x);
    ca.x_stride = x_stride;
    ca.w = static_cast<const IO*>(w);
    ca.y = static_cast<IO*>(y);
    ca.tail_pool = static_cast<IO*>(tail_pool);
    ca.slot_ids = slot_ids;
    ca.rows = rows;
    ca.status = status;
    ca.n_slots = n_slots;
    ca.n_rows = rows ? n_rows : (int64_t)n_req;
    ca.channels = L.channels;
    ca.qk_channels = 2 * (int64_t)L.Hqk * L.D;
    ca.head_dim = L.D;
    ca.act = L.act;
  };
  if (L.io == GDN_BF16) {
    ConvDecodeArgs<bf16_bits> ca;
    fill(ca, bf16_bits{});
    return hip_status(launch_conv_decode(ca, n_req, stream));
  }
  ConvDecodeArgs<float> ca;
  fill(ca, float{});
  return hip_status(launch_conv_decode(ca, n_req, stream));
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
  s = check_gates(L, n_tokens, ba, ba_stride, A_log, dt_bias, a, b);
  if (s != GDN_OK) return s;
  return launch_gates_call(L, stream, n_tokens, ba, ba_stride, A_log, dt_bias, a, b);
}

gdn_status gdn_gated_norm(const gdn_layer* layer, hipStream_t stream, int64_t n_tokens, const float* o,
                          const void* z, int64_t z_stride, const void* weight, float eps, void* out) {
  LayerInfo L;
  gdn_status s = check_layer(layer, &L);
  if (s != GDN_OK) return s;
  s = check_gated_norm(L, n_tokens, o, z, z_stride, weight, eps, out);
  if (s != GDN_OK) return s;
  return launch_gated_norm_call(L, stream, n_tokens, o, z, z_stride, weight, eps, out);
}

int64_t gdn_core_prefill_workspace_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  CoreLayout c;
  if (core_layout(layer, varlen, block, nullptr, &c) != GDN_OK) return -1;
  return (int64_t)c.total;
}

int64_t gdn_core_prefill_staging_bytes(const gdn_layer* layer, const gdn_varlen* varlen, int32_t block) {
  CoreLayout c;
  if (core_layout(layer, varlen, block, nullptr, &c) != GDN_OK) return -1;
  return (int64_t)c.stage_total;
}

gdn_status gdn_core_prefill(const gdn_layer* layer, hipStream_t stream, const gdn_varlen* varlen, const void* qkvz,
                            int64_t qkvz_stride, const void* ba, int64_t ba_stride, const void* conv_w,
                            const float* A_log, const void* dt_bias, const void* norm_weight, float eps,
                            const gdn_state_ref* tails, const gdn_state_ref* states, const gdn_ckpt* ckpt,
                            void* out, void* workspace, size_t workspace_bytes, const gdn_staging* staging) {
  if (!ckpt) return GDN_ERR_NULL_ARG;
  CoreLayout c;
  gdn_status s = core_layout(layer, varlen, ckpt->block, ckpt, &c);
  if (s != GDN_OK) return s;
  const LayerInfo& L = c.conv.L;
  if (c.tokens > 0 && !qkvz) return GDN_ERR_NULL_ARG;
  if (qkvz_stride < L.channels + (int64_t)L.Hv * L.D) return GDN_ERR_BAD_SHAPE;
  s = check_workspace(workspace, workspace_bytes, c.total);
  if (s != GDN_OK) return s;
  if (c.stage_total > 0 && (!staging || !staging->host || staging->bytes < c.stage_total)) return GDN_ERR_STAGING;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* y = ws + c.off_y;
  float* a = reinterpret_cast<float*>(ws + c.off_a);
  float* b = reinterpret_cast<float*>(ws + c.off_b);
  float* o = reinterpret_cast<float*>(ws + c.off_o);
  void* pre_ws = ws + c.off_prefill;
  gdn_staging conv_stage{}, pre_stage{};
  if (c.stage_total > 0) {
    conv_stage = gdn_staging{staging->host, c.stage_prefill};
    pre_stage = gdn_staging{static_cast<uint8_t*>(staging->host) + c.stage_prefill, staging->bytes - c.stage_prefill};
  }
  // every stage checked before the first is enqueued
  const size_t io = L.io_bytes;
  const uint8_t* row = static_cast<const uint8_t*>(qkvz);
  const int64_t qk = (int64_t)L.Hqk * L.D;
  const uint8_t* yb = static_cast<const uint8_t*>(y);
  ConvCall cc;
  s = prep_conv_call(layer, varlen, qkvz, qkvz_stride, conv_w, tails, ckpt, y, ws,
                     c.conv.plan.staged ? c.conv.plan.table_bytes : 0, &conv_stage, &cc);
  if (s != GDN_OK) return s;
  s = check_gates(L, c.tokens, ba, ba_stride, A_log, dt_bias, a, b);
  if (s != GDN_OK) return s;
  PrefillPrep P;
  s = prep_prefill_call(layer, varlen, yb, yb + qk * io, yb + 2 * qk * io, L.channels, L.channels, a, b, states,
                        ckpt, o, pre_ws, c.pre.plan.total_bytes, &pre_stage, &P);
  if (s != GDN_OK) return s;
  const void* z = row ? row + L.channels * io : nullptr;
  s = check_gated_norm(L, c.tokens, o, z, qkvz_stride, norm_weight, eps, out);
  if (s != GDN_OK) return s;
  // conv (+ q/k norm) -> gates -> prefill (q, k, v read in place from the conv rows) ->
  // gated norm (z read in place from the packed rows)
  s = launch_conv_call(cc, stream, qkvz, qkvz_stride, conv_w, ckpt, y, ws, &conv_stage);
  if (s != GDN_OK) return s;
  s = launch_gates_call(L, stream, c.tokens, ba, ba_stride, A_log, dt_bias, a, b);
  if (s != GDN_OK) return s;
  s = launch_prefill_call(P, stream, yb, yb + qk * io, yb + 2 * qk * io, L.channels, L.channels, a, b, ckpt, o,
                          pre_ws, &pre_stage);
  if (s != GDN_OK) return s;
  return launch_gated_norm_call(L, stream, c.tokens, o, z, qkvz_stride, norm_weight, eps, out);
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
  // a 64-row log block of fp32 rows at head_dim 128 (keys, values, their transposes and
  // the new queries) needs more LDS than one CU holds; such logs take at most 32 rows
  if (L.io == GDN_F32 && L.D >= 128 && buf_rows > 32) return GDN_ERR_CAPACITY;
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
