// stream_kernels.hip -- the bandwidth-bound kernels of libgdn: decode step and conv update.
//
// Both read every byte once and write every byte once; the work is spread so that
// consecutive lanes touch consecutive 16-byte pieces of a row.
#include <hip/hip_runtime.h>

#include "call_table.h"
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace gdn {

namespace {

template <typename IO, int N>
__device__ __forceinline__ void load_vec(const IO* p, float (&out)[N]) {
  if constexpr (sizeof(IO) == 2) {
    static_assert(N % 8 == 0, "bf16 vectors of 8");
#pragma unroll
    for (int u = 0; u < N / 8; ++u) {
      uint4 v = reinterpret_cast<const uint4*>(p)[u];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        out[8 * u + e] = bf16_to_f32((bf16_bits)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu)));
    }
  } else {
    static_assert(N % 4 == 0, "fp32 vectors of 4");
#pragma unroll
    for (int u = 0; u < N / 4; ++u) {
      float4 v = reinterpret_cast<const float4*>(p)[u];
      out[4 * u] = v.x;
      out[4 * u + 1] = v.y;
      out[4 * u + 2] = v.z;
      out[4 * u + 3] = v.w;
    }
  }
}

template <typename IO, int N>
__device__ __forceinline__ void store_vec(IO* p, const float (&in)[N]) {
  if constexpr (sizeof(IO) == 2) {
#pragma unroll
    for (int u = 0; u < N / 8; ++u) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(in[8 * u + 2 * e], in[8 * u + 2 * e + 1]);
      reinterpret_cast<uint4*>(p)[u] = uint4{w[0], w[1], w[2], w[3]};
    }
  } else {
#pragma unroll
    for (int u = 0; u < N / 4; ++u)
      reinterpret_cast<float4*>(p)[u] = float4{in[4 * u], in[4 * u + 1], in[4 * u + 2], in[4 * u + 3]};
  }
}

// Value of lane (lane with the DPP pattern CTRL applied) within its 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (2, 4, 8 or 16) by DPP moves inside a 16-lane
// row: swap neighbours, swap pairs, mirror halves of 8, mirror the 16.  Each step adds
// two groups that hold equal values, so every lane of a group ends with the same bits.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "group of 1..16 lanes");
  if constexpr (LPR >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}

}  // namespace

// ==================================================================================
// Decode: one workgroup per (request, value head).  A state row is covered by D/8
// lanes; lane `sub` of a row holds columns 4 sub .. 4 sub + 3 and D/2 + 4 sub .. + 3, so
// each load or store instruction covers whole 256-byte row halves.  One pass computes,
// per row i,
//   r_k = s_i . k,  r_q = s_i . q,  delta_i = b (v_i - a r_k),
//   s_i <- a s_i + delta_i k,  o_i = scale (a r_q + delta_i (k . q)),
// which is S_t = a S (I - b k k^T) + b v k^T and o = S_t q expanded, with the state
// read and written exactly once (non-temporal: it is not reused by this launch).
template <typename IO, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs<IO> p) {
  constexpr int LPR = D / 8;
  constexpr int NTH = (D * LPR < 256) ? D * LPR : 256;
  constexpr int RPP = NTH / LPR;
  constexpr int NP = D / RPP;
  constexpr int HALF = D / 2;
  // head-major grid: consecutive workgroups take consecutive heads of one request, so
  // they sweep that request's contiguous state block in address order
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int slot = p.slot_ids[r];
  // the request's token row: its own index, or (a mixed batch) a row of the packed
  // token arrays it shares with prefill sequences
  const int64_t row = p.rows ? (int64_t)p.rows[r] : (int64_t)r;
  if (slot < -1 || slot >= p.n_slots || (slot >= 0 && (row < 0 || row >= p.n_rows))) {
    if (tid == 0 && h == 0 && p.status) atomicOr(p.status, 1 << GDN_ERR_CAPACITY);
    return;
  }
  if (slot < 0) return;  // padding: nothing read, nothing written
  const int sub = tid % LPR, rowi = tid / LPR;
  const int j0 = 4 * sub, j1 = HALF + 4 * sub;
  const int hk = h / p.group;
  float* st = p.state_pool + ((size_t)slot * p.Hv + h) * D * D;

  f32x4 s[NP][2];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int i = pp * RPP + rowi;
    s[pp][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + (size_t)i * D + j0));
    s[pp][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + (size_t)i * D + j1));
  }
  float k[8], q[8];
  {
    const IO* kr = p.k + row * p.qk_stride + (int64_t)hk * D;
    const IO* qr = p.q + row * p.qk_stride + (int64_t)hk * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[e] = to_f32(kr[j0 + e]);
      k[4 + e] = to_f32(kr[j1 + e]);
      q[e] = to_f32(qr[j0 + e]);
      q[4 + e] = to_f32(qr[j1 + e]);
    }
  }
  const float a = p.a[row * p.Hv + h];
  const float b = p.b[row * p.Hv + h];
  const IO* vrow = p.v + row * p.v_stride + (int64_t)h * D;
  float vi[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) vi[pp] = to_f32(vrow[pp * RPP + rowi]);

  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) kq = fmaf(k[e], q[e], kq);
  kq = group_sum<LPR>(kq);

  float* orow = p.o + (row * p.Hv + h) * D;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int i = pp * RPP + rowi;
    float rk = 0.f, rq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rk = fmaf(s[pp][0][e], k[e], rk);
      rq = fmaf(s[pp][0][e], q[e], rq);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rk = fmaf(s[pp][1][e], k[4 + e], rk);
      rq = fmaf(s[pp][1][e], q[4 + e], rq);
    }
    rk = group_sum<LPR>(rk);
    rq = group_sum<LPR>(rq);
    const float delta = b * (vi[pp] - a * rk);
    f32x4 n0, n1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      n0[e] = fmaf(a, s[pp][0][e], delta * k[e]);
      n1[e] = fmaf(a, s[pp][1][e], delta * k[4 + e]);
    }
    __builtin_nontemporal_store(n0, reinterpret_cast<f32x4*>(st + (size_t)i * D + j0));
    __builtin_nontemporal_store(n1, reinterpret_cast<f32x4*>(st + (size_t)i * D + j1));
    if (sub == 0) orow[i] = p.scale * fmaf(a, rq, delta * kq);
  }
}

// ==================================================================================
// Conv: thread = VEC consecutive channels x one tile of up to kConvTile rows of one
// sequence.  All kConvTile + 3 input rows the tile needs are requested before any is
// used; rows before a sequence's first token come from its tail source (or are zero,
// never read), rows past the tile's end are clamped to its last row and not used.
//   y[t][c] = act(w[c][0] x[t-3][c] + w[c][1] x[t-2][c] + w[c][2] x[t-1][c] + w[c][3] x[t][c])
// At an absolute block boundary the three raw rows before it go to that page's tail
// region.  The first tile of each sequence also writes the sequence's new tail; it is
// the only tile that reads the old one, so an in-place tail update is safe.
template <typename IO>
__device__ __forceinline__ void unpack_row(const uint4& v, float (&out)[16 / sizeof(IO)]) {
  if constexpr (sizeof(IO) == 2) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32((bf16_bits)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu)));
  } else {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
}

template <typename IO, bool SILU, bool NORM>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs<IO> p) {
  constexpr int VEC = 16 / sizeof(IO);
  constexpr int TR = kConvTile;
  // channel group fastest: consecutive workgroups cover one tile's rows across all
  // channels, sweeping whole rows in address order
  const int ng = (int)((p.channels / VEC + 255) / 256);
  const int tix = (int)(blockIdx.x / ng), cg = (int)(blockIdx.x % ng);
  const int64_t c0 = ((int64_t)cg * 256 + threadIdx.x) * VEC;
  if (c0 >= p.channels) return;
  // the tile's sequence, and its rows [rel0, rel0 + n) within it
  const_table* tab = kernarg_table();
  const SeqEntry sq = seq_entry(tab, unit_sequence(tab, tix));
  const int64_t C = p.channels, XS = p.x_stride;
  const int64_t rel0 = (int64_t)(tix - sq.unit0) * TR;
  const int n = (int)min((int64_t)TR, (int64_t)sq.len - rel0);
  const int64_t tile_row = sq.row0 + rel0;
  const IO* src = reinterpret_cast<const IO*>(sq.src);
  auto row_ptr = [&](int64_t rel) -> const uint4* {
    if (rel >= 0) return reinterpret_cast<const uint4*>(p.x + (sq.row0 + rel) * XS + c0);
    if (src) return reinterpret_cast<const uint4*>(src + (3 + rel) * C + c0);
    return nullptr;  // zero rows: never read
  };

  // rows rel0 - 3 + i, i = 0 .. TR + 2
  uint4 raw[TR + 3];
  if (rel0 >= 3) {
    // a running row pointer (no 64-bit multiply per row); rows past the tile repeat its last
    const IO* ptr = p.x + (sq.row0 + rel0 - 3) * XS + c0;
#pragma unroll
    for (int i = 0; i < TR + 3; ++i) {
      raw[i] = *reinterpret_cast<const uint4*>(ptr);
      if (i + 1 < n + 3) ptr += XS;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TR + 3; ++i) {
      const uint4* ptr = row_ptr(rel0 - 3 + (i < n + 3 ? i : n + 2));
      raw[i] = ptr ? *ptr : uint4{0u, 0u, 0u, 0u};
    }
  }
  float w[4][VEC];
  {
    float wr[4 * VEC];
    load_vec<IO, 4 * VEC>(p.w + c0 * 4, wr);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j][e] = wr[4 * e + j];
  }

  // rows of this tile that end on an absolute block boundary (bit t: position
  // p0 + rel0 + t + 1), and the ordinal of the first such boundary in the sequence
  uint32_t bmask = 0;
  int64_t bord0 = 0;
  const int64_t block = tab->block;
  if (block > 0) {
    const int64_t first = sq.p0 + rel0 + 1, last = sq.p0 + rel0 + n;
    const int64_t nb = (first + block - 1) / block;  // first boundary index >= first
    bord0 = nb - sq.p0 / block - 1;
    for (int64_t P = nb * block; P <= last; P += block) bmask |= 1u << (uint32_t)(P - first);
  }
  int64_t bord = bord0;
  // sliding window over the unpacked rows: each input row is converted once
  float x0[VEC], x1[VEC], x2[VEC];
  unpack_row<IO>(raw[0], x0);
  unpack_row<IO>(raw[1], x1);
  unpack_row<IO>(raw[2], x2);
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    if (t >= n) continue;  // uniform; keeps the loop fully unrolled (raw[] stays in registers)
    float x3[VEC], yv[VEC];
    unpack_row<IO>(raw[t + 3], x3);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float acc = w[0][e] * x0[e];
      acc = fmaf(w[1][e], x1[e], acc);
      acc = fmaf(w[2][e], x2[e], acc);
      acc = fmaf(w[3][e], x3[e], acc);
      // SiLU with the hardware exp and reciprocal: acc / (1 + exp(-acc)); the limits
      // (exp overflow to inf -> rcp 0 -> -0) come out right
      if constexpr (SILU) acc = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
      yv[e] = acc;
    }
    if constexpr (NORM) {
      // unit L2 norm per q / k head: the head's values sit in head_dim / VEC consecutive
      // lanes of one wave (heads start on such a lane group), summed by an xor butterfly
      // (every lane ends with the same bits)
      if (c0 < p.qk_channels) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss = fmaf(yv[e], yv[e], ss);
        for (int off = 1; off < p.head_dim / VEC; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = rsqrtf(ss + 1e-6f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) yv[e] *= inv;
      }
    }
    store_vec<IO, VEC>(p.y + (tile_row + t) * C + c0, yv);
    if (bmask & (1u << t)) {
      {
        const int32_t pid = page_list(tab)[sq.page0 + bord++];
        if (pid >= 0) {
          uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<IO*>(p.ckpt_pool + (size_t)pid * p.page_bytes +
                                                                      p.tail_offset) + c0);
          const size_t rs = C * sizeof(IO) / 16;
          dst[0] = raw[t + 1];
          dst[rs] = raw[t + 2];
          dst[2 * rs] = raw[t + 3];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      x0[e] = x1[e];
      x1[e] = x2[e];
      x2[e] = x3[e];
    }
  }
  if (rel0 == 0) {
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<IO*>(sq.dst) + c0);
    const size_t rs = C * sizeof(IO) / 16;
    uint4 tl[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {  // all read before any is written (the tail may be updated in place)
      const uint4* ptr = row_ptr(sq.len - 3 + i);
      tl[i] = ptr ? *ptr : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) dst[i * rs] = tl[i];
  }
}

// ==================================================================================
// Conv, decode regime: one new row per request, its three previous rows in a slot of a
// tail pool.  Thread = VEC consecutive channels of one request (grid: channel groups x
// requests).  The tail slot is read whole before it is rewritten with the last three
// raw rows, so the in-place update is safe; slot -1 reads and writes nothing.
template <typename IO, bool SILU, bool NORM>
__global__ __launch_bounds__(256) void conv_decode_kernel(ConvDecodeArgs<IO> p) {
  constexpr int VEC = 16 / sizeof(IO);
  const int r = blockIdx.y;
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
  const int slot = p.slot_ids[r];
  const int64_t row = p.rows ? (int64_t)p.rows[r] : (int64_t)r;
  if (slot < -1 || slot >= p.n_slots || (slot >= 0 && (row < 0 || row >= p.n_rows))) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && p.status) atomicOr(p.status, 1 << GDN_ERR_CAPACITY);
    return;
  }
  if (slot < 0 || c0 >= p.channels) return;
  const int64_t C = p.channels;
  IO* tail = p.tail_pool + (int64_t)slot * 3 * C + c0;
  const uint4 t0 = *reinterpret_cast<const uint4*>(tail);
  const uint4 t1 = *reinterpret_cast<const uint4*>(tail + C);
  const uint4 t2 = *reinterpret_cast<const uint4*>(tail + 2 * C);
  const uint4 xr = *reinterpret_cast<const uint4*>(p.x + row * p.x_stride + c0);
  float wr[4 * VEC];
  load_vec<IO, 4 * VEC>(p.w + c0 * 4, wr);
  float x0[VEC], x1[VEC], x2[VEC], x3[VEC], yv[VEC];
  unpack_row<IO>(t0, x0);
  unpack_row<IO>(t1, x1);
  unpack_row<IO>(t2, x2);
  unpack_row<IO>(xr, x3);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float acc = wr[4 * e] * x0[e];
    acc = fmaf(wr[4 * e + 1], x1[e], acc);
    acc = fmaf(wr[4 * e + 2], x2[e], acc);
    acc = fmaf(wr[4 * e + 3], x3[e], acc);
    if constexpr (SILU) acc = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
    yv[e] = acc;
  }
  if constexpr (NORM) {
    if (c0 < p.qk_channels) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss = fmaf(yv[e], yv[e], ss);
      for (int off = 1; off < p.head_dim / VEC; off <<= 1) ss += __shfl_xor(ss, off);
      const float inv = rsqrtf(ss + 1e-6f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) yv[e] *= inv;
    }
  }
  store_vec<IO, VEC>(p.y + row * C + c0, yv);
  *reinterpret_cast<uint4*>(tail) = t1;
  *reinterpret_cast<uint4*>(tail + C) = t2;
  *reinterpret_cast<uint4*>(tail + 2 * C) = xr;
}

template <typename IO>
static hipError_t launch_conv_decode_t(const ConvDecodeArgs<IO>& a, int n_req, hipStream_t st) {
  if (n_req == 0) return hipSuccess;
  constexpr int VEC = 16 / sizeof(IO);
  const int64_t groups = (a.channels / VEC + 255) / 256;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)groups, (unsigned)n_req);
  const bool silu = (a.act & ~GDN_CONV_QK_L2NORM) == GDN_ACT_SILU, norm = (a.act & GDN_CONV_QK_L2NORM) != 0;
  if (silu && norm)
    hipLaunchKernelGGL((conv_decode_kernel<IO, true, true>), grid, dim3(256), 0, st, a);
  else if (silu)
    hipLaunchKernelGGL((conv_decode_kernel<IO, true, false>), grid, dim3(256), 0, st, a);
  else if (norm)
    hipLaunchKernelGGL((conv_decode_kernel<IO, false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((conv_decode_kernel<IO, false, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_conv_decode(const ConvDecodeArgs<bf16_bits>& a, int n_req, hipStream_t st) {
  return launch_conv_decode_t(a, n_req, st);
}
hipError_t launch_conv_decode(const ConvDecodeArgs<float>& a, int n_req, hipStream_t st) {
  return launch_conv_decode_t(a, n_req, st);
}

// ==================================================================================
template <typename IO, int D>
static hipError_t launch_decode_t(const DecodeArgs<IO>& a, int n_req, hipStream_t st) {
  if (n_req == 0) return hipSuccess;
  constexpr int LPR = D / 8;
  constexpr int NTH = (D * LPR < 256) ? D * LPR : 256;
  hipLaunchKernelGGL((decode_kernel<IO, D>), dim3(a.Hv, n_req), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs<bf16_bits>& a, int D, int n_req, hipStream_t st) {
  switch (D) {
    case 16: return launch_decode_t<bf16_bits, 16>(a, n_req, st);
    case 32: return launch_decode_t<bf16_bits, 32>(a, n_req, st);
    case 64: return launch_decode_t<bf16_bits, 64>(a, n_req, st);
    case 128: return launch_decode_t<bf16_bits, 128>(a, n_req, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_decode(const DecodeArgs<float>& a, int D, int n_req, hipStream_t st) {
  switch (D) {
    case 16: return launch_decode_t<float, 16>(a, n_req, st);
    case 32: return launch_decode_t<float, 32>(a, n_req, st);
    case 64: return launch_decode_t<float, 64>(a, n_req, st);
    case 128: return launch_decode_t<float, 128>(a, n_req, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename IO>
static hipError_t launch_conv_t(const ConvArgs<IO>& a, hipStream_t st) {
  const int n_tiles = a.tab.n_units;
  if (n_tiles == 0) return hipSuccess;
  constexpr int VEC = 16 / sizeof(IO);
  const int64_t groups = a.channels / VEC;
  const int64_t blocks = (int64_t)n_tiles * ((groups + 255) / 256);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  const bool silu = (a.act & ~GDN_CONV_QK_L2NORM) == GDN_ACT_SILU, norm = (a.act & GDN_CONV_QK_L2NORM) != 0;
  if (silu && norm)
    hipLaunchKernelGGL((conv_kernel<IO, true, true>), grid, dim3(256), 0, st, a);
  else if (silu)
    hipLaunchKernelGGL((conv_kernel<IO, true, false>), grid, dim3(256), 0, st, a);
  else if (norm)
    hipLaunchKernelGGL((conv_kernel<IO, false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((conv_kernel<IO, false, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_conv(const ConvArgs<bf16_bits>& a, hipStream_t st) { return launch_conv_t<bf16_bits>(a, st); }
hipError_t launch_conv(const ConvArgs<float>& a, hipStream_t st) { return launch_conv_t<float>(a, st); }

// ==================================================================================
// Gates of the packed core ("Hybrid linear attention (gated DeltaNet)", "Packed-core
// traces": the core owns dt_bias and an fp32 A_log and takes the "ba" projection):
//   b = sigmoid(ba_b),   a = exp(-exp(A_log) * softplus(ba_a + dt_bias))
// per (token, value head), in fp32.  a is kept at or above the smallest normal float
// so that its logarithm (the prefill's log-decay) stays finite.
template <typename IO>
__global__ __launch_bounds__(256) void gates_kernel(GateArgs<IO> p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.n_tokens * p.Hv) return;
  const int64_t t = i / p.Hv;
  const int h = (int)(i - t * p.Hv);
  const IO* row = p.ba + t * p.ba_stride;
  const float bx = to_f32(row[h]), ax = to_f32(row[p.Hv + h]);
  const float x = ax + to_f32(p.dt_bias[h]);
  // softplus(x) = log(1 + e^x), = x once e^-x is below fp32 resolution
  const float sp = x > 20.f ? x : log1pf(expf(x));
  p.a[i] = fmaxf(expf(-expf(p.A_log[h]) * sp), 1.17549435e-38f);
  p.b[i] = 1.f / (1.f + expf(-bx));
}

// Gated RMSNorm of the output rows (the packed core's output is "gated-normalized value
// rows", with a norm scale replicated over heads):
//   out = o * (mean(o^2) + eps)^(-1/2) * w * silu(z)
// per (token, value head) row of D values; D / 8 lanes per row, 8 values per lane, the
// mean by an xor butterfly inside the lane group.
template <typename IO, int D>
__global__ __launch_bounds__(256) void gated_norm_kernel(NormArgs<IO> p) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int j0 = (threadIdx.x % LPR) * 8;
  if (row >= p.n_rows) return;  // whole lane groups leave together
  const int64_t t = row / p.Hv;
  const int h = (int)(row - t * p.Hv);
  float ov[8], zv[8], wv[8];
  load_vec<float, 8>(p.o + row * D + j0, ov);
  load_vec<IO, 8>(p.z + t * p.z_stride + (int64_t)h * D + j0, zv);
  load_vec<IO, 8>(p.w + j0, wv);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(ov[e], ov[e], ss);
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off);
  const float r = rsqrtf(ss * (1.f / D) + p.eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (ov[e] * r) * wv[e] * (zv[e] / (1.f + __expf(-zv[e])));
  store_vec<IO, 8>(p.out + row * D + j0, y);
}

template <typename IO>
static hipError_t launch_gates_t(const GateArgs<IO>& a, hipStream_t st) {
  const int64_t n = a.n_tokens * a.Hv;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gates_kernel<IO>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_gates(const GateArgs<bf16_bits>& a, hipStream_t st) { return launch_gates_t(a, st); }
hipError_t launch_gates(const GateArgs<float>& a, hipStream_t st) { return launch_gates_t(a, st); }

template <typename IO, int D>
static hipError_t launch_norm_t(const NormArgs<IO>& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 8);
  const int64_t blocks = (a.n_rows + RPB - 1) / RPB;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_norm_kernel<IO, D>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename IO>
static hipError_t launch_norm_d(const NormArgs<IO>& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch_norm_t<IO, 16>(a, st);
    case 32: return launch_norm_t<IO, 32>(a, st);
    case 64: return launch_norm_t<IO, 64>(a, st);
    case 128: return launch_norm_t<IO, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_gated_norm(const NormArgs<bf16_bits>& a, int D, hipStream_t st) { return launch_norm_d(a, D, st); }
hipError_t launch_gated_norm(const NormArgs<float>& a, int D, hipStream_t st) { return launch_norm_d(a, D, st); }

}  // namespace gdn
