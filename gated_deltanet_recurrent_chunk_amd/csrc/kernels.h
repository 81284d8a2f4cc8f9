// kernels.h -- kernel argument blocks and launchers of libgdn (host and device view).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.h"


namespace gdn {

typedef uint16_t bf16_bits;

// Argument blocks of the prefill and conv kernels carry the call's table (plan.h) by
// value: up to kInlineSeqs sequences and kInlinePages checkpoint pages travel inline.
template <typename IO>
struct FactorizeArgs {
  CallTable tab;  // units = chunks
  const IO* q;
  const IO* k;
  int64_t qk_stride;  // elements per token row of q and k
  const float* a;
  const float* b;
  uint8_t* factors;
  size_t factor_stride;
  int32_t Hv;
  int32_t group;  // value heads per query/key head
  float scale;
};

template <typename IO>
struct ScanArgs {
  CallTable tab;  // units = chunks; src / dst are the states
  const IO* q;
  const IO* k;
  const IO* v;
  int64_t qk_stride;
  int64_t v_stride;
  const uint8_t* factors;
  size_t factor_stride;
  int32_t Hv;
  int32_t group;
  float* o;
  uint8_t* ckpt_pool;
  size_t page_bytes;
};

template <typename IO>
struct FlushArgs {
  float* state_pool;
  const int32_t* slot_ids;
  const int32_t* n_accepted;
  const IO* buf_k;
  const IO* buf_v;
  const float* buf_a;
  const float* buf_b;
  int32_t* status;
  int64_t n_slots;
  int32_t buf_rows;
  int32_t Hqk;
  int32_t Hv;
  int32_t group;
};

template <typename IO>
struct ReplayArgs {
  const float* state_pool;
  const int32_t* slot_ids;
  const int32_t* n_logged;
  const int32_t* n_new;
  const IO* buf_k;
  const IO* buf_v;
  const float* buf_a;
  const float* buf_b;
  const IO* q_new;
  float* o;
  int32_t* status;
  int64_t n_slots;
  int32_t buf_rows;
  int32_t max_new;
  int32_t Hqk;
  int32_t Hv;
  int32_t group;
  float scale;
};

template <typename IO>
struct DecodeArgs {
  const IO* q;
  const IO* k;
  const IO* v;
  const float* a;
  const float* b;
  float* state_pool;
  const int32_t* slot_ids;
  float* o;
  int32_t* status;
  int64_t n_slots;
  int32_t Hqk;
  int32_t Hv;
  int32_t group;
  float scale;
  const int32_t* rows;  // token row of each request (nullptr: row r)
  int64_t n_rows;       // rows in the token arrays
  int64_t qk_stride;    // elements per q / k row
  int64_t v_stride;     // elements per v row
};

template <typename IO>
struct ConvArgs {
  CallTable tab;  // units = tiles of kConvTile rows; src / dst are the tails
  const IO* x;          // row t at x + t * x_stride
  int64_t x_stride;     // elements, >= channels (the packed qkvz row width, or channels)
  const IO* w;
  IO* y;
  uint8_t* ckpt_pool;
  size_t page_bytes;
  size_t tail_offset;  // byte offset of the conv tail inside a page
  int64_t channels;
  int64_t qk_channels;  // 2 * Hqk * head_dim: the channels normalized per head (flag)
  int32_t head_dim;
  int32_t act;          // gdn_act, optionally | GDN_CONV_QK_L2NORM
};

template <typename IO>
struct ConvDecodeArgs {
  const IO* x;           // row t at x + t * x_stride
  int64_t x_stride;      // elements, >= channels
  const IO* w;           // [channels][4]
  IO* y;                 // row t at y + t * channels
  IO* tail_pool;         // [n_slots][3][channels], updated in place
  const int32_t* slot_ids;
  const int32_t* rows;   // token row of each request (nullptr: row r)
  int32_t* status;
  int64_t n_slots;
  int64_t n_rows;
  int64_t channels;
  int64_t qk_channels;
  int32_t head_dim;
  int32_t act;
};

template <typename IO>
struct GateArgs {
  const IO* ba;          // [tokens][ba_stride]: b part at columns 0..Hv-1, a part at Hv..2Hv-1
  const float* A_log;    // [Hv]
  const IO* dt_bias;     // [Hv]
  float* a;              // [tokens][Hv]
  float* b;              // [tokens][Hv]
  int64_t n_tokens;
  int64_t ba_stride;
  int32_t Hv;
};

template <typename IO>
struct NormArgs {
  const float* o;        // [rows][D] (rows = tokens * Hv)
  const IO* z;           // token t: z + t * z_stride, heads [Hv][D]
  const IO* w;           // [D]
  IO* out;               // [rows][D]
  int64_t n_rows;
  int64_t z_stride;
  int32_t Hv;
  float eps;
};

// Argument blocks stay within 4 KiB, a size every HIP launch path accepts, and carry
// their table first: kernels read it at offset 0 of the kernel-argument segment.
static_assert(sizeof(FactorizeArgs<float>) <= 4096 && sizeof(ScanArgs<float>) <= 4096 &&
                  sizeof(ConvArgs<float>) <= 4096, "kernel argument size");
static_assert(offsetof(FactorizeArgs<float>, tab) == 0 && offsetof(FactorizeArgs<bf16_bits>, tab) == 0 &&
                  offsetof(ScanArgs<float>, tab) == 0 && offsetof(ScanArgs<bf16_bits>, tab) == 0 &&
                  offsetof(ConvArgs<float>, tab) == 0 && offsetof(ConvArgs<bf16_bits>, tab) == 0,
              "the call table leads every argument block");

hipError_t launch_gates(const GateArgs<bf16_bits>& a, hipStream_t st);
hipError_t launch_gates(const GateArgs<float>& a, hipStream_t st);
hipError_t launch_gated_norm(const NormArgs<bf16_bits>& a, int D, hipStream_t st);
hipError_t launch_gated_norm(const NormArgs<float>& a, int D, hipStream_t st);
hipError_t launch_factorize(const FactorizeArgs<bf16_bits>& a, int D, hipStream_t st);
hipError_t launch_factorize(const FactorizeArgs<float>& a, int D, hipStream_t st);
hipError_t launch_scan(const ScanArgs<bf16_bits>& a, int D, hipStream_t st);
hipError_t launch_scan(const ScanArgs<float>& a, int D, hipStream_t st);
hipError_t launch_flush(const FlushArgs<bf16_bits>& a, int D, int n_req, hipStream_t st);
hipError_t launch_flush(const FlushArgs<float>& a, int D, int n_req, hipStream_t st);
hipError_t launch_replay(const ReplayArgs<bf16_bits>& a, int D, int n_req, int ct, hipStream_t st);
hipError_t launch_replay(const ReplayArgs<float>& a, int D, int n_req, int ct, hipStream_t st);
hipError_t launch_decode(const DecodeArgs<bf16_bits>& a, int D, int n_req, hipStream_t st);
hipError_t launch_decode(const DecodeArgs<float>& a, int D, int n_req, hipStream_t st);
hipError_t launch_conv(const ConvArgs<bf16_bits>& a, hipStream_t st);
hipError_t launch_conv_decode(const ConvDecodeArgs<bf16_bits>& a, int n_req, hipStream_t st);
hipError_t launch_conv_decode(const ConvDecodeArgs<float>& a, int n_req, hipStream_t st);
hipError_t launch_conv(const ConvArgs<float>& a, hipStream_t st);

}  // namespace gdn
