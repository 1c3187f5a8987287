// Definitions shared by the sparse MLA translation units (sparse_mla.hip:
// the 16..64-head kernels, the plan and the entry points; sparse_mla_h128.hip:
// the 128-head kernel, built with its own code-generation options).
#pragma once

#include "common.h"

namespace nsa_mla {

constexpr int kStep = 32;                 // slots per step
constexpr int kDQK = 576, kDV = 512;
constexpr int kKsStride = kDQK + 8;       // bf16 elements per staged K row
constexpr int kKsRow = kKsStride * 2;     // bytes per staged K row (1168)
constexpr int kKsBytes = kStep * kKsRow;  // 37376
constexpr int kMaxSplit = 2048;           // slots per block of the 64/128-head kernels
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const uint16_t* q;
  int64_t q_tok_stride, q_head_stride;
  const uint8_t* kv;
  int64_t num_slots;
  const int32_t* idx;
  int64_t idx_stride;
  const int32_t* seqlens;  // nullable
  int T, H, topk;
  float scale_log2;
  uint16_t* out;
  float* lse;              // nullable
  float* ws_o;             // split partials when n_splits > 1 (fp32 rows; bf16 rows for
                           // the 128-head kernel)
  float* ws_lse;           // [n_splits][T][H]
  int n_splits, split_slots, n_hb;
};

// Work groups are dealt to the 8 XCDs round-robin: logical block ids that
// are consecutive land on one XCD (its L2).
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t bid, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = bid % 8;
  return x * q + (x < r ? x : r) + bid / 8;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 4 bf16 of one value dim across 4 slot rows: within each 16-lane group,
// source lane s points at slot row base + s/4 and dims +4(s%4); the
// hardware transposes, giving lane i dim i of the 4 rows.
__device__ __forceinline__ v4i16 read_tr(const uint8_t* lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) uint8_t*)lds_byte_addr);
}

// 128-head kernel (sparse_mla_h128.hip): one block per (query row, KV split),
// blocks = T * n_splits, p.split_slots <= kMaxSplit. With n_splits > 1 each
// block writes its split's bf16 partial rows to p.ws_o (as uint16,
// [n_splits][T][128][512]) and its log-sum-exp to p.ws_lse.
int launch_sparse_mla_h128(const Params& p, unsigned blocks, hipStream_t s);

}  // namespace nsa_mla
