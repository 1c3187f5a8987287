// a3: logical top-k position -> physical KV slot.
//
// "nsa_backend.py (EngineX-Hygon sglang fork)", forward_decode /
// forward_extend: the top-k indices are mapped through page_table_1 (one
// slot per token, page_size 1) by transform_index_page_table_decode /
// _prefill before sparse attention. The compact form reaches the same slot
// through the 64-token page table (_transform_table_1_to_real). -1 passes
// through. Rows reach their request's table row through token_to_req.
//
// Launch shape: a 1-D grid of 256-thread blocks, each block one row chunk of
// 1024 entries (4 per thread, int4 loads and stores when aligned).
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;

__device__ __forceinline__ int32_t map_one(int32_t i, const int32_t* pt1_row,
                                           int64_t pt1_width,
                                           const int32_t* rpt_row,
                                           int64_t rpt_width) {
  if (i < 0) return -1;
  if (pt1_row != nullptr) {
    if (i < pt1_width) return pt1_row[i];
  } else {
    const int32_t p = i >> 6;
    if (p < rpt_width) return (rpt_row[p] << 6) + (i & 63);
  }
  flag_device_error(NSA_DEVERR_INDEX);   // past the table's width
  return -1;
}

__global__ void __launch_bounds__(kThreads)
page_table_transform_kernel(const int32_t* __restrict__ idx, int64_t in_stride,
                            int topk, int chunks_per_row,
                            const int32_t* __restrict__ pt1, int64_t pt1_stride,
                            int64_t pt1_width, const int32_t* __restrict__ rpt,
                            int64_t rpt_stride, int64_t rpt_width,
                            int64_t table_rows,
                            const int32_t* __restrict__ t2r, int32_t* out,
                            int64_t out_stride, bool vec) {
  const int64_t t = blockIdx.x / chunks_per_row;
  const int c = blockIdx.x % chunks_per_row;
  const int32_t r = t2r[t];
  const int32_t* in = idx + t * in_stride;
  int32_t* o = out + t * out_stride;
  const int j0 = c * kChunk + threadIdx.x * kPerThread;
  if (r < 0 || r >= table_rows) {   // a row of no known request: all -1
    if (c == 0 && threadIdx.x == 0) flag_device_error(NSA_DEVERR_REQUEST);
    for (int k = 0; k < kPerThread; ++k)
      if (j0 + k < topk) o[j0 + k] = -1;
    return;
  }
  const int32_t* pt1_row = pt1 ? pt1 + (int64_t)r * pt1_stride : nullptr;
  const int32_t* rpt_row = rpt ? rpt + (int64_t)r * rpt_stride : nullptr;
  if (vec && j0 + kPerThread <= topk) {
    const int4 v = *reinterpret_cast<const int4*>(in + j0);
    int4 w;
    w.x = map_one(v.x, pt1_row, pt1_width, rpt_row, rpt_width);
    w.y = map_one(v.y, pt1_row, pt1_width, rpt_row, rpt_width);
    w.z = map_one(v.z, pt1_row, pt1_width, rpt_row, rpt_width);
    w.w = map_one(v.w, pt1_row, pt1_width, rpt_row, rpt_width);
    *reinterpret_cast<int4*>(o + j0) = w;
    return;
  }
  for (int k = 0; k < kPerThread; ++k) {
    const int j = j0 + k;
    if (j < topk) o[j] = map_one(in[j], pt1_row, pt1_width, rpt_row, rpt_width);
  }
}

}  // namespace

extern "C" int nsa_page_table_transform(
    const int32_t* topk_indices, int64_t in_stride, int T, int topk,
    const int32_t* page_table_1, int64_t pt1_stride, int64_t pt1_width,
    const int32_t* real_page_table, int64_t rpt_stride, int64_t rpt_width,
    int64_t table_rows, int page_size, const int32_t* token_to_req,
    int32_t* out, int64_t out_stride, void* stream) {
  const char* fn = "nsa_page_table_transform";
  NSA_REQUIRE(T >= 0 && topk >= 0 && table_rows >= 0, NSA_ERR_INVALID_ARG,
              "%s: negative size", fn);
  NSA_REQUIRE(page_size == NSA_PAGE_SIZE, NSA_ERR_UNSUPPORTED,
              "%s: page_size %d (only 64 is supported)", fn, page_size);
  NSA_REQUIRE((page_table_1 == nullptr) != (real_page_table == nullptr),
              NSA_ERR_INVALID_ARG,
              "%s: give exactly one of page_table_1 / real_page_table", fn);
  if (T == 0 || topk == 0) return nsa::ok();
  NSA_REQUIRE(topk_indices && token_to_req && out, NSA_ERR_INVALID_ARG,
              "%s: null pointer", fn);
  NSA_REQUIRE(in_stride >= topk && out_stride >= topk, NSA_ERR_INVALID_ARG,
              "%s: row stride < topk", fn);
  if (page_table_1)
    NSA_REQUIRE(pt1_width >= 0 && pt1_stride >= pt1_width, NSA_ERR_INVALID_ARG,
                "%s: bad page_table_1 stride/width", fn);
  else
    NSA_REQUIRE(rpt_width >= 0 && rpt_stride >= rpt_width, NSA_ERR_INVALID_ARG,
                "%s: bad real_page_table stride/width", fn);
  const int chunks = (topk + kChunk - 1) / kChunk;
  const int64_t blocks = (int64_t)T * chunks;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  const bool vec = nsa::aligned(topk_indices, 16) && nsa::aligned(out, 16) &&
                   in_stride % 4 == 0 && out_stride % 4 == 0;
  hipLaunchKernelGGL(page_table_transform_kernel, dim3((unsigned)blocks),
                     dim3(kThreads), 0, (hipStream_t)stream, topk_indices,
                     in_stride, topk, chunks, page_table_1, pt1_stride,
                     pt1_width, real_page_table, rpt_stride, rpt_width,
                     table_rows, token_to_req, out, out_stride, vec);
  return nsa::check_launch(fn);
}
