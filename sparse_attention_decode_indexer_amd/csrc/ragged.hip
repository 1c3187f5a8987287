// f3: the RAGGED extend route of "dsa_backend.py (sglang main)".
//
// Besides the paged prefill route, the page scores every extend token against
// the concatenated keys of the batch and attends over a contiguous bf16 copy
// of the batch's latent rows:
//   * init_forward_metadata, extend branch: page_table_1_flattened (every
//     cached token's slot, request after request) and topk_indices_offset
//     (cu_seqlens_k[:-1] repeated once per extend token);
//   * _cal_indexer_k_start_end: the logits window [ks, ke) of each token;
//   * forward_extend, RAGGED: valid top-k positions shifted by the offset
//     (the paged dequantization of the flattened table is in quant.hip);
//   * the aiter decode route's get_valid_kv_indices: CSR lists of the
//     entries != -1 of an index matrix.
// Here every one of these is a device kernel fed by the per-forward metadata,
// so the route needs no host sync (the pages build ks / ke with a host loop).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// ks, ke and the top-k offset of every query row.
__global__ void __launch_bounds__(kThreads)
ragged_rows_kernel(const int32_t* __restrict__ cu_seqlens_k, int bs,
                   const int32_t* __restrict__ seqlens_expanded,
                   const int32_t* __restrict__ token_to_req, int T,
                   int32_t* __restrict__ ks, int32_t* __restrict__ ke,
                   int32_t* __restrict__ offset) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;
  const int r = token_to_req[t];
  const bool r_ok = r >= 0 && r < bs;
  if (!r_ok) flag_device_error(NSA_DEVERR_REQUEST);
  const int32_t s = r_ok ? cu_seqlens_k[r] : 0;
  ks[t] = s;
  ke[t] = s + seqlens_expanded[t];
  if (offset) offset[t] = s;
}

// page_table_1_flattened[cu_seqlens_k[r] + s] = slot of token s of request r,
// from the compact table; block (r, c) covers positions c*kSpan.. of r.
constexpr int kSpan = kThreads * 8;
__global__ void __launch_bounds__(kThreads)
ragged_flat_table_kernel(const int32_t* __restrict__ cu_seqlens_k,
                         const int32_t* __restrict__ cache_seqlens,
                         const int32_t* __restrict__ real_page_table,
                         int64_t rpt_stride, int max_seqlen_k, int chunks,
                         int64_t capacity, int32_t* __restrict__ flat) {
  const int r = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  const int n = min(cache_seqlens[r], max_seqlen_k);
  const int64_t base = cu_seqlens_k[r];
  const int32_t* rpt = real_page_table + (int64_t)r * rpt_stride;
  for (int s = c * kSpan + threadIdx.x; s < min(n, (c + 1) * kSpan); s += kThreads) {
    const int64_t o = base + s;
    if (o >= 0 && o < capacity) flat[o] = (rpt[s >> 6] << 6) + (s & 63);
  }
}

// out = idx + offset[t] for idx != -1, else -1 (out may alias idx: each
// element is read and written by the same thread).
__global__ void __launch_bounds__(kThreads)
ragged_index_kernel(const int32_t* idx, int64_t in_stride, int T, int topk,
                    const int32_t* __restrict__ offset, int32_t* out,
                    int64_t out_stride) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= (int64_t)T * topk) return;
  const int64_t t = e / topk;
  const int j = (int)(e % topk);
  const int32_t v = idx[t * in_stride + j];
  out[t * out_stride + j] = v != -1 ? v + offset[t] : -1;
}

// CSR pass 1: valid entries (!= -1) of every row into kv_indptr[t + 1].
__global__ void __launch_bounds__(kThreads)
csr_count_kernel(const int32_t* __restrict__ idx, int64_t stride, int topk,
                 int32_t* __restrict__ indptr) {
  __shared__ int red[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int32_t* row = idx + t * stride;
  int c = 0;
  for (int j = threadIdx.x; j < topk; j += kThreads) c += row[j] != -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    indptr[t + 1] = s;
  }
}

// CSR pass 2: inclusive scan of indptr[1..T] in place, one block, chunks of
// kScanThreads with a running carry; indptr[0] = 0.
constexpr int kScanThreads = 1024;
__global__ void __launch_bounds__(kScanThreads)
csr_scan_kernel(int32_t* __restrict__ indptr, int T) {
  __shared__ int wsum[kScanThreads / 64];
  __shared__ int carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    carry = 0;
    indptr[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < T; base += kScanThreads) {
    const int i = base + threadIdx.x;
    int x = i < T ? indptr[i + 1] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (i < T) indptr[i + 1] = before + x;
    __syncthreads();
    if (threadIdx.x == kScanThreads - 1) carry = before + x;
    __syncthreads();
  }
}

// CSR pass 3: every row writes its valid entries, in column order, from
// kv_indptr[t]; entries past the capacity are dropped.
__global__ void __launch_bounds__(kThreads)
csr_write_kernel(const int32_t* __restrict__ idx, int64_t stride, int topk,
                 const int32_t* __restrict__ indptr, int64_t capacity,
                 int32_t* __restrict__ out) {
  __shared__ int wsum[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int32_t* row = idx + t * stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t pos = indptr[t];
  for (int j0 = 0; j0 < topk; j0 += kThreads) {
    const int j = j0 + threadIdx.x;
    const int32_t v = j < topk ? row[j] : -1;
    const int f = v != -1;
    int x = f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    const int64_t o = pos + before + x - f;
    if (f && o < capacity) out[o] = v;
    pos += total;
    __syncthreads();
  }
}

}  // namespace

extern "C" int nsa_ragged_extend_metadata(
    const int32_t* cu_seqlens_k, const int32_t* cache_seqlens, int bs,
    const int32_t* seqlens_expanded, const int32_t* token_to_req, int T,
    const int32_t* real_page_table, int64_t rpt_stride, int max_seqlen_k,
    int32_t* ks, int32_t* ke, int32_t* topk_indices_offset,
    int32_t* page_table_1_flattened, int64_t flat_capacity, void* stream) {
  const char* fn = "nsa_ragged_extend_metadata";
  NSA_REQUIRE(bs >= 0 && T >= 0 && max_seqlen_k >= 0 && flat_capacity >= 0,
              NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  hipStream_t s = (hipStream_t)stream;
  if (T > 0) {
    NSA_REQUIRE(cu_seqlens_k && seqlens_expanded && token_to_req && ks && ke,
                NSA_ERR_INVALID_ARG, "%s: null per-row pointer", fn);
    hipLaunchKernelGGL(ragged_rows_kernel, dim3((unsigned)((T + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, cu_seqlens_k, bs, seqlens_expanded,
                       token_to_req, T, ks, ke, topk_indices_offset);
    const int st = nsa::check_launch(fn);
    if (st != NSA_OK) return st;
  }
  if (page_table_1_flattened != nullptr && bs > 0 && max_seqlen_k > 0) {
    NSA_REQUIRE(cu_seqlens_k && cache_seqlens && real_page_table, NSA_ERR_INVALID_ARG,
                "%s: null table input", fn);
    NSA_REQUIRE(rpt_stride >= (max_seqlen_k + NSA_PAGE_SIZE - 1) / NSA_PAGE_SIZE,
                NSA_ERR_INVALID_ARG, "%s: rpt_stride < ceil(max_seqlen_k/64)", fn);
    const int chunks = (max_seqlen_k + kSpan - 1) / kSpan;
    NSA_REQUIRE((int64_t)bs * chunks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: grid too large", fn);
    hipLaunchKernelGGL(ragged_flat_table_kernel, dim3((unsigned)(bs * chunks)),
                       dim3(kThreads), 0, s, cu_seqlens_k, cache_seqlens,
                       real_page_table, rpt_stride, max_seqlen_k, chunks,
                       flat_capacity, page_table_1_flattened);
    return nsa::check_launch(fn);
  }
  return nsa::ok();
}

extern "C" int nsa_ragged_index_transform(const int32_t* topk_indices,
                                          int64_t in_stride, int T, int topk,
                                          const int32_t* offset, int32_t* out,
                                          int64_t out_stride, void* stream) {
  const char* fn = "nsa_ragged_index_transform";
  NSA_REQUIRE(T >= 0 && topk >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (T == 0 || topk == 0) return nsa::ok();
  NSA_REQUIRE(topk_indices && offset && out, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(in_stride >= topk && out_stride >= topk, NSA_ERR_INVALID_ARG,
              "%s: stride < topk", fn);
  const int64_t n = (int64_t)T * topk;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many entries", fn);
  hipLaunchKernelGGL(ragged_index_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, topk_indices, in_stride, T, topk, offset,
                     out, out_stride);
  return nsa::check_launch(fn);
}

extern "C" int nsa_valid_kv_indices(const int32_t* indices, int64_t idx_stride,
                                    int T, int topk, int32_t* kv_indptr,
                                    int32_t* kv_indices, int64_t capacity,
                                    void* stream) {
  const char* fn = "nsa_valid_kv_indices";
  NSA_REQUIRE(T >= 0 && topk >= 0 && capacity >= 0, NSA_ERR_INVALID_ARG,
              "%s: negative size", fn);
  NSA_REQUIRE(kv_indptr != nullptr, NSA_ERR_INVALID_ARG, "%s: null kv_indptr", fn);
  NSA_REQUIRE(T == 0 || (indices && idx_stride >= topk), NSA_ERR_INVALID_ARG,
              "%s: null indices or stride < topk", fn);
  NSA_REQUIRE(capacity == 0 || kv_indices, NSA_ERR_INVALID_ARG, "%s: null kv_indices", fn);
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {   // kv_indptr = [0]
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, kv_indptr, 0);
    return nsa::check_launch(fn);
  }
  hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)T), dim3(kThreads), 0, s,
                     indices, idx_stride, topk, kv_indptr);
  int st = nsa::check_launch(fn);
  if (st != NSA_OK) return st;
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, kv_indptr, T);
  st = nsa::check_launch(fn);
  if (st != NSA_OK) return st;
  hipLaunchKernelGGL(csr_write_kernel, dim3((unsigned)T), dim3(kThreads), 0, s,
                     indices, idx_stride, topk, kv_indptr, capacity, kv_indices);
  return nsa::check_launch(fn);
}
