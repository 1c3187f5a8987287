// a0: per-forward metadata of the sparse attention step in one launch.
//
// Follows the metadata construction of "nsa_backend.py (EngineX-Hygon sglang
// fork)" (NSAMetadata, compute_cu_seqlens, _transform_table_1_to_real,
// NativeSparseAttnBackend.init_forward_metadata) and "dsa_backend.py (sglang
// main)" (DeepseekSparseAttnBackend.init_forward_metadata: decode,
// target-verify, draft-extend and extend branches). The pages build these tensors with a
// chain of torch ops plus a host sync for max(seq_lens); here one kernel
// writes all of them with the bound given by the host.
//
// Launch shape: one 256-thread block per request for the lengths, then one
// block per (request, 256 page columns) for the page tables (a block per
// request alone gathering 2048 strided entries was bound by one CU's memory
// throughput). A request's block needs three
// exclusive prefix sums over the requests before it (KV lengths, query
// rows, clipped lengths); it recomputes them itself (O(bs) per block), which
// avoids a second launch or a grid-wide barrier. The clipped-length sum of
// one request has a closed form: its query rows see a, a+1, ..., a+n-1 KV
// tokens, so sum_j min(a+j, K) = m*a + m(m-1)/2 + (n-m)*K with
// m = clamp(K-a, 0, n).
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBatch = 16384;

__device__ __forceinline__ long long clipped_sum(long long a, long long n,
                                                 long long k) {
  long long m = k - a;
  m = m < 0 ? 0 : (m > n ? n : m);
  return m * a + m * (m - 1) / 2 + (n - m) * k;
}

__device__ __forceinline__ int q_rows_of(int mode, int draft,
                                         const int32_t* extend_lens, int i) {
  if (mode == NSA_MODE_DECODE) return 1;
  if (mode == NSA_MODE_TARGET_VERIFY || mode == NSA_MODE_DRAFT_EXTEND_V2) return draft;
  return extend_lens[i];   // EXTEND, DRAFT_EXTEND
}

// Block-wide sums of three values: wave reductions with shuffles, then one
// exchange through LDS.
__device__ void block_sum3(long long& a, long long& b, long long& c, long long* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
    c += __shfl_xor(c, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[3 * wave] = a; red[3 * wave + 1] = b; red[3 * wave + 2] = c; }
  __syncthreads();
  a = b = c = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {   // fixed order: every thread gets the same sums
    a += red[3 * w];
    b += red[3 * w + 1];
    c += red[3 * w + 2];
  }
}

__global__ void __launch_bounds__(kThreads)
build_metadata_kernel(int mode, int bs, int draft, int topk,
                      const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ extend_lens,
                      const int32_t* __restrict__ req_to_token,
                      int64_t rtt_stride, int64_t pool_rows,
                      const int32_t* __restrict__ req_pool_indices,
                      int max_seqlen_k, int T, int32_t* cache_seqlens,
                      int32_t* cu_seqlens_k, int32_t* cu_seqlens_q,
                      int32_t* seqlens_expanded, int32_t* nsa_cache_seqlens,
                      int32_t* nsa_cu_seqlens_k, int32_t* nsa_cu_seqlens_q,
                      int32_t* real_page_table, int64_t rpt_stride,
                      int32_t* token_to_req, int32_t* page_table_1,
                      int64_t pt1_stride) {
  __shared__ long long red[3 * (kThreads / 64)];
  const int tid = threadIdx.x;
  const int nreq_blocks = bs > 0 ? bs : 1;
  if ((int)blockIdx.x >= nreq_blocks) {
    // page tables: request r, page columns c*kThreads .. (one per thread);
    // the compact entry is every 64th token slot divided by 64 (arithmetic
    // shift = floor division), the wide table copies the 64 token slots
    const int ncols = (max_seqlen_k + NSA_PAGE_SIZE - 1) / NSA_PAGE_SIZE;
    const int chunks = (ncols + kThreads - 1) / kThreads;
    const int b = blockIdx.x - nreq_blocks;
    const int r = b / chunks, c = b % chunks;
    // a pool row outside req_to_token gives -1 (absent) entries
    const int32_t pr = req_pool_indices[r];
    const bool pr_ok = pr >= 0 && pr < pool_rows;
    if (!pr_ok && c == 0 && tid == 0) flag_device_error(NSA_DEVERR_POOL_ROW);
    const int32_t* row = req_to_token + (int64_t)(pr_ok ? pr : 0) * rtt_stride;
    const int p = c * kThreads + tid;
    if (p < ncols)
      real_page_table[(int64_t)r * rpt_stride + p] = pr_ok ? row[(int64_t)p * NSA_PAGE_SIZE] >> 6 : -1;
    if (page_table_1 != nullptr) {
      int32_t* pt = page_table_1 + (int64_t)r * pt1_stride;
      const int c0 = c * kThreads * NSA_PAGE_SIZE;
      const int c1 = min(c0 + kThreads * NSA_PAGE_SIZE, max_seqlen_k);
      for (int k = c0 + tid; k < c1; k += kThreads) pt[k] = pr_ok ? row[k] : -1;
    }
    return;
  }
  const int r = blockIdx.x;
  const int d = (mode == NSA_MODE_TARGET_VERIFY) ? draft : 0;

  // exclusive prefix sums over requests 0..r-1
  long long pk = 0, pq = 0, pn = 0;
  const int upto = r < bs ? r : bs;
  for (int i = tid; i < upto; i += kThreads) {
    const long long kv = (long long)seq_lens[i] + d;
    const long long ql = q_rows_of(mode, draft, extend_lens, i);
    pk += kv;
    pq += ql;
    pn += clipped_sum(kv - ql + 1, ql, topk);
  }
  block_sum3(pk, pq, pn, red);

  if (r == 0 && tid == 0) {
    cu_seqlens_k[0] = 0;
    cu_seqlens_q[0] = 0;
    nsa_cu_seqlens_k[0] = 0;
    nsa_cu_seqlens_q[0] = 0;
  }
  if (r >= bs) return;

  const int kv = seq_lens[r] + d;
  const int ql = q_rows_of(mode, draft, extend_lens, r);
  const long long a = (long long)kv - ql + 1;  // visible length of row 0
  if (tid == 0) {
    cache_seqlens[r] = kv;
    cu_seqlens_k[r + 1] = (int32_t)(pk + kv);
    if (mode == NSA_MODE_EXTEND) cu_seqlens_q[r + 1] = (int32_t)(pq + ql);
  }
  for (int j = tid; j < ql; j += kThreads) {
    const long long t = pq + j;
    if (t >= T) break;
    const long long se = a + j;
    seqlens_expanded[t] = (int32_t)se;
    nsa_cache_seqlens[t] = (int32_t)(se < topk ? se : topk);
    nsa_cu_seqlens_k[t + 1] = (int32_t)(pn + clipped_sum(a, j + 1, topk));
    nsa_cu_seqlens_q[t + 1] = (int32_t)(t + 1);
    token_to_req[t] = r;
    if (mode != NSA_MODE_EXTEND) cu_seqlens_q[t + 1] = (int32_t)(t + 1);
  }
  // extend modes: the rows from the end of the last request up to T (a host
  // bound above sum(extend_lens)) become empty rows of request 0
  if (r == bs - 1) {
    const long long t_end = pq + ql;
    const long long n_end = pn + clipped_sum(a, ql, topk);
    for (long long t = t_end + tid; t < T; t += kThreads) {
      seqlens_expanded[t] = 0;
      nsa_cache_seqlens[t] = 0;
      nsa_cu_seqlens_k[t + 1] = (int32_t)n_end;
      nsa_cu_seqlens_q[t + 1] = (int32_t)(t + 1);
      token_to_req[t] = 0;
      if (mode != NSA_MODE_EXTEND) cu_seqlens_q[t + 1] = (int32_t)(t + 1);
    }
  }
}

}  // namespace

extern "C" int nsa_build_metadata(
    int mode, int bs, int draft_token_num, int topk, int page_size,
    const int32_t* seq_lens, const int32_t* extend_lens,
    const int32_t* req_to_token, int64_t rtt_stride, int64_t pool_rows,
    const int32_t* req_pool_indices, int max_seqlen_k, int num_q_rows,
    int32_t* cache_seqlens, int32_t* cu_seqlens_k, int32_t* cu_seqlens_q,
    int32_t* seqlens_expanded, int32_t* nsa_cache_seqlens,
    int32_t* nsa_cu_seqlens_k, int32_t* nsa_cu_seqlens_q,
    int32_t* real_page_table, int64_t rpt_stride, int32_t* token_to_req,
    int32_t* page_table_1, int64_t pt1_stride, void* stream) {
  const char* fn = "nsa_build_metadata";
  NSA_REQUIRE(mode >= NSA_MODE_DECODE && mode <= NSA_MODE_DRAFT_EXTEND_V2,
              NSA_ERR_INVALID_ARG, "%s: unknown mode %d", fn, mode);
  NSA_REQUIRE(bs >= 0 && bs <= kMaxBatch, NSA_ERR_UNSUPPORTED,
              "%s: bs %d outside [0, %d]", fn, bs, kMaxBatch);
  NSA_REQUIRE(topk > 0, NSA_ERR_INVALID_ARG, "%s: topk %d <= 0", fn, topk);
  NSA_REQUIRE(page_size == NSA_PAGE_SIZE, NSA_ERR_UNSUPPORTED,
              "%s: page_size %d (only 64 is supported)", fn, page_size);
  NSA_REQUIRE(max_seqlen_k >= 0 && num_q_rows >= 0, NSA_ERR_INVALID_ARG,
              "%s: negative max_seqlen_k or num_q_rows", fn);
  if (mode == NSA_MODE_TARGET_VERIFY || mode == NSA_MODE_DRAFT_EXTEND_V2) {
    NSA_REQUIRE(draft_token_num >= 1, NSA_ERR_INVALID_ARG,
                "%s: mode %d needs draft_token_num >= 1", fn, mode);
    NSA_REQUIRE((int64_t)num_q_rows == (int64_t)bs * draft_token_num,
                NSA_ERR_INVALID_ARG,
                "%s: num_q_rows %d != bs * draft_token_num", fn, num_q_rows);
  } else if (mode == NSA_MODE_DECODE) {
    NSA_REQUIRE(num_q_rows == bs, NSA_ERR_INVALID_ARG,
                "%s: decode needs num_q_rows == bs", fn);
  } else {
    NSA_REQUIRE(extend_lens != nullptr, NSA_ERR_INVALID_ARG,
                "%s: extend and draft-extend need extend_lens", fn);
    NSA_REQUIRE(bs > 0 || num_q_rows == 0, NSA_ERR_INVALID_ARG,
                "%s: an empty batch has no query rows", fn);
  }
  // buffers of zero length may be NULL (an empty batch has no rows)
  NSA_REQUIRE(cu_seqlens_k && cu_seqlens_q && nsa_cu_seqlens_k && nsa_cu_seqlens_q,
              NSA_ERR_INVALID_ARG, "%s: null cumulative-length output", fn);
  NSA_REQUIRE(bs == 0 || (cache_seqlens && (real_page_table || max_seqlen_k == 0)),
              NSA_ERR_INVALID_ARG, "%s: null per-request output", fn);
  NSA_REQUIRE(num_q_rows == 0 || (seqlens_expanded && nsa_cache_seqlens && token_to_req),
              NSA_ERR_INVALID_ARG, "%s: null per-row output", fn);
  NSA_REQUIRE(bs == 0 || (seq_lens && req_to_token && req_pool_indices),
              NSA_ERR_INVALID_ARG, "%s: null input pointer", fn);
  const int64_t ncols = (max_seqlen_k + NSA_PAGE_SIZE - 1) / NSA_PAGE_SIZE;
  NSA_REQUIRE(rtt_stride >= max_seqlen_k, NSA_ERR_INVALID_ARG,
              "%s: rtt_stride %lld < max_seqlen_k %d", fn,
              (long long)rtt_stride, max_seqlen_k);
  NSA_REQUIRE(rpt_stride >= ncols, NSA_ERR_INVALID_ARG,
              "%s: rpt_stride %lld < ceil(max_seqlen_k/64) = %lld", fn,
              (long long)rpt_stride, (long long)ncols);
  NSA_REQUIRE(page_table_1 == nullptr || pt1_stride >= max_seqlen_k,
              NSA_ERR_INVALID_ARG, "%s: pt1_stride < max_seqlen_k", fn);
  NSA_REQUIRE(bs == 0 || pool_rows >= 1, NSA_ERR_INVALID_ARG,
              "%s: pool_rows %lld < 1", fn, (long long)pool_rows);

  const int64_t chunks = (ncols + kThreads - 1) / kThreads;
  const int64_t grid = (bs > 0 ? bs : 1) + (int64_t)bs * chunks;
  NSA_REQUIRE(grid < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  hipLaunchKernelGGL(build_metadata_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, mode, bs, draft_token_num, topk,
                     seq_lens, extend_lens, req_to_token, rtt_stride,
                     pool_rows, req_pool_indices, max_seqlen_k, num_q_rows, cache_seqlens,
                     cu_seqlens_k, cu_seqlens_q, seqlens_expanded,
                     nsa_cache_seqlens, nsa_cu_seqlens_k, nsa_cu_seqlens_q,
                     real_page_table, rpt_stride, token_to_req, page_table_1,
                     pt1_stride);
  return nsa::check_launch(fn);
}
