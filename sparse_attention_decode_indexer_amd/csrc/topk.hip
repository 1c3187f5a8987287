// a2 (+ a3 fused): length-masked top-k of the indexer logits.
//
// "nsa_backend.py (EngineX-Hygon sglang fork)", NSAIndexerMetadata.
// topk_transform: fast_topk_v2(logits, lengths=seqlens_expanded, topk) keeps
// at most topk positions per row ("clipped to topk", NSAMetadata); the fused
// variant fast_topk_transform_fused returns physical slots through the page
// table instead of logical positions.
//
// Method (MI355X design, one 1024-thread block per row):
//   * rows with n <= topk keep 0..n-1 (no logits are read);
//   * otherwise a radix select on the order-preserving uint32 image of the
//     fp32 logits (NaN -> lowest) finds the topk-th largest key in at most
//     three histogram passes (11, 11, 10 bits) over the row, stopping early
//     when the threshold bin is taken whole;
//   * a final pass writes every key above the threshold and the first
//     (lowest-position) keys equal to it, in ascending position order, using
//     block-wide prefix sums so the result is deterministic.
// The row (<= 512 KB) is re-read from L2/MALL by each pass.
#include "common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

// Order-preserving image of a float in uint32: NaN ranks lowest and -0.0
// equals +0.0 (so equal values tie and are broken by position).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = x == 0.0f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Calls f(i, key) for every i in [0, n), 4 consecutive elements per thread
// per iteration (float4 loads when the row is 16-byte aligned).
template <typename F>
__device__ __forceinline__ void for_each_key(const float* row, int n, bool vec,
                                             F&& f) {
  for (int base = threadIdx.x * 4; base < n; base += kThreads * 4) {
    if (vec && base + 4 <= n) {
      const float4 v = *reinterpret_cast<const float4*>(row + base);
      f(base, order_key(v.x));
      f(base + 1, order_key(v.y));
      f(base + 2, order_key(v.z));
      f(base + 3, order_key(v.w));
    } else {
      for (int k = 0; k < 4 && base + k < n; ++k) f(base + k, order_key(row[base + k]));
    }
  }
}

// Exclusive block-wide prefix sum of v; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot,
                                                    int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? wave_tot[lane] : 0;
    int s = w;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < kWaves) wave_tot[kWaves + lane] = s - w;  // exclusive
    if (lane == kWaves - 1) wave_tot[2 * kWaves] = s;
  }
  __syncthreads();
  const int res = wave_tot[kWaves + wave] + x - v;
  *total = wave_tot[2 * kWaves];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(kThreads)
topk_transform_kernel(const float* __restrict__ logits, int64_t logits_stride,
                      const int32_t* __restrict__ lengths, int topk,
                      int max_seqlen_k, const int32_t* __restrict__ table,
                      int64_t table_stride, const int32_t* __restrict__ t2r,
                      int32_t* __restrict__ out, int64_t out_stride,
                      bool vec_ok) {
  __shared__ uint32_t hist[kBins];
  __shared__ int scan_buf[2 * kWaves + 1];
  __shared__ uint32_t s_sel[3];  // bin, remaining k, exact-fit flag

  const int64_t t = blockIdx.x;
  int n = lengths[t];
  n = n < 0 ? 0 : (n > max_seqlen_k ? max_seqlen_k : n);
  int32_t* orow = out + t * out_stride;
  const int32_t* trow = table ? table + (int64_t)t2r[t] * table_stride : nullptr;
  auto map = [&](int i) -> int32_t {
    return trow ? (trow[i >> 6] << 6) + (i & 63) : i;
  };

  if (n <= topk) {
    for (int j = threadIdx.x; j < topk; j += kThreads) orow[j] = j < n ? map(j) : -1;
    return;
  }

  const float* row = logits + t * logits_stride;
  const bool vec = vec_ok;
  uint32_t prefix = 0, pmask = 0;
  int krem = topk;

  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = threadIdx.x; b < nb; b += kThreads) hist[b] = 0;
    __syncthreads();
    for_each_key(row, n, vec, [&](int, uint32_t k) {
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
    });
    __syncthreads();
    // wave 0 finds the bin holding the krem-th largest key: lanes own
    // descending chunks of bins, scan their chunk sums, then the crossing
    // lane walks its chunk.
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int per = nb / 64;
      const int hi_bin = nb - 1 - lane * per;  // chunk = [hi_bin-per+1, hi_bin]
      uint32_t csum = 0;
      for (int b = 0; b < per; ++b) csum += hist[hi_bin - b];
      uint32_t incl = csum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const uint32_t excl = incl - csum;
      if (excl < (uint32_t)krem && incl >= (uint32_t)krem) {
        uint32_t above = excl;
        for (int b = 0; b < per; ++b) {
          const uint32_t c = hist[hi_bin - b];
          if (above + c >= (uint32_t)krem) {
            s_sel[0] = hi_bin - b;
            s_sel[1] = krem - above;
            s_sel[2] = (above + c == (uint32_t)krem) ? 1u : 0u;
            break;
          }
          above += c;
        }
      }
    }
    __syncthreads();
    const uint32_t bin = s_sel[0];
    krem = (int)s_sel[1];
    const bool exact = s_sel[2] != 0;
    prefix |= bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
    if (exact) break;
  }

  // collect: keys above the threshold prefix, and the first krem equal ones
  int eq_run = 0, sel_run = 0;
  for (int base0 = 0; base0 < n; base0 += kThreads * 4) {
    const int base = base0 + threadIdx.x * 4;
    uint32_t keys[4];
    int cnt = 0;
    if (vec && base + 4 <= n) {
      const float4 v = *reinterpret_cast<const float4*>(row + base);
      keys[0] = order_key(v.x); keys[1] = order_key(v.y);
      keys[2] = order_key(v.z); keys[3] = order_key(v.w);
      cnt = 4;
    } else {
      for (int k = 0; k < 4; ++k) {
        if (base + k < n) { keys[k] = order_key(row[base + k]); cnt = k + 1; }
        else keys[k] = 0;
      }
    }
    int gt[4], eq[4], neq = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t mk = keys[k] & pmask;
      gt[k] = (k < cnt) && mk > prefix;
      eq[k] = (k < cnt) && mk == prefix;
      neq += eq[k];
    }
    int eq_tot;
    const int eq_before = eq_run + block_exclusive_scan(neq, scan_buf, &eq_tot);
    int sel[4], nsel = 0, e = eq_before;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sel[k] = gt[k] || (eq[k] && e < krem);
      e += eq[k];
      nsel += sel[k];
    }
    int sel_tot;
    int pos = sel_run + block_exclusive_scan(nsel, scan_buf, &sel_tot);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (sel[k] && pos < topk) orow[pos++] = map(base + k);
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
}

}  // namespace

extern "C" int nsa_topk_workspace_size(int T, int max_seqlen_k, int topk,
                                       size_t* bytes) {
  NSA_REQUIRE(bytes != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_topk_workspace_size: null output");
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0 && topk >= 0, NSA_ERR_INVALID_ARG,
              "nsa_topk_workspace_size: negative size");
  *bytes = 0;  // the single-block-per-row select keeps its state in LDS
  return nsa::ok();
}

extern "C" int nsa_topk_transform(const float* logits, int64_t logits_stride,
                                  const int32_t* lengths, int T, int topk,
                                  int max_seqlen_k, const int32_t* table,
                                  int64_t table_stride,
                                  const int32_t* token_to_req, int page_size,
                                  int32_t* out, int64_t out_stride,
                                  void* workspace, size_t ws_bytes,
                                  void* stream) {
  (void)workspace;
  (void)ws_bytes;
  const char* fn = "nsa_topk_transform";
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG,
              "%s: negative size", fn);
  NSA_REQUIRE(topk > 0, NSA_ERR_INVALID_ARG, "%s: topk must be positive", fn);
  NSA_REQUIRE(page_size == NSA_PAGE_SIZE, NSA_ERR_UNSUPPORTED,
              "%s: page_size %d (only 64 is supported)", fn, page_size);
  if (T == 0) return nsa::ok();
  NSA_REQUIRE(lengths && out, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(max_seqlen_k <= topk || logits != nullptr, NSA_ERR_INVALID_ARG,
              "%s: null logits", fn);
  NSA_REQUIRE(logits == nullptr || logits_stride >= max_seqlen_k,
              NSA_ERR_INVALID_ARG, "%s: logits_stride < max_seqlen_k", fn);
  NSA_REQUIRE(out_stride >= topk, NSA_ERR_INVALID_ARG, "%s: out_stride < topk",
              fn);
  if (table != nullptr) {
    NSA_REQUIRE(token_to_req != nullptr, NSA_ERR_INVALID_ARG,
                "%s: a table needs token_to_req", fn);
    NSA_REQUIRE(table_stride >= (max_seqlen_k + 63) / 64, NSA_ERR_INVALID_ARG,
                "%s: table_stride < ceil(max_seqlen_k/64)", fn);
  }
  const bool vec = logits && nsa::aligned(logits, 16) && logits_stride % 4 == 0;
  hipLaunchKernelGGL(topk_transform_kernel, dim3(T), dim3(kThreads), 0,
                     (hipStream_t)stream, logits, logits_stride, lengths, topk,
                     max_seqlen_k, table, table_stride, token_to_req, out,
                     out_stride, vec);
  return nsa::check_launch(fn);
}
