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

// Wave 0 finds the bin holding the krem-th largest key of an LDS histogram of
// nb bins (nb a multiple of 64): lanes own descending chunks of bins, scan the
// chunk sums, then the crossing lane walks its chunk. Publishes
// s_sel = {bin, krem - count above the bin, bin taken whole}.
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, int nb,
                                                   int krem, uint32_t* s_sel) {
  if (threadIdx.x >= 64) return;
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

// Multi-pass radix select over the row in global memory: the general path,
// used when the threshold bin of the first-pass histogram holds too many
// candidates for LDS (heavy ties) or topk exceeds the fast path's lists.
// Writes exactly topk entries of out_row (n > topk), ascending positions.
template <typename Map>
__device__ void select_multipass(const float* row, int n, bool vec, int topk,
                                 int32_t* orow, Map&& map, uint32_t* hist,
                                 int* scan_buf, uint32_t* s_sel) {
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
    find_threshold_bin(hist, nb, krem, s_sel);
    __syncthreads();
    const uint32_t bin = s_sel[0];
    krem = (int)s_sel[1];
    const bool exact = s_sel[2] != 0;
    prefix |= bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
    if (exact) break;
  }
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

constexpr int kChunk = 16384;       // positions per histogram block
constexpr int kHistBins = 4096;     // first digit: key bits 31..20
constexpr int kHistThreads = 256;
constexpr int kMaxAbove = 2048;     // fast path: topk <= 2048
constexpr int kCap = 12288;         // fast path: threshold-bin candidates in LDS

// Pass 1: per-(row, chunk) histogram of the top 12 key bits, over all CUs.
// Each wave counts into its own LDS sub-histogram; the block writes 4096
// 16-bit counts (a chunk holds at most 16384 positions).
__global__ void __launch_bounds__(kHistThreads)
topk_hist_kernel(const float* __restrict__ logits, int64_t logits_stride,
                 const int32_t* __restrict__ lengths, int topk,
                 int max_seqlen_k, int chunks, uint16_t* __restrict__ ws,
                 bool vec) {
  __shared__ uint32_t sub[4][kHistBins];
  const int64_t t = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  int n = lengths[t];
  n = n < 0 ? 0 : (n > max_seqlen_k ? max_seqlen_k : n);
  const int start = c * kChunk;
  if (n <= topk || start >= n) return;
  const int end = min(start + kChunk, n);
  const int wave = threadIdx.x >> 6;
  uint4* z = reinterpret_cast<uint4*>(&sub[0][0]);
  for (int i = threadIdx.x; i < 4 * kHistBins / 4; i += kHistThreads)
    z[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const float* row = logits + t * logits_stride;
  uint32_t* h = sub[wave];
  // all 64 positions of a thread are loaded before any is counted; load k
  // of the block covers 1024 consecutive positions
  constexpr int kPer = kChunk / kHistThreads / 4;   // 16 float4 per thread
  float4 v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int pos = start + k * (kHistThreads * 4) + threadIdx.x * 4;
    if (vec && pos + 4 <= end) {
      v[k] = *reinterpret_cast<const float4*>(row + pos);
    } else {
      v[k].x = pos < end ? row[pos] : 0.0f;
      v[k].y = pos + 1 < end ? row[pos + 1] : 0.0f;
      v[k].z = pos + 2 < end ? row[pos + 2] : 0.0f;
      v[k].w = pos + 3 < end ? row[pos + 3] : 0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int pos = start + k * (kHistThreads * 4) + threadIdx.x * 4;
    if (pos < end) atomicAdd(&h[order_key(v[k].x) >> 20], 1u);
    if (pos + 1 < end) atomicAdd(&h[order_key(v[k].y) >> 20], 1u);
    if (pos + 2 < end) atomicAdd(&h[order_key(v[k].z) >> 20], 1u);
    if (pos + 3 < end) atomicAdd(&h[order_key(v[k].w) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(ws + (t * chunks + c) * kHistBins);
  for (int b2 = threadIdx.x; b2 < kHistBins / 2; b2 += kHistThreads) {
    const int b = 2 * b2;
    const uint32_t lo = sub[0][b] + sub[1][b] + sub[2][b] + sub[3][b];
    const uint32_t hi = sub[0][b + 1] + sub[1][b + 1] + sub[2][b + 1] + sub[3][b + 1];
    dst[b2] = lo | (hi << 16);
  }
}

// Pass 2: one block per row. Sums the row's chunk histograms, finds the
// threshold bin, then in one ordered pass over the row collects the
// positions above it (list A) and the (key, position) candidates inside it
// (list B) in LDS; resolves the exact threshold among the candidates with two
// more 10-bit radix passes in LDS; merges A with the chosen candidates in
// position order and writes them (through the page table when given).
__global__ void __launch_bounds__(kThreads)
topk_select_kernel(const float* __restrict__ logits, int64_t logits_stride,
                   const int32_t* __restrict__ lengths, int topk,
                   int max_seqlen_k, int chunks,
                   const uint16_t* __restrict__ ws,
                   const int32_t* __restrict__ table, int64_t table_stride,
                   const int32_t* __restrict__ t2r, int32_t* __restrict__ out,
                   int64_t out_stride, bool vec) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int32_t list_a[kMaxAbove];
  __shared__ int32_t sel_b[kMaxAbove];
  __shared__ uint32_t cand_key[kCap];
  __shared__ int32_t cand_pos[kCap];
  __shared__ int scan_buf[2 * kWaves + 1];
  __shared__ uint32_t s_sel[3];

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

  // ---- row histogram of the top 12 key bits and its threshold bin
  const int nch = (n + kChunk - 1) / kChunk;
  const uint16_t* hrow = ws + t * chunks * kHistBins;
  for (int b = threadIdx.x; b < kHistBins; b += kThreads) {
    uint32_t s = 0;
    for (int c = 0; c < nch; ++c) s += hrow[c * kHistBins + b];
    hist[b] = s;
  }
  __syncthreads();
  find_threshold_bin(hist, kHistBins, topk, s_sel);
  __syncthreads();
  const uint32_t bin = s_sel[0];
  int krem = (int)s_sel[1];
  const uint32_t cnt_b = hist[bin];
  __syncthreads();
  if (topk > kMaxAbove || cnt_b > (uint32_t)kCap) {
    select_multipass(row, n, vec, topk, orow, map, hist, scan_buf, s_sel);
    return;
  }

  // ---- one ordered pass: 32 consecutive positions per thread per round; the
  // next round's loads are issued before this round's scan
  constexpr int kRun = 32;
  constexpr int kRound = kThreads * kRun;
  auto load_round = [&](float4* v, int b0) {
    const int base = b0 + threadIdx.x * kRun;
#pragma unroll
    for (int k = 0; k < kRun / 4; ++k) {
      const int pos = base + 4 * k;
      if (vec && pos + 4 <= n) {
        v[k] = *reinterpret_cast<const float4*>(row + pos);
      } else {
        v[k].x = pos < n ? row[pos] : 0.0f;
        v[k].y = pos + 1 < n ? row[pos + 1] : 0.0f;
        v[k].z = pos + 2 < n ? row[pos + 2] : 0.0f;
        v[k].w = pos + 3 < n ? row[pos + 3] : 0.0f;
      }
    }
  };
  int na = 0, nb = 0;
  float4 cur[kRun / 4], nxt[kRun / 4];
  load_round(cur, 0);
  for (int base0 = 0; base0 < n; base0 += kRound) {
    if (base0 + kRound < n) load_round(nxt, base0 + kRound);
    const int base = base0 + threadIdx.x * kRun;
    uint32_t kb[kRun];
#pragma unroll
    for (int k = 0; k < kRun / 4; ++k) {
      kb[4 * k] = order_key(cur[k].x); kb[4 * k + 1] = order_key(cur[k].y);
      kb[4 * k + 2] = order_key(cur[k].z); kb[4 * k + 3] = order_key(cur[k].w);
    }
    int ga = 0, gb = 0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const uint32_t d = kb[k] >> 20;
      const bool in = base + k < n;
      ga += (in && d > bin);
      gb += (in && d == bin);
    }
    int tot;
    const int off = block_exclusive_scan(ga | (gb << 16), scan_buf, &tot);
    int pa = na + (off & 0xFFFF), pb = nb + (off >> 16);
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const uint32_t d = kb[k] >> 20;
      if (base + k < n) {
        if (d > bin) {
          if (pa < kMaxAbove) list_a[pa] = base + k;
          ++pa;
        } else if (d == bin) {
          if (pb < kCap) { cand_key[pb] = kb[k]; cand_pos[pb] = base + k; }
          ++pb;
        }
      }
    }
    na += tot & 0xFFFF;
    nb += tot >> 16;
#pragma unroll
    for (int k = 0; k < kRun / 4; ++k) cur[k] = nxt[k];
  }
  __syncthreads();
  na = min(na, kMaxAbove);
  nb = min(nb, kCap);

  // ---- exact threshold among the candidates (bits 19..10, then 9..0)
  uint32_t prefix = bin << 20, pmask = 0xFFF00000u;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    for (int b = threadIdx.x; b < 1024; b += kThreads) hist[b] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kThreads) {
      const uint32_t k = cand_key[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1u);
    }
    __syncthreads();
    find_threshold_bin(hist, 1024, krem, s_sel);
    __syncthreads();
    const uint32_t b2 = s_sel[0];
    krem = (int)s_sel[1];
    const bool exact = s_sel[2] != 0;
    prefix |= b2 << shift;
    pmask |= 1023u << shift;
    __syncthreads();
    if (exact) break;
  }

  // ---- chosen candidates, in position order
  int eq_run = 0, nsel = 0;
  for (int i0 = 0; i0 < nb; i0 += kThreads) {
    const int i = i0 + threadIdx.x;
    const uint32_t mk = i < nb ? (cand_key[i] & pmask) : 0u;
    const int gt = i < nb && mk > prefix;
    const int eq = i < nb && mk == prefix;
    int eq_tot;
    const int er = eq_run + block_exclusive_scan(eq, scan_buf, &eq_tot);
    const int sel = gt || (eq && er < krem);
    int sel_tot;
    const int ps = nsel + block_exclusive_scan(sel, scan_buf, &sel_tot);
    if (sel && ps < kMaxAbove) sel_b[ps] = cand_pos[i];
    eq_run += eq_tot;
    nsel += sel_tot;
  }
  __syncthreads();
  nsel = min(nsel, kMaxAbove);

  // ---- merge the two position-sorted lists: rank = own index + number of
  // smaller entries in the other list
  for (int i = threadIdx.x; i < na; i += kThreads) {
    const int v = list_a[i];
    int lo = 0, hi = nsel;
    while (lo < hi) { const int m = (lo + hi) >> 1; if (sel_b[m] < v) lo = m + 1; else hi = m; }
    const int r = i + lo;
    if (r < topk) orow[r] = map(v);
  }
  for (int j = threadIdx.x; j < nsel; j += kThreads) {
    const int v = sel_b[j];
    int lo = 0, hi = na;
    while (lo < hi) { const int m = (lo + hi) >> 1; if (list_a[m] < v) lo = m + 1; else hi = m; }
    const int r = j + lo;
    if (r < topk) orow[r] = map(v);
  }
}

}  // namespace

extern "C" int nsa_topk_workspace_size(int T, int max_seqlen_k, int topk,
                                       size_t* bytes) {
  NSA_REQUIRE(bytes != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_topk_workspace_size: null output");
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0 && topk >= 0, NSA_ERR_INVALID_ARG,
              "nsa_topk_workspace_size: negative size");
  // 16-bit first-digit histograms of every (row, chunk)
  const size_t chunks = (size_t)(max_seqlen_k + kChunk - 1) / kChunk;
  *bytes = max_seqlen_k > topk ? (size_t)T * chunks * kHistBins * sizeof(uint16_t) : 0;
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
  size_t need = 0;
  nsa_topk_workspace_size(T, max_seqlen_k, topk, &need);
  NSA_REQUIRE(need == 0 || (workspace != nullptr && ws_bytes >= need),
              NSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
              fn, need, ws_bytes);
  NSA_REQUIRE(need == 0 || nsa::aligned(workspace, 16), NSA_ERR_INVALID_ARG,
              "%s: workspace must be 16-byte aligned", fn);
  const bool vec = logits && nsa::aligned(logits, 16) && logits_stride % 4 == 0;
  const int chunks = (max_seqlen_k + kChunk - 1) / kChunk;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* ws = static_cast<uint16_t*>(workspace);
  if (need > 0) {
    const int64_t hb = (int64_t)T * chunks;
    NSA_REQUIRE(hb < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
    hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)hb), dim3(kHistThreads), 0,
                       s, logits, logits_stride, lengths, topk, max_seqlen_k,
                       chunks, ws, vec);
    int st = nsa::check_launch(fn);
    if (st != NSA_OK) return st;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3(T), dim3(kThreads), 0, s, logits,
                     logits_stride, lengths, topk, max_seqlen_k, chunks, ws,
                     table, table_stride, token_to_req, out, out_stride, vec);
  return nsa::check_launch(fn);
}
