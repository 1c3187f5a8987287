// a2 (+ a3 fused): length-masked top-k of the indexer logits.
//
// "nsa_backend.py (EngineX-Hygon sglang fork)", NSAIndexerMetadata.
// topk_transform: fast_topk_v2(logits, lengths=seqlens_expanded, topk) keeps
// at most topk positions per row (NSAMetadata limits the lengths to topk); the fused
// variant fast_topk_transform_fused returns physical slots through the page
// table instead of logical positions.
//
// Method (MI355X design): rows with n <= topk keep 0..n-1 and read no
// logits. Longer rows run a radix select on the order-preserving uint32 image
// of the fp32 logits (NaN -> lowest, -0 -> +0):
//   * pass 1 spreads every row over many blocks: 16-bit histograms of the
//     top 12 key bits per 16384-position chunk;
//   * pass 2 is one 1024-thread block per row: it sums the chunk histograms,
//     finds the bin holding the topk-th largest key, then reads the row once,
//     marking keys above that bin in an LDS bitmap of positions and gathering
//     the keys inside it; two 10-bit radix passes over those candidates give
//     the exact threshold, ties on it keep the lowest positions, and a scan of
//     the bitmap writes the result in ascending position order, so the output
//     does not depend on scheduling.
// Rows longer than the bitmap, or whose threshold bin overflows the LDS
// candidate store, take a slower multi-pass select over the row in global
// memory.
#include "common.h"

#include <type_traits>

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

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

// Exclusive prefix sum of v over a block of NT threads; *total receives the
// sum. wave_tot holds 2 * NT / 64 + 1 ints.
template <int NT = kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot,
                                                    int* total) {
  constexpr int kWaves = NT / 64;
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

// Block-wide form of the same search: thread tid owns bins NB*tid ..
// NB*tid + NB - 1 with counts c[] in registers, and `above` counts the keys
// in the bins of all higher threads (from a block scan). The one thread whose
// bins hold the krem-th largest key publishes s_sel = {bin, krem - keys
// above the bin, bin taken whole, keys in the bin}; callers ensure the total
// is at least krem and synchronise before reading s_sel.
template <int NB>
__device__ __forceinline__ void publish_threshold(const uint32_t (&c)[NB], uint32_t above,
                                                  int krem, uint32_t* s_sel) {
  // walk the bins from the top with selects only (no early exit, so the
  // counts stay in registers)
  uint32_t a = above, sel_a = 0, sel_c = 0;
  int sel_i = -1;
#pragma unroll
  for (int i = NB - 1; i >= 0; --i) {
    const bool hit = sel_i < 0 && a + c[i] >= (uint32_t)krem;
    sel_i = hit ? i : sel_i;
    sel_a = hit ? a : sel_a;
    sel_c = hit ? c[i] : sel_c;
    a += c[i];
  }
  if (above < (uint32_t)krem && a >= (uint32_t)krem) {
    s_sel[0] = NB * threadIdx.x + sel_i;
    s_sel[1] = krem - sel_a;
    s_sel[2] = (sel_a + sel_c == (uint32_t)krem) ? 1u : 0u;
    s_sel[3] = sel_c;
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
constexpr int kCap = 12288;         // fast path: threshold-bin candidates in LDS
constexpr int kMapBits = 262144;    // fast path: rows of at most this many positions
constexpr int kMapWords = kMapBits / 32;
constexpr int kTieBins = 512;       // position radix for exact ties: 2 x 9 bits
constexpr int kBatch = 4;           // float4 per thread per batch of the row pass

static_assert(kMapBits == kTieBins * kTieBins, "tie radix spans the bitmap");

// OR of w over the 8 lanes of the lane's aligned group of 8, in registers:
// DPP quad_perm [1,0,3,2] and [2,3,0,1] combine each quad, row_half_mirror
// (lane i of a half row reads lane 7 - i) then joins the group's two quads.
__device__ __forceinline__ uint32_t or_lanes8(uint32_t w) {
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0xB1, 0xF, 0xF, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x4E, 0xF, 0xF, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x141, 0xF, 0xF, false);
  return w;
}

// Raw values of positions pos..pos+3 with no branch around the loads (a load
// under a branch makes the compiler wait for every load in flight). VEC: one
// 16-byte load at min(pos, vlast), where vlast is a multiple of 4 with
// vlast + 4 <= n; otherwise four loads clamped to n - 1. Values of positions
// past the caller's bound are stale and the caller masks them.
template <bool VEC>
__device__ __forceinline__ void load4(const float* row, int pos, int vlast,
                                      int n, float* v) {
  if constexpr (VEC) {
    const float4 x = *reinterpret_cast<const float4*>(row + min(pos, vlast));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = row[min(pos + e, n - 1)];
  }
}

// Pass 1: per-(row, chunk) histogram of the top 12 key bits, over all CUs.
// Each wave counts into its own LDS sub-histogram; the block writes 4096
// 16-bit counts (a chunk holds at most 16384 positions).
template <bool VEC>
__global__ void __launch_bounds__(kHistThreads)
topk_hist_kernel(const float* __restrict__ logits, int64_t logits_stride,
                 const int32_t* __restrict__ lengths, int topk,
                 int max_seqlen_k, int chunks, uint16_t* __restrict__ ws) {
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
  const float* row = logits + t * logits_stride;
  uint32_t* h = sub[wave];
  // [start, vend) is read 4 positions at a time; with VEC the 0..3 positions
  // of [vend, end) are read one per thread afterwards
  const int vend = VEC ? min(end, n & ~3) : end;
  constexpr int kPer = kChunk / kHistThreads / 4;   // 16 loads per thread
  float v[kPer][4];
  if (vend > start) {
    // every load of the thread is issued before any value is counted; load k
    // of the block covers 1024 consecutive positions
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      load4<VEC>(row, start + k * (kHistThreads * 4) + threadIdx.x * 4,
                 vend - 4, n, v[k]);
  }
  __syncthreads();   // sub-histograms cleared
  if (vend > start) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int pos = start + k * (kHistThreads * 4) + threadIdx.x * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pos + e < vend) atomicAdd(&h[order_key(v[k][e]) >> 20], 1u);
    }
  }
  if (VEC) {
    const int t0 = max(start, vend);
    if ((int)threadIdx.x < end - t0)
      atomicAdd(&h[order_key(row[t0 + threadIdx.x]) >> 20], 1u);
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

// The exact selection once the keys of a row are classified against the
// threshold bin `bin` (the bin holding the topk-th largest key, krem of its
// keys still to keep; `exact`: the whole bin is kept): the LDS `bitmap` holds
// the positions of the keys above the bin, cand_pos[0, nc) those of the keys
// inside it, in any order. Two 10-bit radix passes over the candidates' keys
// find the exact threshold, ties on it keep the lowest positions (a radix
// select on position), the kept candidates are marked too, and a block-wide
// scan of the bitmap writes the kept positions in ascending order (through
// the page-table row trow when given). Every thread of the block calls it.
template <int kCP>
__device__ __forceinline__ void finish_select(
    const float* row, int n, int topk, uint32_t bin, int krem, bool exact, int nc,
    const int32_t* trow, const int32_t* lengths, uint32_t* hist, uint32_t* bitmap,
    uint32_t* cand_key, int32_t* cand_pos, int* scan_buf, uint32_t* s_sel,
    int32_t* orow) {
  const int tid = threadIdx.x;
  const int nw = (n + 31) >> 5;
  // keys of the candidates, read back from the row (recently read, so
  // mostly cache hits)
  for (int i = tid; i < nc; i += kThreads) cand_key[i] = order_key(row[cand_pos[i]]);
  // the row's page-table entries for the output, loaded now (branch-free:
  // without a table the loads read lengths[0]) and put in LDS once the
  // candidates are no longer needed
  constexpr int kTabPer = kMapBits / NSA_PAGE_SIZE / kThreads;
  int32_t tab[kTabPer];
  {
    const int32_t* tsrc = trow ? trow : lengths;
    const int lim = trow ? ((n + NSA_PAGE_SIZE - 1) >> 6) - 1 : 0;
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) tab[k] = tsrc[min(tid + k * kThreads, lim)];
  }

  // ---- exact threshold among the candidates (bits 19..10, then 9..0)
  uint32_t prefix = bin << 20, pmask = 0xFFF00000u;
  for (int pass = 0; pass < 2 && !exact; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    hist[tid] = 0;   // 1024 bins
    __syncthreads();
    for (int i = tid; i < nc; i += kThreads) {
      const uint32_t k = cand_key[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1u);
    }
    __syncthreads();
    {
      const uint32_t c1[1] = {hist[tid]};
      int tot1;
      const int ex1 = block_exclusive_scan((int)c1[0], scan_buf, &tot1);
      publish_threshold<1>(c1, (uint32_t)(tot1 - ex1) - c1[0], krem, s_sel);
    }
    __syncthreads();
    prefix |= s_sel[0] << shift;
    pmask |= 1023u << shift;
    krem = (int)s_sel[1];
    exact = s_sel[2] != 0;
    __syncthreads();
  }
  // ---- equal full keys at the threshold: keep the krem lowest positions,
  // a radix select on tk = kMapBits - 1 - position (unique, so exact)
  uint32_t tprefix = 0, tmask = 0;
  for (int pass = 0; pass < 2 && !exact; ++pass) {
    const int shift = pass == 0 ? 9 : 0;
    if (tid < kTieBins) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nc; i += kThreads) {
      const uint32_t tk = (uint32_t)(kMapBits - 1 - cand_pos[i]);
      if (cand_key[i] == prefix && (tk & tmask) == tprefix)
        atomicAdd(&hist[(tk >> shift) & (kTieBins - 1)], 1u);
    }
    __syncthreads();
    {
      const uint32_t c1[1] = {tid < kTieBins ? hist[tid] : 0u};
      int tot1;
      const int ex1 = block_exclusive_scan((int)c1[0], scan_buf, &tot1);
      publish_threshold<1>(c1, (uint32_t)(tot1 - ex1) - c1[0], krem, s_sel);
    }
    __syncthreads();
    tprefix |= s_sel[0] << shift;
    tmask |= (uint32_t)(kTieBins - 1) << shift;
    krem = (int)s_sel[1];
    __syncthreads();
  }
  for (int i = tid; i < nc; i += kThreads) {
    const uint32_t mk = cand_key[i] & pmask;
    const int pos = cand_pos[i];
    const bool keep = mk > prefix ||
        (mk == prefix && (exact || (uint32_t)(kMapBits - 1 - pos) >= tprefix));
    if (keep) atomicOr(&bitmap[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  int32_t* ptab = reinterpret_cast<int32_t*>(cand_key);   // >= 4096 entries
  static_assert(kCP >= kTabPer * kThreads, "page table fits the candidate store");
  if (trow) {
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) ptab[tid + k * kThreads] = tab[k];
  }

  // ---- kept positions in ascending order: each thread owns a run of words
  // (the scan's barriers also publish the page table)
  const int per = (nw + kThreads - 1) / kThreads;
  const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
  int kept;
  int o = block_exclusive_scan(cnt, scan_buf, &kept);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      const int i = w * 32 + b;
      if (o < topk) orow[o] = trow ? (ptab[i >> 6] << 6) + (i & 63) : i;
      ++o;
    }
  }
}

// Pass 2: one block per row. Sums the row's chunk histograms and finds the
// threshold bin; one pass over the row then marks every key above that bin in
// an LDS bitmap of positions and gathers the keys inside it as candidates
// (unordered); the exact threshold comes from two more 10-bit radix passes
// over the candidates, and ties on the threshold key keep the lowest
// positions (a radix select on position). The chosen candidates are marked
// too, and a block-wide scan of the bitmap writes the kept positions in
// ascending order (through the page table when given).
// GIVEN: the row histograms come from the indexer (key_hist, [T][4096]
// uint32) instead of pass 1; each row of key_hist is cleared once read, and a
// row whose counts do not add up to its length takes the multi-pass select.
// SMALL: batches of at least kSmallMinRows rows of at most kSmallMapBits
// positions (max_seqlen_k bounds them), such as chunked extend. An 8 KB
// bitmap, a 4096-entry candidate store and a 2048-bin radix histogram take
// 48 KB of LDS instead of 144, and the kernel keeps to 64 VGPRs, so two
// blocks share a CU and their row passes and barriers overlap. With fewer
// rows than CUs there is nothing to overlap and the smaller register budget
// only costs time, hence the row minimum.
constexpr int kSmallMapBits = 65536;
constexpr int kSmallMinRows = 512;
template <bool VEC, bool GIVEN, bool SMALL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SMALL ? 8 : 1)))
topk_select_kernel(const float* __restrict__ logits, int64_t logits_stride,
                   const int32_t* __restrict__ lengths, int topk,
                   int max_seqlen_k, int chunks,
                   const uint16_t* __restrict__ ws,
                   uint32_t* __restrict__ key_hist,
                   const int32_t* __restrict__ table, int64_t table_stride,
                   int64_t table_rows, const int32_t* __restrict__ t2r,
                   int32_t* __restrict__ out, int64_t out_stride) {
  constexpr int kMB = SMALL ? kSmallMapBits : kMapBits;   // bitmap bits
  constexpr int kMW = kMB / 32;
  constexpr int kCP = SMALL ? 4096 : kCap;                 // candidate store
  static_assert(kCP >= kMapBits / NSA_PAGE_SIZE, "page table fits the candidate store");
  __shared__ uint32_t hist[SMALL ? 2048 : kHistBins];     // radix passes use <= 2048 bins
  __shared__ uint32_t bitmap[kMW];
  __shared__ uint32_t cand_key[kCP];
  __shared__ int32_t cand_pos[kCP];
  __shared__ int scan_buf[2 * kWaves + 1];
  __shared__ uint32_t s_sel[4];
  __shared__ int s_ncand;

  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  int n = lengths[t];
  n = n < 0 ? 0 : (n > max_seqlen_k ? max_seqlen_k : n);
  int32_t* orow = out + t * out_stride;
  static_assert(kThreads * 4 == kHistBins && kHistBins == kKeyBins, "one thread per 4 bins");
  uint4* hrow4 = GIVEN ? reinterpret_cast<uint4*>(key_hist + t * kHistBins) : nullptr;
  const int32_t req = table ? t2r[t] : 0;
  if (table && (req < 0 || req >= table_rows)) {
    // a row of no known request has no slots: all -1
    if (tid == 0) flag_device_error(NSA_DEVERR_REQUEST);
    for (int j = tid; j < topk; j += kThreads) orow[j] = -1;
    if (GIVEN) hrow4[tid] = make_uint4(0, 0, 0, 0);
    return;
  }
  const int32_t* trow = table ? table + (int64_t)req * table_stride : nullptr;
  auto map = [&](int i) -> int32_t {
    return trow ? (trow[i >> 6] << 6) + (i & 63) : i;
  };
  if (n <= topk) {
    for (int j = tid; j < topk; j += kThreads) orow[j] = j < n ? map(j) : -1;
    if (GIVEN) hrow4[tid] = make_uint4(0, 0, 0, 0);
    return;
  }
  const float* row = logits + t * logits_stride;

  // the first batch of the row pass does not depend on the threshold: its
  // loads are issued now and land while the histogram is read and scanned
  const int vend = VEC ? (n & ~3) : n;
  constexpr int kSpan = kThreads * 4;           // positions per load step
  // the short-row instantiation takes half batches: with 64 registers a
  // full batch pair spills, and each spill store waits for every load in
  // flight (extend: 343 against 459 us)
  constexpr int kB = SMALL ? kBatch / 2 : kBatch;
  constexpr int kPerBatch = kSpan * kB;
  // last vector start; n >= 1 here, and a vector row (16-byte aligned,
  // stride a multiple of 4) always holds positions 0..3, so 0 is a safe
  // clamp for rows shorter than one vector
  const int vlast = vend >= 4 ? vend - 4 : 0;
  float va[kB][4], vb[kB][4];
  auto fetch = [&](float (&v)[kB][4], int b0) {
#pragma unroll
    for (int j = 0; j < kB; ++j) load4<VEC>(row, b0 + j * kSpan + tid * 4, vlast, n, v[j]);
  };
  fetch(va, 0);   // no branch: a load under one would be waited for at once

  // ---- row histogram of the top 12 key bits and its threshold bin: each
  // thread owns 4 bins in registers (given, then cleared; or summed over the
  // chunks of pass 1 with 8-byte loads); one block scan gives the total and,
  // for every thread, the keys in higher bins
  uint32_t hc[4] = {0, 0, 0, 0};
  {
    const int b4 = tid * 4;
    if constexpr (GIVEN) {
      const uint4 v = hrow4[tid];
      hrow4[tid] = make_uint4(0, 0, 0, 0);
      hc[0] = v.x; hc[1] = v.y; hc[2] = v.z; hc[3] = v.w;
    } else {
      const int nch = (n + kChunk - 1) / kChunk;
      const uint16_t* hrow = ws + t * chunks * kHistBins;
      for (int c = 0; c < nch; ++c) {
        const uint2 v = *reinterpret_cast<const uint2*>(hrow + c * kHistBins + b4);
        hc[0] += v.x & 0xFFFFu; hc[1] += v.x >> 16; hc[2] += v.y & 0xFFFFu; hc[3] += v.y >> 16;
      }
    }
  }
  const uint32_t hs = hc[0] + hc[1] + hc[2] + hc[3];
  int tot;
  const int hex = block_exclusive_scan((int)hs, scan_buf, &tot);
  if (tot != n) {   // not the histogram of these logits
    select_multipass(row, n, VEC, topk, orow, map, hist, scan_buf, s_sel);
    return;
  }
  const int nw = (n + 31) >> 5;
  if (n <= kMB)
    for (int w = tid; w < nw; w += kThreads) bitmap[w] = 0u;
  if (tid == 0) s_ncand = 0;
  publish_threshold<4>(hc, (uint32_t)(tot - hex) - hs, topk, s_sel);
  __syncthreads();
  const uint32_t bin = s_sel[0];
  int krem = (int)s_sel[1];
  bool exact = s_sel[2] != 0;
  const uint32_t cnt_b = s_sel[3];
  __syncthreads();
  if (cnt_b > (uint32_t)kCP || n > kMB) {
    select_multipass(row, n, VEC, topk, orow, map, hist, scan_buf, s_sel);
    return;
  }

  // ---- one pass over the row, batches of kB loads per thread, the next
  // batch in flight while one is classified (two register batches used in
  // turn). Loads past the row are clamped onto its last vector, so the
  // prefetch needs no branch.
  //
  // The order key is monotone in the value (-0 == +0, NaN lowest), so for a
  // bin strictly inside the finite range (8 <= bin <= 4087: bins 0..7 hold
  // NaN and -inf, bins >= 4088 +inf and no finite value) "key >= K" is
  // "x >= key_floor(K)", the smallest float with that key; the pass then
  // compares floats and computes the key of candidates only.
  auto key_floor = [](uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  };
  const bool fcmp = bin >= 8 && bin <= 4087;
  const float lo_bin = key_floor(bin << 20), lo_above = key_floor((bin + 1) << 20);
  auto row_pass = [&](auto fc) {
    constexpr bool FC = decltype(fc)::value;
    auto above = [&](float x) {
      if constexpr (FC) return x >= lo_above;
      else return (order_key(x) >> 20) > bin;
    };
    auto in_bin = [&](float x) {
      if constexpr (FC) return x >= lo_bin && !(x >= lo_above);
      else return (order_key(x) >> 20) == bin;
    };
    // Classifies one batch: the bits of keys above the bin go straight into
    // the bitmap (the 8 lanes sharing a 32-bit word OR their nibbles in
    // registers and one of them stores it, so no LDS atomics), and the
    // positions of keys in the bin are appended to the candidate store (a
    // loop over the set bits of a 16-bit mask; the keys are read back after
    // the pass).
    auto classify = [&](const float (&v)[kB][4], int b0) {
      uint32_t cm = 0;   // bit 4j + e: candidate
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int pos = b0 + j * kSpan + tid * 4;
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool in = pos + e < vend;
          m |= (in && above(v[j][e])) ? (1u << e) : 0u;
          cm |= (in && in_bin(v[j][e])) ? (1u << (4 * j + e)) : 0u;
        }
        const uint32_t w = or_lanes8(m << ((tid & 7) * 4));
        const int word = pos >> 5;
        if ((tid & 7) == 0 && word < kMW) bitmap[word] = w;
      }
      // a lane with candidates reserves its slots with one LDS atomic (the
      // order of the candidates does not matter to the exact selection)
      int q = 0;
      if (cm) q = atomicAdd(&s_ncand, __popc(cm));
      while (cm) {
        const int b = __ffs(cm) - 1;
        cm &= cm - 1;
        if (q < kCP) cand_pos[q] = b0 + (b >> 2) * kSpan + tid * 4 + (b & 3);
        ++q;
      }
    };
    if (vend <= 0) return;   // VEC rows of 1..3 positions are all tail
    for (int b0 = 0; b0 < vend; b0 += 2 * kPerBatch) {
      fetch(vb, b0 + kPerBatch);
      classify(va, b0);
      fetch(va, b0 + 2 * kPerBatch);
      classify(vb, b0 + kPerBatch);     // positions past vend are masked
    }
  };
  if (fcmp) row_pass(std::true_type{});
  else row_pass(std::false_type{});
  __syncthreads();   // every bitmap word of the pass is stored
  if (VEC && tid < n - vend) {   // the 0..3 positions past the last vector
    const int pos = vend + tid;
    const uint32_t k = order_key(row[pos]);
    if ((k >> 20) > bin) {
      atomicOr(&bitmap[pos >> 5], 1u << (pos & 31));
    } else if ((k >> 20) == bin) {
      const int q = atomicAdd(&s_ncand, 1);
      if (q < kCP) cand_pos[q] = pos;
    }
  }
  __syncthreads();
  finish_select<kCP>(row, n, topk, bin, krem, exact, min(s_ncand, kCP), trow,
                     lengths, hist, bitmap, cand_key, cand_pos, scan_buf, s_sel,
                     orow);
}


// ---- split select (key_hist given, a workspace, rows longer than one
// segment). One block per row reads at most ~20-25 GB/s, so a long row's pass
// over its logits bounds the one-kernel select; here that pass is spread over
// blocks of kSeg positions (topk_mark_kernel), which classify their keys
// against the row's threshold bin into two bitmaps in the workspace, and one
// block per row then finishes the exact selection from those bitmaps
// (topk_finish_kernel), as the one-kernel select does after its pass.
// Workspace row t (ws_row uint32 words, 16-byte aligned):
//   [0, 4)                    {take the multi-pass select, bin, krem, exact},
//                             written by the row's first segment block
//   [kSplitParams, +mw)       bit p: the key of position p lies above the bin
//   [kSplitParams + mw, +mw)  bit p: the key of position p lies in the bin
// with mw = ceil(max_seqlen_k / 32) rounded up to a multiple of 4. Words of
// positions at or past the row's length are never written; nothing has to be
// zero on entry.
constexpr int kSeg = 16384;                     // positions per mark block
constexpr int kSegThreads = 256;
constexpr int kSegVec = kSeg / (kSegThreads * 4);   // float4 per thread
constexpr int kSplitParams = 16;

__host__ __device__ constexpr int split_map_words(int max_seqlen_k) {
  return ((max_seqlen_k + 31) / 32 + 3) & ~3;
}

template <bool VEC>
__global__ void __launch_bounds__(kSegThreads)
topk_mark_kernel(const float* __restrict__ logits, int64_t logits_stride,
                 const int32_t* __restrict__ lengths, int64_t rows, int topk,
                 int max_seqlen_k, int segs,
                 const uint32_t* __restrict__ key_hist,
                 uint32_t* __restrict__ ws, int64_t ws_row, int mw) {
  __shared__ int scan_buf[2 * (kSegThreads / 64) + 1];
  __shared__ uint32_t s_sel[4];
  // work groups are dealt to the 8 XCDs in turn (block b to XCD b % 8): the
  // segments of row t all run on XCD t % 8, so each XCD's L2 fetches a row's
  // histogram once for all of its segments (the grid covers T rounded up to
  // a multiple of 8 rows)
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int64_t t = 8 * (int64_t)(j / segs) + xcd;
  const int seg0 = (j % segs) * kSeg;
  const int tid = threadIdx.x;
  if (t >= rows) return;
  int n = lengths[t];
  n = n < 0 ? 0 : (n > max_seqlen_k ? max_seqlen_k : n);
  if (n <= topk || seg0 >= n) return;   // the finish kernel keeps 0..n-1
  const float* row = logits + t * logits_stride;

  // the whole segment is loaded before the threshold is known (clamped
  // branch-free loads, as in the one-kernel select; VEC: positions
  // [vend, n) are fixed up below)
  const int vend = VEC ? (n & ~3) : n;
  const int vlast = vend >= 4 ? vend - 4 : 0;
  float v[kSegVec][4];
#pragma unroll
  for (int k = 0; k < kSegVec; ++k)
    load4<VEC>(row, seg0 + k * (kSegThreads * 4) + tid * 4, vlast, n, v[k]);

  // threshold bin from the row histogram: thread tid owns bins 16 tid ..
  // 16 tid + 15
  uint32_t c[16];
  {
    const uint4* h4 = reinterpret_cast<const uint4*>(key_hist + t * kKeyBins) + tid * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = h4[i];
      c[4 * i] = x.x; c[4 * i + 1] = x.y; c[4 * i + 2] = x.z; c[4 * i + 3] = x.w;
    }
  }
  uint32_t hs = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) hs += c[i];
  int tot;
  const int hex = block_exclusive_scan<kSegThreads>((int)hs, scan_buf, &tot);
  uint32_t* prow = ws + t * ws_row;
  if (tot != n) {   // not the histogram of these logits: multi-pass select
    if (seg0 == 0 && tid == 0)
      *reinterpret_cast<uint4*>(prow) = make_uint4(1u, 0u, 0u, 0u);
    return;
  }
  publish_threshold<16>(c, (uint32_t)(tot - hex) - hs, topk, s_sel);
  __syncthreads();
  const uint32_t bin = s_sel[0];
  const bool multipass = s_sel[3] > (uint32_t)kCap || n > kMapBits;
  if (seg0 == 0 && tid == 0)
    *reinterpret_cast<uint4*>(prow) =
        make_uint4(multipass ? 1u : 0u, bin, s_sel[1], s_sel[2]);
  if (multipass) return;

  if (VEC && vend < n) {   // the 1..3 positions past the last whole vector
#pragma unroll
    for (int k = 0; k < kSegVec; ++k) {
      const int pos = seg0 + k * (kSegThreads * 4) + tid * 4;
      if (pos == vend) {
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (vend + e < n) v[k][e] = row[vend + e];
      }
    }
  }
  // the 8 lanes sharing a 32-bit word OR their nibbles in registers and one
  // of them stores the word of each bitmap
  uint32_t* amap = prow + kSplitParams;
  uint32_t* bmap = amap + mw;
  const int nw = (n + 31) >> 5;
#pragma unroll
  for (int k = 0; k < kSegVec; ++k) {
    const int pos = seg0 + k * (kSegThreads * 4) + tid * 4;
    uint32_t ma = 0, mb = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = pos + e < n;
      const uint32_t kb = order_key(v[k][e]) >> 20;
      ma |= (in && kb > bin) ? (1u << e) : 0u;
      mb |= (in && kb == bin) ? (1u << e) : 0u;
    }
    const uint32_t wa = or_lanes8(ma << ((tid & 7) * 4));
    const uint32_t wb = or_lanes8(mb << ((tid & 7) * 4));
    const int word = pos >> 5;
    if ((tid & 7) == 0 && word < nw) {
      amap[word] = wa;
      bmap[word] = wb;
    }
  }
}

// One 1024-thread block per row after topk_mark_kernel: clears the row of
// key_hist, takes the threshold bin from the workspace, loads the above-bin
// bitmap into LDS and lists the in-bin positions (ascending) as candidates,
// then runs the same exact selection and ordered write as the one-kernel
// select. Rows the mark kernel left to the multi-pass select, and rows of
// at most topk positions, are done here as there.
template <bool VEC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
topk_finish_kernel(const float* __restrict__ logits, int64_t logits_stride,
                   const int32_t* __restrict__ lengths, int topk,
                   int max_seqlen_k, uint32_t* __restrict__ key_hist,
                   const uint32_t* __restrict__ ws, int64_t ws_row, int mw,
                   const int32_t* __restrict__ table, int64_t table_stride,
                   int64_t table_rows, const int32_t* __restrict__ t2r,
                   int32_t* __restrict__ out, int64_t out_stride) {
  __shared__ uint32_t hist[2048];   // multi-pass digits (<= 2048 bins)
  __shared__ uint32_t bitmap[kMapWords];
  __shared__ uint32_t cand_key[kCap];
  __shared__ int32_t cand_pos[kCap];
  __shared__ int scan_buf[2 * kWaves + 1];
  __shared__ uint32_t s_sel[4];

  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  // the row's threshold and both bitmaps are loaded before its length is
  // known (words past the row's end are masked once it is; rows that need
  // none of them ignore them), so these loads overlap the others
  const uint32_t* prow = ws + t * ws_row;
  const uint4 par = *reinterpret_cast<const uint4*>(prow);
  const uint4* amap4 = reinterpret_cast<const uint4*>(prow + kSplitParams);
  const uint4* bmap4 = reinterpret_cast<const uint4*>(prow + kSplitParams + mw);
  // thread tid owns words 8 tid .. 8 tid + 7 of both bitmaps (mw and the
  // row stride are multiples of 4 words, so the 16-byte loads stay in the
  // row's mw words)
  static_assert(kMapWords == 8 * kThreads, "8 bitmap words per thread");
  uint32_t a[8], b[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = 8 * tid + 4 * h;
    uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
    if (w < mw) { xa = amap4[w >> 2]; xb = bmap4[w >> 2]; }
    a[4 * h] = xa.x; a[4 * h + 1] = xa.y; a[4 * h + 2] = xa.z; a[4 * h + 3] = xa.w;
    b[4 * h] = xb.x; b[4 * h + 1] = xb.y; b[4 * h + 2] = xb.z; b[4 * h + 3] = xb.w;
  }
  int n = lengths[t];
  n = n < 0 ? 0 : (n > max_seqlen_k ? max_seqlen_k : n);
  int32_t* orow = out + t * out_stride;
  static_assert(kThreads * 4 == kKeyBins, "one uint4 of key_hist per thread");
  // every mark block of the row has read it (stream order)
  reinterpret_cast<uint4*>(key_hist + t * kKeyBins)[tid] = make_uint4(0, 0, 0, 0);
  const int32_t req = table ? t2r[t] : 0;
  if (table && (req < 0 || req >= table_rows)) {
    if (tid == 0) flag_device_error(NSA_DEVERR_REQUEST);
    for (int j = tid; j < topk; j += kThreads) orow[j] = -1;
    return;
  }
  const int32_t* trow = table ? table + (int64_t)req * table_stride : nullptr;
  auto map = [&](int i) -> int32_t {
    return trow ? (trow[i >> 6] << 6) + (i & 63) : i;
  };
  if (n <= topk) {
    for (int j = tid; j < topk; j += kThreads) orow[j] = j < n ? map(j) : -1;
    return;
  }
  const float* row = logits + t * logits_stride;
  if (par.x != 0) {
    select_multipass(row, n, VEC, topk, orow, map, hist, scan_buf, s_sel);
    return;
  }
  const uint32_t bin = par.y;
  const int krem = (int)par.z;
  const bool exact = par.w != 0;
  // words at or past nw (<= kMapWords: longer rows take the multi-pass
  // select) were never written and count as zero
  const int nw = (n + 31) >> 5;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (8 * tid + i >= nw) { a[i] = 0u; b[i] = 0u; }
    cnt += __popc(b[i]);
  }
  if (8 * tid < nw) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      reinterpret_cast<uint4*>(bitmap)[2 * tid + h] =
          make_uint4(a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]);
  }
  int ncand;
  int q = block_exclusive_scan(cnt, scan_buf, &ncand);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t bits = b[i];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (q < kCap) cand_pos[q] = (8 * tid + i) * 32 + bit;
      ++q;
    }
  }
  __syncthreads();
  finish_select<kCap>(row, n, topk, bin, krem, exact, min(ncand, kCap), trow,
                      lengths, hist, bitmap, cand_key, cand_pos, scan_buf, s_sel,
                      orow);
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
                                  int64_t table_stride, int64_t table_rows,
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
    NSA_REQUIRE(table_rows >= 0, NSA_ERR_INVALID_ARG, "%s: negative table_rows", fn);
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
    auto hist = vec ? topk_hist_kernel<true> : topk_hist_kernel<false>;
    hipLaunchKernelGGL(hist, dim3((unsigned)hb), dim3(kHistThreads), 0, s,
                       logits, logits_stride, lengths, topk, max_seqlen_k,
                       chunks, ws);
    int st = nsa::check_launch(fn);
    if (st != NSA_OK) return st;
  }
  const bool small = max_seqlen_k <= kSmallMapBits && T >= kSmallMinRows;
  auto sel = vec ? (small ? topk_select_kernel<true, false, true> : topk_select_kernel<true, false, false>)
                 : (small ? topk_select_kernel<false, false, true> : topk_select_kernel<false, false, false>);
  hipLaunchKernelGGL(sel, dim3(T), dim3(kThreads), 0, s, logits, logits_stride,
                     lengths, topk, max_seqlen_k, chunks, ws, nullptr, table,
                     table_stride, table_rows, token_to_req, out, out_stride);
  return nsa::check_launch(fn);
}

// Rows split over mark blocks: only for rows longer than a segment that fit
// the bitmaps, and for at most kSplitMaxRows rows. The one-kernel select runs
// one block per row, so with at most half as many rows as the 256 CUs of an
// MI355X most CUs idle and a long row's pass over its logits bounds it; with
// more rows it already uses every CU, and the finish launch's fixed cost
// (about 60% of the one-kernel time at 256 rows) makes the split slower.
constexpr int kSplitMaxRows = 128;
static bool split_select(int T, int max_seqlen_k, int topk) {
  return T <= kSplitMaxRows && max_seqlen_k > topk && max_seqlen_k > kSeg &&
         max_seqlen_k <= kMapBits;
}

extern "C" int nsa_topk_hist_workspace_size(int T, int max_seqlen_k, int topk,
                                            size_t* bytes) {
  NSA_REQUIRE(bytes != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_topk_hist_workspace_size: null output");
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0 && topk >= 0, NSA_ERR_INVALID_ARG,
              "nsa_topk_hist_workspace_size: negative size");
  *bytes = T > 0 && split_select(T, max_seqlen_k, topk)
               ? (size_t)T * (kSplitParams + 2 * (size_t)split_map_words(max_seqlen_k)) *
                     sizeof(uint32_t)
               : 0;
  return nsa::ok();
}

extern "C" int nsa_topk_transform_hist(const float* logits, int64_t logits_stride,
                                       const int32_t* lengths, int T, int topk,
                                       int max_seqlen_k, const int32_t* table,
                                       int64_t table_stride, int64_t table_rows,
                                       const int32_t* token_to_req, int page_size,
                                       uint32_t* key_hist, int32_t* out,
                                       int64_t out_stride, void* workspace,
                                       size_t ws_bytes, void* stream) {
  const char* fn = "nsa_topk_transform_hist";
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0, NSA_ERR_INVALID_ARG,
              "%s: negative size", fn);
  NSA_REQUIRE(topk > 0, NSA_ERR_INVALID_ARG, "%s: topk must be positive", fn);
  NSA_REQUIRE(page_size == NSA_PAGE_SIZE, NSA_ERR_UNSUPPORTED,
              "%s: page_size %d (only 64 is supported)", fn, page_size);
  if (T == 0) return nsa::ok();
  NSA_REQUIRE(lengths && out && key_hist, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(nsa::aligned(key_hist, 16), NSA_ERR_INVALID_ARG,
              "%s: key_hist must be 16-byte aligned", fn);
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
    NSA_REQUIRE(table_rows >= 0, NSA_ERR_INVALID_ARG, "%s: negative table_rows", fn);
  }
  size_t need = 0;
  nsa_topk_hist_workspace_size(T, max_seqlen_k, topk, &need);
  if (workspace != nullptr && need > 0) {
    NSA_REQUIRE(ws_bytes >= need, NSA_ERR_WORKSPACE,
                "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    NSA_REQUIRE(nsa::aligned(workspace, 16), NSA_ERR_INVALID_ARG,
                "%s: workspace must be 16-byte aligned", fn);
  }
  const bool vec = logits && nsa::aligned(logits, 16) && logits_stride % 4 == 0;
  hipStream_t s = (hipStream_t)stream;
  if (workspace != nullptr && need > 0) {
    const int segs = (max_seqlen_k + kSeg - 1) / kSeg;
    const int mw = split_map_words(max_seqlen_k);
    const int64_t ws_row = kSplitParams + 2 * (int64_t)mw;
    const int64_t mark_blocks = ((int64_t)T + 7) / 8 * 8 * segs;
    NSA_REQUIRE(mark_blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
    uint32_t* w = static_cast<uint32_t*>(workspace);
    hipLaunchKernelGGL(vec ? topk_mark_kernel<true> : topk_mark_kernel<false>,
                       dim3((unsigned)mark_blocks), dim3(kSegThreads), 0, s, logits,
                       logits_stride, lengths, (int64_t)T, topk, max_seqlen_k, segs,
                       key_hist, w, ws_row, mw);
    int st = nsa::check_launch(fn);
    if (st != NSA_OK) return st;
    hipLaunchKernelGGL(vec ? topk_finish_kernel<true> : topk_finish_kernel<false>,
                       dim3(T), dim3(kThreads), 0, s, logits, logits_stride, lengths,
                       topk, max_seqlen_k, key_hist, w, ws_row, mw, table,
                       table_stride, table_rows, token_to_req, out, out_stride);
    return nsa::check_launch(fn);
  }
  const bool small = max_seqlen_k <= kSmallMapBits && T >= kSmallMinRows;
  auto sel = vec ? (small ? topk_select_kernel<true, true, true> : topk_select_kernel<true, true, false>)
                 : (small ? topk_select_kernel<false, true, true> : topk_select_kernel<false, true, false>);
  hipLaunchKernelGGL(sel, dim3(T), dim3(kThreads), 0, s,
                     logits, logits_stride, lengths, topk, max_seqlen_k, 0,
                     nullptr, key_hist, table, table_stride, table_rows,
                     token_to_req, out, out_stride);
  return nsa::check_launch(fn);
}
