// a1: indexer logits ("paged MQA logits") over the 64-token paged index-key
// cache.
//
// The pages feed the indexer the compact 64-token page table
// ("nsa_backend.py (EngineX-Hygon sglang fork)",
// NSAIndexerMetadata.get_page_table_64) and one context length per query row
// ("dsa_backend.py (sglang main)", _to_2d_context_lens). The scoring formula
// is the reading stated in nsa.h:
//   logits[t, s] = kscale[s] * sum_h w[t, h] * relu(q[t, h, :] . k[s, :]).
//
// fp8 path (Hi = 64 heads, Di = 128), MI355X design:
//   * one block of 4 waves per (row, chunk of 32 pages; 16 or 8 for a batch
//     too small to give 1024 blocks), in plain row-major
//     order with the chunk count per row padded to an odd number: work groups
//     are dealt to the 8 XCDs round-robin, so a row's chunks start on a
//     different XCD than the previous row's and rows of unequal length
//     spread evenly (an even count pins chunk c to XCD c mod 8, and the
//     XCDs holding the low chunks, which every row has, finish last);
//   * rows that share a request in fixed groups (target-verify, draft-extend
//     v2: `group` consecutive rows per request) read the same pages: their
//     blocks for one chunk are made consecutive on one XCD (work group b
//     runs on XCD b % 8), so the first fills that XCD's L2 and the others
//     hit it;
//   * wave w takes pages
//     w, w+4, ... of the chunk, so a wave always works on a whole page
//     (64 tokens = 8 KB of keys + 256 B of scales, contiguous); two page
//     buffers per wave keep the register count at 140 (three waves per
//     SIMD), which measured faster than deeper prefetch at lower occupancy;
//   * v_mfma_f32_16x16x128_f8f6f4 with A = 16 heads x 128 dims of q (held in
//     registers for the whole block) and B = 128 dims x 16 tokens of keys, so
//     the dot products over all 128 dims take one instruction and the output
//     holds 4 heads x 1 token per lane;
//   * ReLU and the head weights are applied in registers; the 64-head sum is
//     16 in-lane FMAs plus a 3-shuffle transpose-reduce that leaves token
//     lane in lane `lane`, so each page is stored as 64 consecutive floats;
//   * keys are read as whole 128-byte lines (each 16-byte load instruction
//     covers 1 KB of the page), non-temporal where each page has one reading
//     row (rows_per_request <= 1), and each page passes
//     through the wave's LDS image into the MFMA operand layout; the next
//     page is in flight while one is scored, and no load sits under a branch.
// The contraction dimension is split over lanes identically for q and for
// the keys (each lane takes bytes [16g, 16g+16) and [64+16g, 64+16g+16) of a
// 128-byte row, g = lane / 16), so the dot products do not depend on the
// hardware's order of the contraction within an instruction.
#include "common.h"

namespace {

constexpr int kPage = 64;
constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kPageBytesFp8 = kPage * kDim + kPage * 4;  // 8448
constexpr int kWaves = 4;
// pages per block of the one-row kernel: 32, or 16 / 8 when that leaves
// fewer than kMinBlocks blocks (a small batch would not fill the CUs)
constexpr int kPagesPerBlock = 32;
constexpr int64_t kMinBlocks = 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Orders one wave's LDS writes before its later LDS reads (and the reads
// before later writes) for the compiler; the hardware runs a wave's LDS
// instructions in order.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct PageKeys {
  i32x8 k[4];  // 4 tiles of 16 tokens
  float ks;    // scale of token `lane`
};

// One page as loaded by the one-row kernel: line k of the page's 8 KB of
// keys (1 KB, rows 8k .. 8k+7) spread over the wave, lane l holding bytes
// [16l, 16l+16) of it, plus the scale of token `lane`. Each load instruction
// reads whole 128-byte lines, which allows non-temporal loads (NT): where
// each page has one reader, streaming the keys past the caches reads faster
// than the MFMA-layout loads below, whose instructions cover half lines.
// Where rows of one request share their pages, plain loads keep the pages
// cached for the other rows.
struct PageLines {
  u32x4 v[8];
  float ks;
};

template <bool NT>
__device__ __forceinline__ void load_page_lines(PageLines& pl, const uint8_t* base,
                                                int lane) {
  const u32x4* kp = reinterpret_cast<const u32x4*>(base + lane * 16);
  const float* sp = reinterpret_cast<const float*>(base + kPage * kDim + 4 * lane);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    pl.v[k] = NT ? __builtin_nontemporal_load(kp + k * 64) : kp[k * 64];
  pl.ks = NT ? __builtin_nontemporal_load(sp) : *sp;
}

// Per-wave LDS image of one page of keys: 64 rows of 8 16-byte pieces, piece
// p of row r stored at slot p ^ ((r >> 1) & 7), so that both the row-major
// writes (2 rows per 16 lanes) and the MFMA-layout reads (16 rows, one piece)
// of one ds_*_b128 cover all 64 banks once.
__device__ __forceinline__ int key_lds(int r, int piece) {
  return r * 8 + (piece ^ ((r >> 1) & 7));
}

// Keys of one page for this lane plus the scale of token `lane`. Always
// issued (an absent page reads page 0 and its results are masked): a load
// under a branch would make the compiler wait for every load in flight.
__device__ __forceinline__ void load_page(PageKeys& pk, const uint8_t* base,
                                          int c, int g, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint8_t* row = base + (j * 16 + c) * kDim;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + g * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(row + 64 + g * 16);
    pk.k[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  pk.ks = *reinterpret_cast<const float*>(base + kPage * kDim + 4 * lane);
}

// ReLU as one integer max on the float's bits: a negative value (sign bit
// set) is a negative int and becomes +0, a positive one is unchanged.
// fmaxf costs two instructions (the compiler first quiets a possible NaN).
// The dot products are finite for finite fp8 codes; a NaN code gives NaN
// or 0 here, and NaN logits are outside the contract.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// HIST: also count the top 12 bits of every written logit's order key into
// key_hist[t][0..4095] (an LDS histogram per block, then one global atomic
// per nonzero bin), so the top-k needs no pass of its own to histogram.
template <bool HIST, bool NT>
__global__ void __launch_bounds__(256)
indexer_fp8_kernel(const uint8_t* __restrict__ q, const float* __restrict__ w,
                   const uint8_t* __restrict__ cache, int64_t num_pages,
                   const int32_t* __restrict__ rpt, int64_t rpt_stride,
                   int64_t num_reqs, const int32_t* __restrict__ t2r,
                   const int32_t* __restrict__ seqlens, int max_seqlen_k,
                   float* __restrict__ logits, int64_t logits_stride,
                   int chunks_per_row, int pages_per_block, int group,
                   int64_t npairs, uint32_t* __restrict__ key_hist) {
  __shared__ uint32_t lhist[HIST ? kKeyBins : 1];
  __shared__ u32x4 kst[kWaves][kPage * 8];   // per-wave page image, 8 KB each
  // block -> (row group, chunk) pair qi and row j of the group: the blocks
  // of one pair are `group` consecutive slots of one XCD's sequence (for
  // group 1 this is the plain order, qi = blockIdx.x)
  const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int64_t qi = (slot / group) * 8 + xcd;
  if (qi >= npairs) return;
  const int64_t t = (qi / chunks_per_row) * group + slot % group;
  const int chunk = (int)(qi % chunks_per_row);
  int L = seqlens[t];
  L = L < 0 ? 0 : (L > max_seqlen_k ? max_seqlen_k : L);
  const int npages = (L + kPage - 1) / kPage;
  const int p_begin = chunk * pages_per_block;
  if (p_begin >= npages) return;
  const int p_end = min(p_begin + pages_per_block, npages);
  // a row of no known request stays unwritten (an empty row)
  const int32_t req = t2r[t];
  if (req < 0 || req >= num_reqs) {
    if (chunk == 0 && threadIdx.x == 0) flag_device_error(NSA_DEVERR_REQUEST);
    return;
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;

  // A operands: q rows of heads ht*16 + c, the lane's two 16-byte pieces
  const uint8_t* qrow = q + t * (kHeads * kDim);
  i32x8 qa[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const uint8_t* hr = qrow + (ht * 16 + c) * kDim;
    const uint4 lo = *reinterpret_cast<const uint4*>(hr + g * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(hr + 64 + g * 16);
    qa[ht] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // weights of the heads this lane's accumulators hold: ht*16 + 4g + r
  float wr[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const float4 v = *reinterpret_cast<const float4*>(w + t * kHeads + ht * 16 + 4 * g);
    wr[ht][0] = v.x; wr[ht][1] = v.y; wr[ht][2] = v.z; wr[ht][3] = v.w;
  }

  const int32_t* prow = rpt + (int64_t)req * rpt_stride;
  float* lrow = logits + t * logits_stride;

  if constexpr (HIST) {
    uint4* z = reinterpret_cast<uint4*>(lhist);
    for (int i = threadIdx.x; i < kKeyBins / 4; i += 256) z[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // this wave's pages: p_begin + wave + 4 i, i < np_w (at most 8); lane i
  // holds the id of the i-th one, so no key load waits on an id load
  const int first = p_begin + wave;
  const int np_w = first < p_end ? (p_end - first + kWaves - 1) / kWaves : 0;
  const int id_lane = lane < np_w ? prow[first + kWaves * lane] : -1;
  if (lane < np_w && (id_lane < 0 || id_lane >= num_pages)) flag_device_error(NSA_DEVERR_PAGE_ID);

  auto page_id = [&](int i) -> int {   // -1: absent or invalid
    const int id = __builtin_amdgcn_readlane(id_lane, i);
    return (id >= 0 && id < num_pages) ? id : -1;
  };
  auto fetch = [&](PageLines& pl, int i) {
    const int id = page_id(i);
    load_page_lines<NT>(pl, cache + (int64_t)(id >= 0 ? id : 0) * kPageBytesFp8, lane);
  };
  u32x4* kl = kst[wave];
  auto score = [&](const PageLines& pl, int i) {
    // through the wave's LDS image into the MFMA layout: tile j, lane (c, g)
    // takes bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row 16j + c. The
    // wave's LDS instructions run in order, so the next page's writes cannot
    // overtake these reads.
#pragma unroll
    for (int k = 0; k < 8; ++k) kl[key_lds(8 * k + (lane >> 3), lane & 7)] = pl.v[k];
    wave_sync();
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 lo = kl[key_lds(16 * j + c, g)];
      const u32x4 hi = kl[key_lds(16 * j + c, 4 + g)];
      const i32x8 kb = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      float s = 0.0f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const f32x4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qa[ht], kb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s = fmaf(wr[ht][r], relu(acc[r]), s);
      }
      v[j] = s;
    }
    // transpose-reduce over the 4 lane groups: group g keeps tile g
    const bool b0 = g & 1, b1 = (g >> 1) & 1;
    const float u0 = (b0 ? v[1] : v[0]) + __shfl_xor(b0 ? v[0] : v[1], 16);
    const float u1 = (b0 ? v[3] : v[2]) + __shfl_xor(b0 ? v[2] : v[3], 16);
    const float tot = (b1 ? u1 : u0) + __shfl_xor(b1 ? u0 : u1, 32);
    const float result = page_id(i) >= 0 ? tot * pl.ks : -INFINITY;
    const int s = (first + kWaves * i) * kPage + lane;   // position of token `lane`
    if (i < np_w && s < L) {
      lrow[s] = result;
      if constexpr (HIST) atomicAdd(&lhist[order_key(result) >> 20], 1u);
    }
    wave_sync();
  };

  // two page buffers: the keys of page i+1 are in flight while page i is
  // scored; a fetch past the wave's pages reads page 0 and is not stored
  if (np_w > 0) {
    PageLines b0, b1;
    fetch(b0, 0);
    for (int i = 0; i < np_w; i += 2) {
      fetch(b1, i + 1);
      score(b0, i);
      fetch(b0, i + 2);
      score(b1, i + 1);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* dst = key_hist + t * kKeyBins;
    const uint4* h4 = reinterpret_cast<const uint4*>(lhist);
    for (int i = threadIdx.x; i < kKeyBins / 4; i += 256) {
      const uint4 v = h4[i];
      if (v.x) atomicAdd(&dst[4 * i], v.x);
      if (v.y) atomicAdd(&dst[4 * i + 1], v.y);
      if (v.z) atomicAdd(&dst[4 * i + 2], v.z);
      if (v.w) atomicAdd(&dst[4 * i + 3], v.w);
    }
  }
}

// Rows that share a request (target-verify, draft-extend v2, extend) read the
// same key pages. This kernel scores each page once for kRows consecutive
// rows: a block takes (group of kRows rows, chunk of 64 pages) and every
// wave scores its page buffer against all rows of the group, so the key
// bytes read per row drop kRows-fold and MFMA work per byte rises as much.
// q (8 KB per row) and the head weights of the group sit in LDS instead of
// registers; the MFMA operands, the order of the ReLU-weight FMAs and the
// transpose-reduce are those of indexer_fp8_kernel, so each row's logits are
// bit-identical to the one-row kernel's. A group whose rows belong to
// different requests is scored one row per pass over that row's pages.
// It always builds the rows' key histograms (the fused top-k input) and
// serves the histogram entry point only.
constexpr int kRows = 4;
constexpr int kQRowBytes = kHeads * kDim;  // 8192
// 64 pages per block (16 per wave): the per-block costs (staging q, clearing
// and flushing four histograms) are spread over twice the MFMA work of the
// one-row kernel's 32; a row's count per bin stays below 2^16 (4096 keys)
constexpr int kRowsPagesPerBlock = 64;

// LDS offset of 16-byte piece `piece` of head h's q row: pieces are rotated by
// (h >> 1) & 7, so the 16 lanes of one ds_read_b128 (heads c = 0..15 of a
// tile, one piece) cover all 64 banks once.
__device__ __forceinline__ int q_lds(int h, int piece) {
  return h * kDim + ((piece ^ ((h >> 1) & 7)) << 4);
}

__global__ void __launch_bounds__(256)
indexer_fp8_rows_kernel(const uint8_t* __restrict__ q, const float* __restrict__ w,
                        const uint8_t* __restrict__ cache, int64_t num_pages,
                        const int32_t* __restrict__ rpt, int64_t rpt_stride,
                        int64_t num_reqs, const int32_t* __restrict__ t2r,
                        const int32_t* __restrict__ seqlens, int max_seqlen_k,
                        int64_t T, float* __restrict__ logits,
                        int64_t logits_stride, int chunks_per_group,
                        uint32_t* __restrict__ key_hist) {
  __shared__ __align__(16) uint8_t sq[kRows * kQRowBytes];
  __shared__ __align__(16) float sw[kRows * kHeads];
  // two 16-bit counts per word: a block writes at most 4096 logits per row
  __shared__ __align__(16) uint32_t lhist[kRows * kKeyBins / 2];

  const int64_t t0 = (int64_t)(blockIdx.x / chunks_per_group) * kRows;
  const int chunk = (int)(blockIdx.x % chunks_per_group);
  const int nrows = (int)min<int64_t>(kRows, T - t0);
  int Lr[kRows];
  int req[kRows];
  bool uniform = true;
  int Lmax = 0;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    int L = r < nrows ? seqlens[t0 + r] : 0;
    L = L < 0 ? 0 : (L > max_seqlen_k ? max_seqlen_k : L);
    int rq = r < nrows ? t2r[t0 + r] : -1;
    if (L > 0 && (rq < 0 || rq >= num_reqs)) {   // no known request: an empty row
      if (chunk == 0 && threadIdx.x == 0) flag_device_error(NSA_DEVERR_REQUEST);
      L = 0;
    }
    Lr[r] = L;
    req[r] = L > 0 ? rq : -1;
    uniform = uniform && (r >= nrows || req[r] == req[0]);
    Lmax = max(Lmax, L);
  }
  const int p_begin = chunk * kRowsPagesPerBlock;
  if (p_begin * kPage >= Lmax) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;

  for (int i = threadIdx.x; i < kRows * kHeads * 8; i += 256) {
    const int r = i >> 9, h = (i >> 3) & 63, piece = i & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < nrows)
      v = *reinterpret_cast<const uint4*>(q + (t0 + r) * kQRowBytes + h * kDim + piece * 16);
    *reinterpret_cast<uint4*>(sq + r * kQRowBytes + q_lds(h, piece)) = v;
  }
  for (int i = threadIdx.x; i < kRows * kHeads; i += 256)
    sw[i] = (i >> 6) < nrows ? w[(t0 + (i >> 6)) * kHeads + (i & 63)] : 0.0f;
  {
    uint4* z = reinterpret_cast<uint4*>(lhist);
    for (int i = threadIdx.x; i < kRows * kKeyBins / 8; i += 256) z[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int npass = uniform ? 1 : nrows;
  for (int pass = 0; pass < npass; ++pass) {
    // rows scored in this pass (bit r = row t0 + r) and their request
    const uint32_t live = uniform ? (1u << nrows) - 1 : 1u << pass;
    const int L = uniform ? Lmax : Lr[pass];
    const int npages = (L + kPage - 1) / kPage;
    if (p_begin >= npages) continue;
    const int p_end = min(p_begin + kRowsPagesPerBlock, npages);
    const int32_t* prow = rpt + (int64_t)req[uniform ? 0 : pass] * rpt_stride;

    const int first = p_begin + wave;
    const int np_w = first < p_end ? (p_end - first + kWaves - 1) / kWaves : 0;
    const int id_lane = lane < np_w ? prow[first + kWaves * lane] : -1;
    if (lane < np_w && (id_lane < 0 || id_lane >= num_pages)) flag_device_error(NSA_DEVERR_PAGE_ID);

    auto page_id = [&](int i) -> int {   // -1: absent or invalid
      const int id = __builtin_amdgcn_readlane(id_lane, i);
      return (id >= 0 && id < num_pages) ? id : -1;
    };
    auto fetch = [&](PageKeys& pk, int i) {
      const int id = page_id(i);
      load_page(pk, cache + (int64_t)(id >= 0 ? id : 0) * kPageBytesFp8, c, g, lane);
    };
    // the 16 (row, head tile) steps of a page run as a software pipeline:
    // the 4 MFMAs of step k+1 are issued before the ReLU-weight FMAs of
    // step k, so the matrix core works while the vector unit reduces
    auto mfma4 = [&](f32x4 (&acc)[4], const PageKeys& pk, int k) {
      const int r = k >> 2, ht = k & 3;
      const uint8_t* qr = sq + r * kQRowBytes;
      const int h = ht * 16 + c;
      const uint4 lo = *reinterpret_cast<const uint4*>(qr + q_lds(h, g));
      const uint4 hi = *reinterpret_cast<const uint4*>(qr + q_lds(h, 4 + g));
      const i32x8 qa = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qa, pk.k[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    };
    auto score = [&](const PageKeys& pk, int i) {
      // q and the weights are re-read from LDS for every page: without this
      // barrier the compiler hoists all four rows' operands into registers
      // (over 300 of them) and the kernel drops to one wave per SIMD
      asm volatile("" ::: "memory");
      const bool b0 = g & 1, b1 = (g >> 1) & 1;
      float res[kRows];
      float v[4];
      f32x4 accA[4], accB[4];
      mfma4(accA, pk, 0);
#pragma unroll
      for (int k = 0; k < kRows * 4; ++k) {
        f32x4 (&cur)[4] = (k & 1) ? accB : accA;
        f32x4 (&nxt)[4] = (k & 1) ? accA : accB;
        if (k + 1 < kRows * 4) mfma4(nxt, pk, k + 1);
        const int r = k >> 2, ht = k & 3;
        const float4 wv = *reinterpret_cast<const float4*>(sw + r * kHeads + ht * 16 + 4 * g);
        const float wr[4] = {wv.x, wv.y, wv.z, wv.w};
        if (ht == 0) v[0] = v[1] = v[2] = v[3] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) v[j] = fmaf(wr[e], relu(cur[j][e]), v[j]);
        if (ht == 3) {
          const float u0 = (b0 ? v[1] : v[0]) + __shfl_xor(b0 ? v[0] : v[1], 16);
          const float u1 = (b0 ? v[3] : v[2]) + __shfl_xor(b0 ? v[2] : v[3], 16);
          res[r] = (b1 ? u1 : u0) + __shfl_xor(b1 ? u0 : u1, 32);
        }
      }
      const bool page_ok = page_id(i) >= 0;
      const int s = (first + kWaves * i) * kPage + lane;   // position of token `lane`
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const float result = page_ok ? res[r] * pk.ks : -INFINITY;
        if (((live >> r) & 1) && i < np_w && s < Lr[r]) {
          logits[(t0 + r) * logits_stride + s] = result;
          const uint32_t bin = order_key(result) >> 20;
          atomicAdd(&lhist[r * (kKeyBins / 2) + (bin >> 1)], (bin & 1) ? 0x10000u : 1u);
        }
      }
    };

    if (np_w > 0) {
      PageKeys b0, b1;
      fetch(b0, 0);
      for (int i = 0; i < np_w; i += 2) {
        fetch(b1, i + 1);
        score(b0, i);
        fetch(b0, i + 2);
        score(b1, i + 1);
      }
    }
  }
  __syncthreads();
  // 16 bytes (8 bins) per thread and step; rows past the group's end skipped
  for (int i = threadIdx.x; i < nrows * kKeyBins / 8; i += 256) {
    const uint4 v4 = reinterpret_cast<const uint4*>(lhist)[i];
    if ((v4.x | v4.y | v4.z | v4.w) == 0) continue;
    const int r = i / (kKeyBins / 8), b = 8 * (i % (kKeyBins / 8));
    uint32_t* dst = key_hist + (t0 + r) * kKeyBins + b;
    const uint32_t v[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[e] & 0xFFFFu) atomicAdd(dst + 2 * e, v[e] & 0xFFFFu);
      if (v[e] >> 16) atomicAdd(dst + 2 * e + 1, v[e] >> 16);
    }
  }
}

// fp32 path (small head counts / dims): one thread per position.
__global__ void __launch_bounds__(256)
indexer_fp32_kernel(const float* __restrict__ q, const float* __restrict__ w,
                    const uint8_t* __restrict__ cache, int64_t num_pages,
                    const int32_t* __restrict__ rpt, int64_t rpt_stride,
                    int64_t num_reqs, const int32_t* __restrict__ t2r,
                    const int32_t* __restrict__ seqlens, int max_seqlen_k,
                    float* __restrict__ logits, int64_t logits_stride, int Hi,
                    int Di, int chunks_per_row) {
  extern __shared__ float smem[];  // q row [Hi*Di] then w [Hi]
  const int64_t t = blockIdx.x / chunks_per_row;
  const int chunk = blockIdx.x % chunks_per_row;
  int L = seqlens[t];
  L = L < 0 ? 0 : (L > max_seqlen_k ? max_seqlen_k : L);
  const int s = chunk * 256 + threadIdx.x;
  if (chunk * 256 >= L) return;
  float* qs = smem;
  float* ws = smem + Hi * Di;
  for (int i = threadIdx.x; i < Hi * Di; i += 256) qs[i] = q[t * Hi * Di + i];
  for (int i = threadIdx.x; i < Hi; i += 256) ws[i] = w[t * Hi + i];
  __syncthreads();
  if (s >= L) return;
  const int32_t req = t2r[t];
  if (req < 0 || req >= num_reqs) {   // no known request: an empty row
    if (chunk == 0 && threadIdx.x == 0) flag_device_error(NSA_DEVERR_REQUEST);
    return;
  }
  const int page = rpt[(int64_t)req * rpt_stride + s / kPage];
  float out = -INFINITY;
  if (page < 0 || page >= num_pages) {
    if (s % kPage == 0) flag_device_error(NSA_DEVERR_PAGE_ID);
  } else {
    const int64_t page_bytes = (int64_t)kPage * Di * 4 + kPage * 4;
    const uint8_t* base = cache + page * page_bytes;
    const float* k = reinterpret_cast<const float*>(base) + (s % kPage) * Di;
    const float ks = reinterpret_cast<const float*>(base + (int64_t)kPage * Di * 4)[s % kPage];
    float acc = 0.0f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.0f;
      for (int e = 0; e < Di; ++e) d = fmaf(qs[h * Di + e], k[e], d);
      acc = fmaf(ws[h], fmaxf(d, 0.0f), acc);
    }
    out = acc * ks;
  }
  logits[t * logits_stride + s] = out;
}

}  // namespace

namespace {

int indexer_run(const char* fn, const void* q, int q_dtype, const float* weights,
                const void* k_index_cache, int k_dtype, int64_t num_pages,
                const int32_t* real_page_table, int64_t rpt_stride,
                int64_t num_reqs, const int32_t* token_to_req,
                const int32_t* seqlens_expanded,
                int T, int Hi, int Di, int page_size, int max_seqlen_k,
                float* logits, int64_t logits_stride, uint32_t* key_hist,
                int rows_per_request, void* stream) {
  NSA_REQUIRE(T >= 0 && max_seqlen_k >= 0 && num_pages >= 0 && num_reqs >= 0,
              NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(page_size == NSA_PAGE_SIZE, NSA_ERR_UNSUPPORTED,
              "%s: page_size %d (only 64 is supported)", fn, page_size);
  NSA_REQUIRE(q_dtype == k_dtype, NSA_ERR_UNSUPPORTED,
              "%s: q and key dtypes must match", fn);
  const bool fp8 = q_dtype == NSA_DTYPE_FP8_E4M3;
  NSA_REQUIRE(fp8 || q_dtype == NSA_DTYPE_FP32, NSA_ERR_UNSUPPORTED,
              "%s: dtype %d (fp8 e4m3 or fp32 only)", fn, q_dtype);
  if (fp8)
    NSA_REQUIRE(Hi == kHeads && Di == kDim, NSA_ERR_UNSUPPORTED,
                "%s: fp8 path needs Hi = 64, Di = 128 (got %d, %d)", fn, Hi, Di);
  else
    NSA_REQUIRE(Hi >= 1 && Hi <= 64 && Di >= 4 && Di <= 128 && Di % 4 == 0,
                NSA_ERR_UNSUPPORTED,
                "%s: fp32 path needs 1 <= Hi <= 64, 4 <= Di <= 128, Di %% 4 == 0",
                fn);
  NSA_REQUIRE(key_hist == nullptr || fp8, NSA_ERR_UNSUPPORTED,
              "%s: the fused histogram needs the fp8 path", fn);
  if (T == 0 || max_seqlen_k == 0) return nsa::ok();
  NSA_REQUIRE(!fp8 || num_pages >= 1, NSA_ERR_INVALID_ARG,
              "%s: empty index-key cache (num_pages 0)", fn);
  NSA_REQUIRE(q && weights && k_index_cache && real_page_table && token_to_req &&
                  seqlens_expanded && logits,
              NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(logits_stride >= max_seqlen_k, NSA_ERR_INVALID_ARG,
              "%s: logits_stride < max_seqlen_k", fn);
  const int64_t ncols = (max_seqlen_k + kPage - 1) / kPage;
  NSA_REQUIRE(rpt_stride >= ncols, NSA_ERR_INVALID_ARG,
              "%s: rpt_stride < ceil(max_seqlen_k/64)", fn);
  NSA_REQUIRE(nsa::aligned(q, 16) && nsa::aligned(weights, 16) &&
                  nsa::aligned(k_index_cache, 16) && nsa::aligned(logits, 4) &&
                  nsa::aligned(key_hist, 4),
              NSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  if (fp8) {
    // odd, so that consecutive rows (row groups) start on different XCDs
    const int chunks = (int)((ncols + kPagesPerBlock - 1) / kPagesPerBlock) | 1;
    if (key_hist && rows_per_request >= kRows) {
      const int rchunks = (int)((ncols + kRowsPagesPerBlock - 1) / kRowsPagesPerBlock) | 1;
      const int64_t blocks = (int64_t)((T + kRows - 1) / kRows) * rchunks;
      NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
      hipLaunchKernelGGL(indexer_fp8_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const uint8_t*>(q), weights,
                         static_cast<const uint8_t*>(k_index_cache), num_pages,
                         real_page_table, rpt_stride, num_reqs, token_to_req,
                         seqlens_expanded, max_seqlen_k, (int64_t)T, logits,
                         logits_stride, rchunks, key_hist);
      return nsa::check_launch(fn);
    }
    const int group = (rows_per_request > 1 && T % rows_per_request == 0) ? rows_per_request : 1;
    int ppb = kPagesPerBlock;
    int chunks_ppb = chunks;
    while (ppb > 8 && (int64_t)T * chunks_ppb < kMinBlocks) {
      ppb /= 2;
      chunks_ppb = (int)((ncols + ppb - 1) / ppb) | 1;
    }
    const int64_t npairs = (int64_t)(T / group) * chunks_ppb;
    const int64_t blocks = (npairs + 7) / 8 * 8 * group;
    NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
    // non-temporal key loads only where no other row reads the same pages
    // (nsa_indexer_logits, which has no hint, passes 1)
    const bool nt = rows_per_request <= 1;
    auto kern = !key_hist ? indexer_fp8_kernel<false, true>
                          : (nt ? indexer_fp8_kernel<true, true> : indexer_fp8_kernel<true, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0,
                       s, static_cast<const uint8_t*>(q), weights,
                       static_cast<const uint8_t*>(k_index_cache), num_pages,
                       real_page_table, rpt_stride, num_reqs, token_to_req,
                       seqlens_expanded, max_seqlen_k, logits, logits_stride,
                       chunks_ppb, ppb, group, npairs, key_hist);
  } else {
    const int chunks = (max_seqlen_k + 255) / 256;
    const int64_t blocks = (int64_t)T * chunks;
    NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
    const size_t shm = (size_t)(Hi * Di + Hi) * sizeof(float);
    hipLaunchKernelGGL(indexer_fp32_kernel, dim3((unsigned)blocks), dim3(256),
                       shm, s, static_cast<const float*>(q), weights,
                       static_cast<const uint8_t*>(k_index_cache), num_pages,
                       real_page_table, rpt_stride, num_reqs, token_to_req,
                       seqlens_expanded, max_seqlen_k, logits, logits_stride,
                       Hi, Di, chunks);
  }
  return nsa::check_launch(fn);
}

}  // namespace

extern "C" int nsa_indexer_logits(const void* q, int q_dtype,
                                  const float* weights,
                                  const void* k_index_cache, int k_dtype,
                                  int64_t num_pages,
                                  const int32_t* real_page_table,
                                  int64_t rpt_stride, int64_t num_reqs,
                                  const int32_t* token_to_req,
                                  const int32_t* seqlens_expanded, int T,
                                  int Hi, int Di, int page_size,
                                  int max_seqlen_k, float* logits,
                                  int64_t logits_stride, void* stream) {
  return indexer_run("nsa_indexer_logits", q, q_dtype, weights, k_index_cache,
                     k_dtype, num_pages, real_page_table, rpt_stride, num_reqs,
                     token_to_req, seqlens_expanded, T, Hi, Di, page_size,
                     max_seqlen_k, logits, logits_stride, nullptr, 1, stream);
}

extern "C" int nsa_indexer_logits_hist(const void* q, int q_dtype,
                                       const float* weights,
                                       const void* k_index_cache, int k_dtype,
                                       int64_t num_pages,
                                       const int32_t* real_page_table,
                                       int64_t rpt_stride, int64_t num_reqs,
                                       const int32_t* token_to_req,
                                       const int32_t* seqlens_expanded, int T,
                                       int Hi, int Di, int page_size,
                                       int max_seqlen_k, float* logits,
                                       int64_t logits_stride, uint32_t* key_hist,
                                       int rows_per_request, void* stream) {
  const char* fn = "nsa_indexer_logits_hist";
  NSA_REQUIRE(T == 0 || key_hist != nullptr, NSA_ERR_INVALID_ARG,
              "%s: null key_hist", fn);
  return indexer_run(fn, q, q_dtype, weights, k_index_cache, k_dtype, num_pages,
                     real_page_table, rpt_stride, num_reqs, token_to_req,
                     seqlens_expanded,
                     T, Hi, Di, page_size, max_seqlen_k, logits, logits_stride,
                     key_hist, rows_per_request, stream);
}
