// a4 / a5 at 128 heads over an fp8 block-scaled cache: MLA attention over
// the selected KV slots ("nsa_backend.py (EngineX-Hygon sglang fork)",
// _forward_flashmla_decode; "dsa_backend.py (sglang main)",
// _forward_flashmla_kv: q [T, 128, 576] over the fp8 cache, output o and
// lse). Same function as the kernels of sparse_mla.hip; this unit is built
// with the VGPR form of the MFMA instructions (the score accumulators), while
// the P.V MFMAs, whose accumulators fill the 256 AGPRs, are written in
// inline asm in their AGPR form.
#include "sparse_mla_shared.h"

namespace nsa_mla {
namespace {

// ---- 128-head kernel (fp8 cache, H = 128) ----------------------------------
// A block owns one query row, all 128 heads and one KV split, so each
// gathered fp8 row is dequantised once for all heads (the 64-head kernel of
// sparse_mla.hip does it once per 64-head block, two blocks per row). More
// than 128 rows (target-verify, draft-extend) take one block per row; fewer
// rows are split over KV so that about 256 blocks fill the CUs. Wave w owns
// heads 32w .. 32w+31 and, for them, the whole 576-wide contraction and all
// 512 value dims: no partial scores are exchanged between waves and each
// softmax runs once. Q (36 bf16x8 B operands) stays in VGPRs, the O^T accumulators
// (16 tiles of 32 value dims x 32 heads) in AGPRs.
//   * S^T = K.Q^T with v_mfma_f32_32x32x16_bf16: A = 32 slots x 16 dims of
//     the bf16 K tile (LDS), B = Q^T; lane (head c32, half kg) receives the
//     16 scores of its head for slots 8(e/4) + 4kg + e%4, so the softmax of a
//     head is in-lane (two lanes per head);
//   * O^T = V^T.P^T: A = V^T read with ds_read_b64_tr_b16 from the same tile,
//     B = P^T straight from the lane's own probabilities; lane (head c32, kg)
//     ends up holding its head's 4-dim groups 8j + 4kg of every value tile, so
//     normalisation needs no shuffle and the output is written in 8-byte runs;
//   * gather: each wave loads the 656-byte rows of its 8 slots of a step with
//     16-byte direct global->LDS loads (no staging registers; one instruction
//     per row, lanes 0..40, the slot id a wave-uniform scalar) into a raw
//     buffer of its own, about two iterations before it dequantises them
//     (bf16(code * block scale), round to nearest even) into the step's K
//     tile, so waiting on its own loads is enough and the step needs one
//     barrier;
//   * pipeline (iteration k): the dequantisation of step k+1 and then the
//     loads of step k+3 into the same raw buffer, and the softmax of step k,
//     are cut into small stages spread over the 36 MFMAs of S^T(k) and the 32
//     of O^T += V^T(k-1).P^T(k-1), each MFMA covering about as much VALU work
//     as the SIMD issues while it runs (with one wave per SIMD a wave's VALU
//     instructions run under its own MFMAs only when they do not wait on each
//     other); three K tiles, two raw buffers, P double-buffered in registers;
//   * softmax as in the 64-head kernel: a fixed per-head reference max (the
//     first step with a valid slot), exponents clamped, an exact re-run of the
//     row when a later score exceeds the reference by more than 2^64;
//   * output: each wave stages its heads' rows (bf16, divided by l) in LDS
//     and writes each head's 1 KB row with one coalesced store, into the
//     output (one split) or into the workspace as the split's partial, with
//     its log-sum-exp, for the merge kernel of sparse_mla.hip.
constexpr int kW128Slots = 8;                               // rows per wave and step
constexpr int kRawRow = 656;
constexpr int kRawWave = kW128Slots * kRawRow;              // 5248
constexpr int kRawStage = 4 * kRawWave;                     // 20992
constexpr int kRowPieces = kRawRow / 16;                    // 41 16-byte pieces per row
constexpr int kDmaInsts = kW128Slots;                       // one load instruction per row
constexpr int kIds128 = kMaxSplit + 4 * kStep;              // ids of a row + overrun
static_assert(kDmaInsts == 8, "a step's row ids are read by lanes 0..7 of the wave");
constexpr int kQSteps = kDQK / 16;                          // 36 contraction steps
constexpr int kVTiles = kDV / 32;                           // 16 value tiles
// output staging: 16 rows of 1024 bytes per wave; the 1040-byte stride puts
// the 8-byte writes of the 32 active lanes on distinct banks
constexpr int kFinRow = 1040;
constexpr int kFinWave = 16 * kFinRow;
static_assert(4 * kFinWave <= 3 * kKsBytes, "output staging fits in the tiles");

typedef __attribute__((address_space(3))) void* lds_void_ptr;

template <int B>
struct RawBuf;
__shared__ __attribute__((aligned(16))) uint8_t g_raw0[kRawStage];
__shared__ __attribute__((aligned(16))) uint8_t g_raw1[kRawStage];
template <>
struct RawBuf<0> { static __device__ __forceinline__ uint8_t* get() { return g_raw0; } };
template <>
struct RawBuf<1> { static __device__ __forceinline__ uint8_t* get() { return g_raw1; } };

// The row loads into LDS are written in inline asm, so the compiler does
// not see them as LDS writes: left to itself it waits for every load in
// flight before any LDS read it cannot prove to lie elsewhere, which after
// its address rewriting is most of them. Ordering is then by hand: a row's
// raw buffer is read only after wait_vm_dma, which (the asm has a memory
// clobber) the compiler does not move reads above, and every wave waits
// for all of its loads before the LDS is used otherwise or the wave ends.
// One load instruction brings one 656-byte row: M0 = the row's LDS
// destination (the operand is bound to M0, so the compiler writes it), lane
// i < 41 writes bytes [16i, 16i+16) at M0 + 16 i; the other lanes are
// switched off inside the asm (EXEC saved and restored there), so that the
// code around it stays one basic block: the compiler does not move work
// between basic blocks of the unrolled loop as it would around a branch.
// One wait state between the write of M0 and the load that reads it.
constexpr uint64_t kRowLanes = (1ull << kRowPieces) - 1;
__device__ __forceinline__ void lds_dma_row(const uint8_t* src, uint32_t lds_addr) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(src), "s"(kRowLanes), "{m0}"(lds_addr)
      : "memory");
}

__device__ __forceinline__ void wait_vm_dma() {
  // every load of this wave but the kDmaInsts most recent ones has landed
  // (the only vector-memory instructions of the loop are these row loads)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaInsts) : "memory");
}
// the same with the 36 Q loads issued after the most recent row loads
__device__ __forceinline__ void wait_vm_dma_q() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaInsts + 36) : "memory");
}

__global__ void __launch_bounds__(256, 1)
sparse_mla_h128_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[3][kKsBytes];
  __shared__ __attribute__((aligned(16))) float bias[3][kStep];
  __shared__ __attribute__((aligned(16))) int32_t ids[kIds128];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, kg = lane >> 5;
  const int grp = lane >> 4, sl = lane & 15;
  const int h = wave * 32 + c32;                       // this lane's head

  // one block per (query row, KV split); the plan keeps split_slots <=
  // kMaxSplit
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int split = lb % p.n_splits;
  const int64_t t = lb / p.n_splits;

  int n_row = p.num_slots > 0 ? p.topk : 0;
  if (p.seqlens) {
    const int sl_ = p.seqlens[t];
    n_row = sl_ < 0 ? 0 : (sl_ < n_row ? sl_ : n_row);
  }
  const int s_begin = split * p.split_slots;
  const int n = min(s_begin + p.split_slots, n_row) - s_begin;   // may be <= 0
  const int nsteps = n > 0 ? (n + kStep - 1) / kStep : 0;

  // ---- slot ids of the row (validated; -1 past its end and for bad ids)
  {
    const int32_t* irow = p.idx + t * p.idx_stride + s_begin;
    const int last = n > 0 ? n - 1 : 0;
    constexpr int kPer = (kIds128 + 255) / 256;
    int32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = irow[min(tid + k * 256, last)];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * 256;
      const int32_t id = v[k];
      if (i < n && (id < -1 || id >= p.num_slots)) flag_device_error(NSA_DEVERR_SLOT);
      if (i < kIds128) ids[i] = (i < n && id >= 0 && id < p.num_slots) ? id : -1;
    }
  }

  // ids visible to every wave (no wait for other loads)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  // Q^T operands: lane (head c32, kg) holds dims 16i + 8kg .. +8; loaded
  // once, behind the first row loads (the load of Q overlaps the rows'
  // latency and the first dequantisation)
  bf16x8 qb[kQSteps];
  static_assert(kQSteps == 36, "the prologue's wait counts 36 Q loads");
  auto load_q = [&]() {
    const uint16_t* qh = p.q + t * p.q_tok_stride + (int64_t)h * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < kQSteps; ++i)
      qb[i] = *reinterpret_cast<const bf16x8*>(qh + 16 * i + 8 * kg);
  };

  // ---- gather (direct to LDS) and dequantisation of this wave's 8 rows
  // row j of this wave's slots of `step`: lane i < 41 loads bytes [16i,
  // 16i+16) of the slot's 656-byte row into the wave's raw buffer
  const uint8_t* kv_lane = p.kv + lane * 16;
  auto dma_row_id = [&](uint8_t* stage, int32_t id, int j) {
    // the row's byte offset in scalar registers, added to the lane's base
    uint64_t off = (uint64_t)(uint32_t)(id >= 0 ? id : 0) * kRawRow;
    asm volatile("" : "+s"(off));
    // 32-bit LDS address arithmetic (a generic-pointer sum would be kept
    // in 64-bit registers)
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_void_ptr)stage + wave * kRawWave + j * kRawRow;
    lds_dma_row(kv_lane + off, __builtin_amdgcn_readfirstlane(dst));
  };
  auto dma_row = [&](uint8_t* stage, int step, int j) {
    dma_row_id(stage, __builtin_amdgcn_readfirstlane(ids[step * kStep + wave * kW128Slots + j]), j);
  };
  auto dma = [&](uint8_t* stage, int step) {
#pragma unroll
    for (int j = 0; j < kDmaInsts; ++j) dma_row(stage, step, j);
  };
  // lane (sub = lane / 8, cc = lane % 8): row 8w + sub of the step, code
  // pieces cc + 8b (128-block b), rope piece cc
  const int dsub = lane >> 3, dcc = lane & 7;
  const int drow = wave * kW128Slots + dsub;
  // Dequantisation of the wave's 8 rows of a step: 32 half-words per lane
  // (two codes each), each in three stages: A converts the codes, B
  // multiplies by the block scale, C rounds to bf16 (and stores the word's 4
  // dims after its second half). Inside the loop the stages of consecutive
  // half-words are skewed over consecutive score MFMAs (C of h-2, B of h-1
  // and A of h together), so no stage waits on the one before it; empty asm
  // statements pin each stage's results where they are computed.
  struct Deq {
    const uint8_t* rr;
    u32x4 pc[2];      // raw pieces b (pc[b & 1]) and b + 1; the rope in pc[0]
    float scale[2];   // block scales of pieces b (scale[b & 1]) and b + 1
    int32_t id;       // the row's slot id (-1: absent)
    float fa[2], fb[2];
    u32x4 bf;         // bf16 pairs of the 8 dims being converted
  };
  auto deq_piece = [&](Deq& d, int b) {
    d.pc[b & 1] = *reinterpret_cast<const u32x4*>(d.rr + (b < 4 ? 16 * (dcc + 8 * b) : 528 + 16 * dcc));
  };
  auto deq_load = [&](Deq& d, const uint8_t* stage, int step) {
    d.rr = stage + wave * kRawWave + dsub * kRawRow;
    d.id = ids[step * kStep + drow];
    d.scale[0] = *reinterpret_cast<const float*>(d.rr + 512);
    deq_piece(d, 0);
  };
  auto deq_scale = [&](Deq& d, int b) {
    d.scale[b & 1] = *reinterpret_cast<const float*>(d.rr + 512 + 4 * b);
  };
  // an absent slot's scales are 0 (applied before the block's first use)
  auto deq_mask = [&](Deq& d, int b) { d.scale[b & 1] = d.id >= 0 ? d.scale[b & 1] : 0.0f; };
  auto deqA = [&](Deq& d, int h) {
    const uint32_t word = d.pc[(h >> 3) & 1][(h >> 1) & 3];
    const auto f = (h & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true)
                           : __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
    d.fa[0] = f[0];
    d.fa[1] = f[1];
    asm volatile("" : "+v"(d.fa[0]), "+v"(d.fa[1]));
  };
  auto deqB = [&](Deq& d, int h) {
    const float s = d.scale[(h >> 3) & 1];
    d.fb[0] = d.fa[0] * s;
    d.fb[1] = d.fa[1] * s;
    asm volatile("" : "+v"(d.fb[0]), "+v"(d.fb[1]));
  };
  auto deqC = [&](Deq& d, uint8_t* kt, int h) {
    const int b = h >> 3, w = (h >> 1) & 3;
    d.bf[h & 3] = pack_bf16x2_hw(d.fb[0], d.fb[1]);
    if ((h & 3) == 3) {
      uint8_t* dst = static_cast<uint8_t*>(__builtin_assume_aligned(kt, 16));
      *reinterpret_cast<u32x4*>(dst + drow * kKsRow + 32 * (dcc + 8 * b) + 16 * (w >> 1)) = d.bf;
    } else {
      asm volatile("" : "+v"(d.bf));
    }
  };
  // the rope piece (held in pc[0]) and the score bias; an absent slot
  // stores zeros and a -inf bias
  auto deq_rope = [&](const Deq& d, uint8_t* kt, float* bs) {
    const uint32_t msk = d.id >= 0 ? 0xFFFFFFFFu : 0u;
    *reinterpret_cast<u32x4*>(kt + drow * kKsRow + kDV * 2 + 16 * dcc) = d.pc[0] & msk;
    if (dcc == 0) bs[drow] = d.id >= 0 ? 0.0f : -INFINITY;
  };
  auto deq_full = [&](const uint8_t* stage, int step, uint8_t* kt, float* bs) __attribute__((always_inline)) {
    Deq d;
    deq_load(d, stage, step);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b > 0) deq_scale(d, b);
      if (b < 3) deq_piece(d, b + 1);
      deq_mask(d, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        deqA(d, 8 * b + i);
        deqB(d, 8 * b + i);
        deqC(d, kt, 8 * b + i);
      }
    }
    deq_piece(d, 4);
    deq_rope(d, kt, bs);
  };

  f32x16 o[kVTiles];
  constexpr float kMaxExp = 64.0f;
  float m, l, mall;
  bool ovf;

  constexpr int kPf = 2;                     // fragment prefetch distance
  constexpr int kRing = kPf + 1;

  // Softmax of one step's scores (lane: head c32, 16 slots e in acc), in
  // stages that the loop skews over consecutive P.V MFMAs:
  //   F(i): scores 2i, 2i + 1 scaled and biased; M(i): their maximum taken;
  //   R: the head's maximum, the reference and the overflow check (after a
  //     lane exchange);
  //   S(e), X(e), L(e): score e minus the reference, its exponential, its
  //     sum into l;
  //   W(e) (e even): slots e, e + 1 of P^T packed (lane (head c32, kg) holds
  //     slots 16ch + 4kg + {0..3, 8..11} of chunk ch = e / 8).
  // The biases bia[j] (slots 8j + 4kg .. +3) are read beforehand.
  float m_use = 0.0f, lmx = -INFINITY, hmx = -INFINITY;
  float4 bia[4];
  uint32_t pk[3];
  auto bias_read = [&](const float* bs, int j) {
    bia[j] = *reinterpret_cast<const float4*>(bs + 8 * j + 4 * kg);
  };
  auto smF = [&](f32x16& acc, int i) {
    const int e = 2 * i;
    const float4 bv = bia[e >> 2];
    acc[e] = fmaf(acc[e], p.scale_log2, (e & 3) == 0 ? bv.x : bv.z);
    acc[e + 1] = fmaf(acc[e + 1], p.scale_log2, (e & 3) == 0 ? bv.y : bv.w);
    asm volatile("" : "+v"(acc[e]), "+v"(acc[e + 1]));
  };
  auto smM = [&](const f32x16& acc, int i) {
    const float mx = fmaxf(acc[2 * i], acc[2 * i + 1]);
    lmx = i == 0 ? mx : fmaxf(lmx, mx);
    asm volatile("" : "+v"(lmx));
  };
  auto smR0 = [&]() {
    mall = fmaxf(mall, lmx);
    // head c32 in both kg: the two 32-lane halves exchanged by a VALU swap
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lmx), __float_as_uint(lmx),
                                                     false, false);
    hmx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    asm volatile("" : "+v"(hmx));
  };
  auto smR1 = [&]() {
    m = m == -INFINITY ? hmx : m;            // first step with a valid slot
    ovf = ovf || lmx > m + kMaxExp;
    m_use = m == -INFINITY ? 0.0f : m;
    asm volatile("" : "+v"(m_use));
  };
  // a score beyond m + kMaxExp sets ovf and the row is run again, so its
  // weight need not be finite
  auto smS = [&](f32x16& acc, int e) {
    acc[e] = acc[e] - m_use;
    asm volatile("" : "+v"(acc[e]));
  };
  auto smX = [&](f32x16& acc, int e) {
    acc[e] = __builtin_amdgcn_exp2f(acc[e]);
    asm volatile("" : "+v"(acc[e]));
  };
  auto smL = [&](const f32x16& acc, int e) {
    l += acc[e];
    asm volatile("" : "+v"(l));
  };
  auto smW = [&](const f32x16& acc, bf16x8 (&pn)[2], int e) {
    const int ch = e >> 3, wd = (e >> 1) & 3;
    const uint32_t w = pack_bf16x2_hw(acc[e], acc[e + 1]);
    if (wd < 3) {
      pk[wd] = w;
      asm volatile("" : "+v"(pk[wd]));
    } else {
      const uint4 u = make_uint4(pk[0], pk[1], pk[2], w);
      pn[ch] = *reinterpret_cast<const bf16x8*>(&u);
    }
  };
  auto softmax_full = [&](f32x16& acc, const float* bs, bf16x8 (&pn)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bias_read(bs, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) { smF(acc, i); smM(acc, i); }
    smR0();
    smR1();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      smS(acc, e);
      smX(acc, e);
      smL(acc, e);
      if (e & 1) smW(acc, pn, e - 1);
    }
  };

  // ---- iteration k: 68 instruction groups, one MFMA each (scheduling
  // barriers between groups), the other work spread so that each group
  // holds about as much VALU work as its MFMA covers:
  //   phase 1, groups 0..35: the MFMAs of S^T(k) from tile k; the
  //     dequantisation of step k+1 (its rows landed in raw buffer
  //     (k+1) % 2) into tile k+1: stages A, B, C of half-word h in groups
  //     3 + h, 4 + h, 5 + h (the last C in phase 2), raw piece b read in
  //     group 8b, block scale b in group 8b + 1, the rope and bias in group
  //     35; the row ids of step k+3 read;
  //   phase 2, groups 0..31: the MFMAs of O^T += V^T(k-1).P^T(k-1) from tile
  //     k-1 (tile q % 16, slot chunk q / 16); the loads of step k+3's rows
  //     into the raw buffer just dequantised (groups 0, 1 and 27..30); the
  //     softmax of step k into pn = P(k): biases read in groups 0, 1, F(i)
  //     in group 3 + i, M(i) in 4 + i, R in 12 and 13, S(e), X(e), L(e) in
  //     14 + e, 15 + e, 16 + e, W(e) in 17 + e.
  // Fragments are read kPf MFMAs ahead into a ring of kPf + 1.
  auto iter = [&](int k, f32x16& acc, bf16x8 (&pa)[2], bf16x8 (&pn)[2], uint8_t* raw) {
    const uint8_t* ktc = ks[k % 3];          // step k: scores
    const uint8_t* ktp = ks[(k + 2) % 3];    // step k-1: P.V
    uint8_t* ktn = ks[(k + 1) % 3];          // step k+1: dequantised now
    const float* bsc = bias[k % 3];
    float* bsn = bias[(k + 1) % 3];
    int32_t idl;
    int32_t sid[kDmaInsts];
    Deq dq;
    {
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(ktc + c32 * kKsRow + (16 * i + 8 * kg) * 2);
      };
      bf16x8 fr[kRing];
#pragma unroll
      for (int i = 0; i < kPf; ++i) fr[i] = kfrag(i);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int g = 0; g < kQSteps; ++g) {
        if (g + kPf < kQSteps) fr[(g + kPf) % kRing] = kfrag(g + kPf);
        __builtin_amdgcn_sched_barrier(0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[g % kRing], qb[g], acc, 0, 0, 0);
        if (g == 0) {
          wait_vm_dma();   // the rows of step k+1
          deq_load(dq, raw, k + 1);
        } else if (g == 1) {
          // lane j < 8 reads the id of row j of step k+3
          idl = ids[(k + 3) * kStep + wave * kW128Slots + (lane & 7)];
        } else if (g == 5 || g == 6) {
#pragma unroll
          for (int j = 4 * (g - 5); j < 4 * (g - 4); ++j) sid[j] = __builtin_amdgcn_readlane(idl, j);
        }
        if (g % 8 == 0 && g > 0 && g <= 32) deq_piece(dq, g / 8);
        if (g % 8 == 1 && g > 1 && g <= 25) deq_scale(dq, g / 8);
        if (g % 8 == 3 && g <= 27) deq_mask(dq, g / 8);
        if (g >= 5) deqC(dq, ktn, g - 5);
        if (g >= 4) deqB(dq, g - 4);
        if (g >= 3 && g < 35) deqA(dq, g - 3);
        if (g == kQSteps - 1) deq_rope(dq, ktn, bsn);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      const uint8_t* vbase = ktp + (4 * kg + (sl >> 2)) * kKsRow + (16 * (grp & 1) + 4 * (sl & 3)) * 2;
      auto vfrag = [&](int q) {
        const uint8_t* src = vbase + 16 * (q >> 4) * kKsRow + (q & 15) * 64;
        const v4i16 b0 = read_tr(src);
        const v4i16 b1 = read_tr(src + 8 * kKsRow);
        const v4i16 bb[2] = {b0, b1};
        return *reinterpret_cast<const bf16x8*>(bb);
      };
      bf16x8 vf[kRing];
#pragma unroll
      for (int i = 0; i < kPf; ++i) vf[i] = vfrag(i);
#pragma unroll
      for (int q = 0; q < 2 * kVTiles; ++q) {
        if (q + kPf < 2 * kVTiles) vf[(q + kPf) % kRing] = vfrag(q + kPf);
        __builtin_amdgcn_sched_barrier(0);
        // inline asm: the AGPR form of the MFMA for O^T (the 256 AGPRs) while
        // the score MFMAs above use the VGPR form; P (pa) was written by VALU
        // at least one phase earlier, so no wait states are owed here
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(o[q & 15]) : "v"(vf[q % kRing]), "v"(pa[q >> 4]));
        if (q == 0) deqC(dq, ktn, 31);
        // loads of step k+3 into the raw buffer whose rows were dequantised
        // in phase 1 (every read of it has been waited for)
        if (q < 2) {
          dma_row_id(raw, sid[2 * q], 2 * q);
          dma_row_id(raw, sid[2 * q + 1], 2 * q + 1);
          bias_read(bsc, 2 * q);
          bias_read(bsc, 2 * q + 1);
        } else if (q >= 27 && q < 31) {
          dma_row_id(raw, sid[q - 23], q - 23);
        }
        // softmax of step k
        if (q >= 4 && q < 12) smM(acc, q - 4);
        if (q >= 3 && q < 11) smF(acc, q - 3);
        if (q == 12) smR0();
        if (q == 13) smR1();
        if (q >= 17 && (q - 17) % 2 == 0) smW(acc, pn, q - 17);
        if (q >= 16) smL(acc, q - 16);
        if (q >= 15 && q < 31) smX(acc, q - 15);
        if (q >= 14 && q < 30) smS(acc, q - 14);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  };

  // scores of step 0 (prologue)
  auto qk0 = [&](f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < kQSteps; ++i) {
      const bf16x8 f = *reinterpret_cast<const bf16x8*>(ks[0] + c32 * kKsRow + (16 * i + 8 * kg) * 2);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qb[i], acc, 0, 0, 0);
    }
  };
  auto run_pass = [&](bool first) {
#pragma unroll
    for (int d = 0; d < kVTiles; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
      asm volatile("" : "+a"(o[d]));   // O^T lives in AGPRs (MFMA C/D operands)
    }
    l = 0.0f;
    if (nsteps > 0) {
      f32x16 acc;
      bf16x8 pA[2], pB[2];
      uint8_t* r0 = RawBuf<0>::get();
      uint8_t* r1 = RawBuf<1>::get();
      // prologue: rows of steps 0 and 1 in flight, step 0 dequantised into
      // tile 0, the rows of step 2 requested, the scores and P of step 0
      // taken, step 1 dequantised into tile 1, the rows of step 3 requested
      dma(r0, 0);
      dma(r1, 1);
      if (first) {
        load_q();
        wait_vm_dma_q();
      } else {
        wait_vm_dma();
      }
      deq_full(r0, 0, ks[0], bias[0]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      dma(r0, 2);   // raw buffer 0 (step 0) was read by this wave only
      qk0(acc);
      softmax_full(acc, bias[0], pA);
      wait_vm_dma();
      deq_full(r1, 1, ks[1], bias[1]);
      dma(r1, 3);   // raw buffer 1 (step 1) was read by this wave only
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      // iteration k: scores of step k, P.V of step k-1, dequantisation of
      // k+1 from raw buffer (k+1) % 2, then the loads of k+3 into it; steps
      // past nsteps are empty (every bias -inf, P zero)
      // (iteration nsteps does the P.V of the last step; its own scores are
      // those of an empty step)
      for (int k = 1; k <= nsteps; k += 2) {
        iter(k, acc, pA, pB, r0);
        if (k + 1 <= nsteps) iter(k + 1, acc, pB, pA, r1);
      }
    }
  };

  // The P.V MFMAs are inline asm, so the compiler cannot see that the AGPRs
  // of O^T are written by an MFMA: wait out the MFMA's write latency by hand
  // before O^T is read (finalize) or cleared (re-run).
  auto mfma_drain = []() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); };
  m = -INFINITY;
  mall = -INFINITY;
  ovf = false;
  run_pass(true);
  mfma_drain();
  // a score beyond the clamp anywhere in the block: run again with the true
  // maximum as reference
  if (tid == 0) s_flag = 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(ovf) != 0 && lane == 0) s_flag = 1;
  __syncthreads();
  if (s_flag != 0) {
    m = fmaxf(mall, __shfl_xor(mall, 32));
    ovf = false;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads of the first pass
    __syncthreads();
    run_pass(false);
    mfma_drain();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // trailing loads into LDS

  // ---- finalize: lane (head c32, kg) element e of tile d holds value dim
  // 32d + 8(e/4) + 4kg + e%4 of head h. The rows (bf16, divided by l) go
  // through LDS, 16 heads of the wave at a time, so that each head's 1 KB
  // row is written by one coalesced store of the wave.
  l += __shfl_xor(l, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse_val = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  const bool direct = p.n_splits == 1;
  uint16_t* obase = direct ? p.out + (t * p.H + wave * 32) * kDV
                           : reinterpret_cast<uint16_t*>(p.ws_o) +
                                 (((int64_t)split * p.T + t) * p.H + wave * 32) * kDV;
  __syncthreads();   // every wave is done with the tiles
  uint8_t* tw = &ks[0][0] + wave * kFinWave;   // this wave's staging rows
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((c32 >> 4) == half) {
      uint8_t* row = tw + (c32 & 15) * kFinRow + 8 * kg;
#pragma unroll
      for (int d = 0; d < kVTiles; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(row + (32 * d + 8 * j) * 2) =
              make_uint2(pack_bf16x2(o[d][4 * j] * inv, o[d][4 * j + 1] * inv),
                         pack_bf16x2(o[d][4 * j + 2] * inv, o[d][4 * j + 3] * inv));
    }
    // one wave writes and reads its own rows (LDS accesses of a wave are
    // performed in order)
#pragma unroll 4
    for (int r = 0; r < 16; ++r)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tw + r * kFinRow + 16 * lane),
                                  reinterpret_cast<u32x4*>(obase + (16 * half + r) * kDV + 8 * lane));
  }
  if (kg == 0) {
    if (direct) {
      if (p.lse) p.lse[t * p.H + h] = lse_val;
    } else {
      p.ws_lse[((int64_t)split * p.T + t) * p.H + h] = lse_val;
    }
  }
}

}  // namespace

int launch_sparse_mla_h128(const Params& p, unsigned blocks, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_h128_kernel, dim3(blocks), dim3(256), 0, s, p);
  return 0;
}

}  // namespace nsa_mla
