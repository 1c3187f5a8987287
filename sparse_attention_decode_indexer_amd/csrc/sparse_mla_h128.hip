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
//     per row, lanes 0..40, the slot id a wave-uniform scalar), two steps
//     ahead, into a raw buffer of its own; the same wave then dequantises
//     those rows (bf16(code * block scale), round to nearest even) into the
//     step's K tile, so waiting on its own loads is enough and the step needs
//     one barrier;
//   * pipeline (iteration k): the loads of step k+2, the softmax of step k-1
//     and the dequantisation of step k+1 are spread between the 36 MFMAs of
//     S^T(k) and the 32 of O^T += V^T(k-1).P^T(k-1); three K tiles, two raw
//     buffers, scores double-buffered in registers;
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
static_assert(kDmaInsts == 8, "row ids are read as two int4");
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
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint32_t lds_addr) {
  // M0 = the wave's LDS destination (the operand is bound to M0, so the
  // compiler writes it); lane i writes 16 bytes at M0 + 16 i. One wait state
  // between the write of M0 and the load that reads it.
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ void wait_vm_dma() {
  // every load of this wave but the kDmaInsts most recent ones has landed
  // (the only vector-memory instructions of the loop are these row loads)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaInsts) : "memory");
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

  // Q^T operands: lane (head c32, kg) holds dims 16i + 8kg .. +8
  bf16x8 qb[kQSteps];
  {
    const uint16_t* qh = p.q + t * p.q_tok_stride + (int64_t)h * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < kQSteps; ++i)
      qb[i] = *reinterpret_cast<const bf16x8*>(qh + 16 * i + 8 * kg);
  }
  __syncthreads();   // ids

  // ---- gather (direct to LDS) and dequantisation of this wave's 8 rows
  // row j of this wave's slots of `step`: lane i < 41 loads bytes [16i,
  // 16i+16) of the slot's 656-byte row into the wave's raw buffer
  auto dma_row_id = [&](uint8_t* stage, int32_t id, int j) {
    const uint8_t* src = p.kv + (int64_t)(id >= 0 ? id : 0) * kRawRow;
    // 32-bit LDS address arithmetic (a generic-pointer sum would be kept
    // in 64-bit registers)
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_void_ptr)stage + wave * kRawWave + j * kRawRow;
    if (lane < kRowPieces) lds_dma16(src + lane * 16, __builtin_amdgcn_readfirstlane(dst));
  };
  auto dma_row = [&](uint8_t* stage, int step, int j) {
    dma_row_id(stage, __builtin_amdgcn_readfirstlane(ids[step * kStep + wave * kW128Slots + j]), j);
  };
  auto dma = [&](uint8_t* stage, int step) {
#pragma unroll
    for (int j = 0; j < kDmaInsts; ++j) dma_row(stage, step, j);
  };
  // the wave's row ids of `step`, read ahead into scalar registers (a read
  // of one in front of each row load would make every load wait for all
  // LDS reads in flight)
  auto read_ids = [&](int32_t (&sid)[kDmaInsts], int step) {
    const int4* ip = reinterpret_cast<const int4*>(ids + step * kStep + wave * kW128Slots);
    const int4 a = ip[0], b = ip[1];
    const int32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < kDmaInsts; ++j) sid[j] = __builtin_amdgcn_readfirstlane(v[j]);
  };
  // lane (sub = lane / 8, cc = lane % 8): row 8w + sub of the step, code
  // pieces cc + 8b (128-block b), rope piece cc
  const int dsub = lane >> 3, dcc = lane & 7;
  const int drow = wave * kW128Slots + dsub;
  // A row's raw piece b (code pieces b < 4, rope piece 4) is read one group
  // before it is stored: a read issued just before its use would make it
  // wait for every fragment read in flight as well.
  struct Deq {
    const uint8_t* rr;
    u32x4 pc[5];
    f32x4 scale;
    bool valid;
  };
  auto deq_fetch = [&](Deq& d, int b) {
    d.pc[b] = *reinterpret_cast<const u32x4*>(d.rr + (b < 4 ? 16 * (dcc + 8 * b) : 528 + 16 * dcc));
  };
  auto deq_load = [&](Deq& d, const uint8_t* stage, int step) {
    d.rr = stage + wave * kRawWave + dsub * kRawRow;
    d.valid = ids[step * kStep + drow] >= 0;
    d.scale = *reinterpret_cast<const f32x4*>(d.rr + 512);
    deq_fetch(d, 0);
  };
  // piece b < 4: bf16(code * scale_b) of block b (32 bytes); piece 4: rope
  // and the score bias. An absent slot stores zeros and a -inf bias.
  auto deq_store = [&](const Deq& d, uint8_t* kt, float* bs, int b) {
    if (b < 4) {
      const u32x4 code = d.pc[b];
      const float s = d.valid ? d.scale[b] : 0.0f;
      const uint32_t w[4] = {code[0], code[1], code[2], code[3]};
      uint32_t bf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        bf[2 * i] = pack_bf16x2_hw(lo[0] * s, lo[1] * s);
        bf[2 * i + 1] = pack_bf16x2_hw(hi[0] * s, hi[1] * s);
      }
      uint8_t* dst = kt + drow * kKsRow + 32 * (dcc + 8 * b);
      *reinterpret_cast<uint4*>(dst) = make_uint4(bf[0], bf[1], bf[2], bf[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(bf[4], bf[5], bf[6], bf[7]);
    } else {
      const u32x4 rope = d.pc[4];
      const uint32_t msk = d.valid ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<u32x4*>(kt + drow * kKsRow + kDV * 2 + 16 * dcc) = rope & msk;
      if (dcc == 0) bs[drow] = d.valid ? 0.0f : -INFINITY;
    }
  };

  f32x16 o[kVTiles];
  constexpr float kMaxExp = 64.0f;
  float m, l, mall;
  bool ovf;

  constexpr int kPf = 2;                     // fragment prefetch distance
  constexpr int kRing = kPf + 2;
  constexpr int kDeq0 = 8;                   // dequantisation: wait + scales, then 5 pieces
  constexpr int kSm0 = 2;                    // softmax slices from this P.V group on

  // Softmax of one step's scores held in acc (lane: head c32, 16 slots),
  // in slices: part 0 scales, biases and takes the maximum, parts 1..8 the
  // weights (2 each), parts 9 and 10 pack P^T for slot chunks 0 and 1
  // (lane (head c32, kg) holds slots 16ch + 4kg + {0..3, 8..11}).
  float m_use = 0.0f;
  auto softmax_part = [&](f32x16& acc, const float* bs, bf16x8 (&pn)[2], int part) {
    if (part == 0) {
      float lmx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 bi = *reinterpret_cast<const float4*>(bs + 8 * j + 4 * kg);
        acc[4 * j] = fmaf(acc[4 * j], p.scale_log2, bi.x);
        acc[4 * j + 1] = fmaf(acc[4 * j + 1], p.scale_log2, bi.y);
        acc[4 * j + 2] = fmaf(acc[4 * j + 2], p.scale_log2, bi.z);
        acc[4 * j + 3] = fmaf(acc[4 * j + 3], p.scale_log2, bi.w);
        lmx = fmaxf(lmx, fmaxf(fmaxf(acc[4 * j], acc[4 * j + 1]),
                               fmaxf(acc[4 * j + 2], acc[4 * j + 3])));
      }
      mall = fmaxf(mall, lmx);
      const float hmx = fmaxf(lmx, __shfl_xor(lmx, 32));   // head c32 in both kg
      m = m == -INFINITY ? hmx : m;                       // first step with a valid slot
      ovf = ovf || lmx > m + kMaxExp;
      m_use = m == -INFINITY ? 0.0f : m;
    } else if (part <= 8) {
      // a score beyond m + kMaxExp sets ovf and the row is run again, so
      // its weight need not be finite
#pragma unroll
      for (int e = 2 * (part - 1); e < 2 * part; ++e) {
        acc[e] = __builtin_amdgcn_exp2f(acc[e] - m_use);
        l += acc[e];
      }
    } else {
      const int ch = part - 9;
      const uint4 u = make_uint4(pack_bf16x2_hw(acc[8 * ch], acc[8 * ch + 1]),
                                 pack_bf16x2_hw(acc[8 * ch + 2], acc[8 * ch + 3]),
                                 pack_bf16x2_hw(acc[8 * ch + 4], acc[8 * ch + 5]),
                                 pack_bf16x2_hw(acc[8 * ch + 6], acc[8 * ch + 7]));
      pn[ch] = *reinterpret_cast<const bf16x8*>(&u);
    }
  };

  // ---- iteration k, two phases of instruction groups (scheduling barriers
  // between groups):
  //   1. the 36 MFMAs of S^T(k) (two accumulator chains) from tile k, with
  //      the loads of step k+2 (groups 0..5) and the dequantisation of step
  //      k+1 into its tile (groups 8..13) between them;
  //   2. the 32 MFMAs of O^T += V^T(k-1).P^T(k-1) from tile k-1 (tile q % 16,
  //      slot chunk q / 16), with the softmax of step k into pn = P(k)
  //      between them (groups 2..12).
  // Fragments are read kPf MFMAs ahead into a ring of kPf + 2 kept live one
  // MFMA longer; only one ring is live at a time.
  auto iter = [&](int k, f32x16& acc, bf16x8 (&pa)[2], bf16x8 (&pn)[2],
                  uint8_t* dma_stage, const uint8_t* deq_stage,
                  const int32_t (&sid)[kDmaInsts], int32_t (&sid_next)[kDmaInsts]) {
    const uint8_t* ktc = ks[k % 3];          // step k: scores
    const uint8_t* ktp = ks[(k + 2) % 3];    // step k-1: P.V
    uint8_t* ktn = ks[(k + 1) % 3];          // step k+1: dequantised now
    const float* bsc = bias[k % 3];
    float* bsn = bias[(k + 1) % 3];
    {
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(ktc + c32 * kKsRow + (16 * i + 8 * kg) * 2);
      };
      bf16x8 fr[kRing];
#pragma unroll
      for (int i = 0; i < kPf; ++i) fr[i] = kfrag(i);
      // two accumulator chains (even and odd contraction steps): a chain of
      // dependent MFMAs issues at half rate
      f32x16 acc2;
#pragma unroll
      for (int e = 0; e < 16; ++e) { acc[e] = 0.0f; acc2[e] = 0.0f; }
      Deq dq;
#pragma unroll
      for (int g = 0; g < kQSteps; ++g) {
        if (g + kPf < kQSteps) fr[(g + kPf) % kRing] = kfrag(g + kPf);
        if (g > 0) asm volatile("" ::"v"(fr[(g - 1) % kRing]));
        __builtin_amdgcn_sched_barrier(0);
        if (g % 2 == 0)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[g % kRing], qb[g], acc, 0, 0, 0);
        else
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[g % kRing], qb[g], acc2, 0, 0, 0);
        // loads of step k+2
        if (g < kDmaInsts) dma_row_id(dma_stage, sid[g], g);
        // dequantisation of step k+1 (its loads were issued one iteration ago)
        if (g == kDeq0) {
          wait_vm_dma();
          deq_load(dq, deq_stage, k + 1);
        } else if (g > kDeq0 && g <= kDeq0 + 5) {
          if (g - kDeq0 < 5) deq_fetch(dq, g - kDeq0);
          deq_store(dq, ktn, bsn, g - kDeq0 - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += acc2[e];
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
        if (q > 0) asm volatile("" ::"v"(vf[(q - 1) % kRing]));
        __builtin_amdgcn_sched_barrier(0);
        // inline asm: the AGPR form of the MFMA for O^T (the 256 AGPRs) while
        // the score MFMAs above use the VGPR form; P (pa) was written by VALU
        // at least one phase earlier, so no wait states are owed here
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(o[q & 15]) : "v"(vf[q % kRing]), "v"(pa[q >> 4]));
        // softmax of step k (its scores were summed after phase 1)
        if (q >= kSm0 && q < kSm0 + 11) softmax_part(acc, bsc, pn, q - kSm0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    read_ids(sid_next, k + 3);   // ids of the next iteration's row loads
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
  auto run_pass = [&]() {
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
      // tile 0, its scores and P taken, step 1 dequantised into tile 1
      dma(r0, 0);
      dma(r1, 1);
      {
        Deq d0;
        wait_vm_dma();
        deq_load(d0, r0, 0);
#pragma unroll
        for (int b = 0; b < 5; ++b) {
          if (b < 4) deq_fetch(d0, b + 1);
          deq_store(d0, ks[0], bias[0], b);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      dma(r0, 2);   // raw buffer 0 (step 0) was read by this wave only
      qk0(acc);
#pragma unroll
      for (int part = 0; part < 11; ++part) softmax_part(acc, bias[0], pA, part);
      {
        Deq d1;
        wait_vm_dma();
        deq_load(d1, r1, 1);
#pragma unroll
        for (int b = 0; b < 5; ++b) {
          if (b < 4) deq_fetch(d1, b + 1);
          deq_store(d1, ks[1], bias[1], b);
        }
      }
      int32_t idA[kDmaInsts], idB[kDmaInsts];
      read_ids(idA, 3);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      // iteration k: scores of step k, P.V of step k-1, loads of k+2,
      // dequantisation of k+1; steps past nsteps are empty (every bias
      // -inf, P zero)
      // (iteration nsteps does the P.V of the last step; its own scores are
      // those of an empty step)
      for (int k = 1; k <= nsteps; k += 2) {
        iter(k, acc, pA, pB, r1, r0, idA, idB);   // loads of k+2 into raw 1, step k+1 from raw 0
        if (k + 1 <= nsteps) iter(k + 1, acc, pB, pA, r0, r1, idB, idA);
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
  run_pass();
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
    run_pass();
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
