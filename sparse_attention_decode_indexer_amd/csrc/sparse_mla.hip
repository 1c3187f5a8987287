// a4 / a5: MLA attention over the selected KV slots of a shared 576-wide
// latent cache (512 no-rope + 64 rope; value = the first 512).
//
// Semantics ("nsa_backend.py (EngineX-Hygon sglang fork)", _forward_fa3 and
// the FlashMLA routes): per query row t and head h, over the valid slots I_t
// of the row's index list (first nsa_cache_seqlens[t] entries, -1 skipped),
//   s_i = sm_scale * q[t,h,:576] . K_i[:576],  o = softmax(s) . K[:, :512],
//   lse = log sum_i exp(s_i).
//
// Three kernels. An fp8 cache with H = 128 (the decode shape of the large
// models) runs the 128-head kernel of sparse_mla_h128.hip: one block per
// (row, KV split), each gathered row dequantized once for all heads, splits
// merged from bf16 partials. An fp8 cache with H = 64 (or shapes the
// 128-head plan does not take) runs the 64-head kernel further below: 32x32
// MFMA tiles, a K tile dequantized once per step for 64 heads,
// software-pipelined steps. Other shapes (16..48 heads, bf16 caches) run the
// narrower kernel:
//
// MI355X design of the narrower kernel (one 256-thread block = 4 waves):
//   * a block owns one query row, HB = 16*NH*HW heads and one KV split; wave
//     w owns NH head tiles of 16 (tile w % HW) and dim slice w / HW of
//     DW = 4 / HW slices (16-head models use all 4 waves by splitting the 576
//     contraction dims in QK and the 512 value dims in PV);
//   * per step, 32 selected slots are gathered with 16-byte loads (issued
//     one step ahead), dequantised to bf16 if the cache is fp8, and staged
//     once in LDS, row-major;
//   * S^T = K.Q^T (v_mfma_f32_16x16x32_bf16, A = 16 slots x 32 dims read
//     from LDS, B = Q^T held in registers) puts one head per lane column, so
//     P is already in the A layout of P.V (heads x slots) and needs no
//     shuffles; each A fragment feeds NH MFMAs;
//   * P.V reads its B operand (8 slots of one value dim per lane) from the
//     same row-major tile with ds_read_b64_tr_b16: within each 16-lane group,
//     source lane s points at 4 dims of slot row s/4 and the hardware
//     transposes, giving lane i dim i of 4 slot rows; each B fragment feeds
//     NH MFMAs;
//   * the online softmax runs in the log2 domain in fp32;
//   * KV splits write (o / l, lse) partials to the workspace and a second
//     kernel merges them in split order (bit-reproducible).
#include "sparse_mla_shared.h"

#include <mutex>

namespace {

using namespace nsa_mla;

constexpr int kThreads = 256;
constexpr int kKSteps = kDQK / 32;        // 18 contraction steps of 32 dims
constexpr float kLazy = 8.0f;             // log2 headroom before O is rescaled





// Prefetch registers of one thread for one step. Loads are branch-free: an
// absent slot (-1) reads slot 0 and its values are zeroed when staged, so no
// load sits behind a branch (a branch around a load makes the compiler wait
// for every load in flight).
template <bool FP8>
struct Stage;

__device__ __forceinline__ uint4 keep_if(bool v, uint4 x) {
  return v ? x : make_uint4(0, 0, 0, 0);
}

// bf16 cache: two (4 slots x 8 dims) pieces of the value part + one rope
// piece of 8 dims.
template <>
struct Stage<false> {
  uint4 v[2][4];
  uint4 rope;
  uint32_t valid;   // bit 4*it+s: slot s of piece it; bit 8: rope slot
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids,
                                       int tid) {
    valid = 0;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + it * kThreads;
      const int qd = item >> 6, ch = item & 63;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int32_t slot = ids[qd * 4 + s];
        valid |= (slot >= 0 ? 1u : 0u) << (4 * it + s);
        v[it][s] = *reinterpret_cast<const uint4*>(
            p.kv + (int64_t)(slot >= 0 ? slot : 0) * (kDQK * 2) + ch * 16);
      }
    }
    const int32_t slot = ids[tid >> 3];
    valid |= (slot >= 0 ? 1u : 0u) << 8;
    rope = *reinterpret_cast<const uint4*>(
        p.kv + (int64_t)(slot >= 0 ? slot : 0) * (kDQK * 2) + kDV * 2 + (tid & 7) * 16);
  }
  __device__ __forceinline__ void store(uint8_t* ks, float*, int tid) const {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + it * kThreads;
      const int qd = item >> 6, ch = item & 63;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(ks + (qd * 4 + s) * kKsRow + ch * 16) =
            keep_if((valid >> (4 * it + s)) & 1u, v[it][s]);
    }
    *reinterpret_cast<uint4*>(ks + (tid >> 3) * kKsRow + kDV * 2 + (tid & 7) * 16) =
        keep_if((valid >> 8) & 1u, rope);
  }
};

// fp8 cache (656-byte rows): one (4 slots x 16 codes) piece with the 4
// block scales + one rope piece of 8 dims.
template <>
struct Stage<true> {
  uint4 code[4];
  float scale[4];
  uint4 rope;
  uint32_t valid;   // bit s: slot s of the piece; bit 4: rope slot
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids,
                                       int tid) {
    const int qd = tid >> 5, cc = tid & 31;
    valid = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int32_t slot = ids[qd * 4 + s];
      valid |= (slot >= 0 ? 1u : 0u) << s;
      const uint8_t* row = p.kv + (int64_t)(slot >= 0 ? slot : 0) * 656;
      code[s] = *reinterpret_cast<const uint4*>(row + cc * 16);
      scale[s] = *reinterpret_cast<const float*>(row + 512 + 4 * (cc >> 3));
    }
    const int32_t slot = ids[tid >> 3];
    valid |= (slot >= 0 ? 1u : 0u) << 4;
    rope = *reinterpret_cast<const uint4*>(p.kv + (int64_t)(slot >= 0 ? slot : 0) * 656 +
                                           528 + (tid & 7) * 16);
  }
  // codes are converted exactly (every e4m3 value is a bf16 value: the fp32
  // image has 16 zero low bits, so the upper halves are taken); the block
  // scales go to LDS and are applied to the scores and to P
  __device__ __forceinline__ void store(uint8_t* ks, float* scl, int tid) const {
    const int qd = tid >> 5, cc = tid & 31;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = (valid >> s) & 1u;
      const uint4 cs = keep_if(ok, code[s]);
      const uint32_t w[4] = {cs.x, cs.y, cs.z, cs.w};
      uint32_t bf[8];  // 16 dims as 8 bf16 pairs
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        bf[2 * i] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
        bf[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
      }
      uint8_t* dst = ks + (qd * 4 + s) * kKsRow + cc * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(bf[0], bf[1], bf[2], bf[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(bf[4], bf[5], bf[6], bf[7]);
      if ((cc & 7) == 0) scl[(qd * 4 + s) * 4 + (cc >> 3)] = ok ? scale[s] : 0.0f;
    }
    *reinterpret_cast<uint4*>(ks + (tid >> 3) * kKsRow + kDV * 2 + (tid & 7) * 16) =
        keep_if((valid >> 4) & 1u, rope);
  }
};

template <int NH, int HW, bool FP8>
__global__ void __launch_bounds__(kThreads, 2)
sparse_mla_kernel(const Params p) {
  constexpr int DW = 4 / HW;                 // dim slices
  constexpr int KSW = (kKSteps + DW - 1) / DW;
  constexpr int NT = kDV / DW / 16;          // value-dim tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t ks[kKsBytes];
  __shared__ float red[DW > 1 ? 4 * 2 * 4 * 64 : 1];   // partial scores
  __shared__ float scl[FP8 ? kStep * 4 : 1];            // block scales of the step
  __shared__ int32_t ids[4][kStep];     // ring: slot ids of steps s..s+3
  __shared__ uint32_t vmask[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hw = wave % HW, dw = wave / HW;

  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int hb = lb % p.n_hb;
  const int split = (lb / p.n_hb) % p.n_splits;
  const int64_t t = lb / (p.n_hb * p.n_splits);
  const int h0 = hb * (16 * NH * HW) + hw * (16 * NH);   // first head of this wave

  int n_row = p.num_slots > 0 ? p.topk : 0;   // no cache rows: every row is empty
  if (p.seqlens) {
    const int sl = p.seqlens[t];
    n_row = sl < 0 ? 0 : (sl < n_row ? sl : n_row);
  }
  const int s_begin = split * p.split_slots;
  const int s_end = min(s_begin + p.split_slots, n_row);
  const int nsteps = s_end > s_begin ? (s_end - s_begin + kStep - 1) / kStep : 0;
  const int32_t* irow = p.idx + t * p.idx_stride;

  // Q as the B operand of S^T = K.Q^T: lane (head c of tile nh, group g)
  // holds dims ks*32 + 8g .. +8 for the wave's contraction steps
  bf16x8 qb[NH][KSW];
#pragma unroll
  for (int nh = 0; nh < NH; ++nh) {
    const uint16_t* qh = p.q + t * p.q_tok_stride +
                         (int64_t)(h0 + nh * 16 + c) * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int kstep = dw + DW * i;
      if (kstep < kKSteps)
        qb[nh][i] = *reinterpret_cast<const bf16x8*>(qh + kstep * 32 + g * 8);
    }
  }

  // Slot ids are loaded a few steps ahead and only checked when published:
  // using a loaded value right away would make the wave wait for every
  // memory load in flight, including the gather of the next steps.
  auto load_ids = [&](int step) -> int32_t {
    // thread j < 32: raw id of slot j of `step` (-1 past the row's end)
    const int pos = s_begin + step * kStep + tid;
    const bool in = tid < kStep && step < nsteps && pos < s_end;
    const int32_t id = irow[in ? pos : s_begin];
    return in ? id : -1;
  };
  auto publish_ids = [&](int buf, int32_t id) {
    if (id < -1 || id >= p.num_slots) flag_device_error(NSA_DEVERR_SLOT);
    if (id < 0 || id >= p.num_slots) id = -1;
    if (tid < kStep) ids[buf][tid] = id;
    if (wave == 0) {
      const unsigned long long b = __ballot(tid < kStep && id >= 0);
      if (lane == 0) vmask[buf] = (uint32_t)b;
    }
  };

  f32x4 o[NH][NT];
#pragma unroll
  for (int nh = 0; nh < NH; ++nh)
#pragma unroll
    for (int i = 0; i < NT; ++i) o[nh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m: reference max (log2 domain) of each head, raised only when a step's
  // max exceeds it by more than kLazy, so O is rarely rescaled
  float m[NH], l[NH];
#pragma unroll
  for (int nh = 0; nh < NH; ++nh) { m[nh] = -INFINITY; l[nh] = 0.0f; }

  // the rows of step i+1 are loaded while step i is computed
  Stage<FP8> sa;
  if (nsteps > 0) {
    publish_ids(0, load_ids(0));
    publish_ids(1, load_ids(1));
    publish_ids(2, load_ids(2));
    __syncthreads();
    sa.load(p, ids[0], tid);
    sa.store(ks, scl, tid);

    __syncthreads();
  }
  int32_t id_ahead = load_ids(3);

  auto run_step = [&](int step) {
    const int buf = step & 3;
    Stage<FP8> nx;
    if (step + 1 < nsteps) nx.load(p, ids[(step + 1) & 3], tid);

    // ---- S^T = K . Q^T (partial over this wave's contraction steps). For an
    // fp8 cache each 128-dim block is accumulated apart and scaled by its
    // slot's block scale; rope dims are unscaled.
    f32x4 acc[2][NH], tmp[2][NH];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nh = 0; nh < NH; ++nh) {
        acc[mt][nh] = f32x4{0.f, 0.f, 0.f, 0.f};
        tmp[mt][nh] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int kstep = dw + DW * i;
      if (kstep < kKSteps) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              ks + (mt * 16 + c) * kKsRow + (kstep * 32 + g * 8) * 2);
#pragma unroll
          for (int nh = 0; nh < NH; ++nh)
            tmp[mt][nh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[nh][i], tmp[mt][nh], 0, 0, 0);
        }
        if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        const int blk = kstep < 16 ? kstep >> 2 : 4;
        const int nk = kstep + DW;
        const int nblk = nk < kKSteps ? (nk < 16 ? nk >> 2 : 4) : -1;
        if (nblk != blk) {   // flush the block's partial scores
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float sc = 1.0f;
              if constexpr (FP8) {
                if (blk < 4) sc = scl[(mt * 16 + 4 * g + r) * 4 + blk];
              }
#pragma unroll
              for (int nh = 0; nh < NH; ++nh) {
                acc[mt][nh][r] = fmaf(sc, tmp[mt][nh][r], acc[mt][nh][r]);
                tmp[mt][nh][r] = 0.0f;
              }
            }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DW > 1) {
      // sum the DW partial scores of this head tile, in slice order
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * 2 + mt) * 4 + r) * 64 + lane] = acc[mt][0][r];
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = 0.0f;
#pragma unroll
          for (int j = 0; j < DW; ++j)
            sum += red[(((j * HW + hw) * 2 + mt) * 4 + r) * 64 + lane];
          acc[mt][0][r] = sum;
        }
    }

    // ---- online softmax with a lazily raised reference max: lane (head c,
    // group g) holds slots mt*16+4g+r. In the common step no lane crosses
    // its head's reference max by more than kLazy, nothing is exchanged
    // between lanes and O keeps its scale; l is kept per lane and summed
    // across the head's lanes at the end.
    const uint32_t valid = vmask[buf];
    float pv[NH][2][4];
    float al[NH][4];
    bool need = false;
    float lmx[NH];
#pragma unroll
    for (int nh = 0; nh < NH; ++nh) {
      lmx[nh] = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = mt * 16 + 4 * g + r;
          pv[nh][mt][r] = ((valid >> j) & 1u) ? acc[mt][nh][r] * p.scale_log2 : -INFINITY;
          lmx[nh] = fmaxf(lmx[nh], pv[nh][mt][r]);
        }
      need = need || lmx[nh] > m[nh] + kLazy;
#pragma unroll
      for (int r = 0; r < 4; ++r) al[nh][r] = 1.0f;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // rare: agree on each head's new reference max and rescale
#pragma unroll
      for (int nh = 0; nh < NH; ++nh) {
        float mx = lmx[nh];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool upd = mx > m[nh] + kLazy;   // same in the head's 4 lanes
        const float alpha = upd ? exp2f(m[nh] - mx) : 1.0f;   // m = -inf -> 0
        if (upd) m[nh] = mx;
        l[nh] *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) al[nh][r] = __shfl(alpha, 4 * g + r);
      }
    }
#pragma unroll
    for (int nh = 0; nh < NH; ++nh) {
      const float m_use = m[nh] == -INFINITY ? 0.0f : m[nh];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[nh][mt][r] = exp2f(pv[nh][mt][r] - m_use);
          l[nh] += pv[nh][mt][r];
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nh][nt][r] *= al[nh][r];
    }

    // ---- P . V: the B operand (slots 4g..4g+3 and 16+4g..16+4g+3 of value
    // dim `dim`) comes from two transposing reads of the row-major tile; for
    // an fp8 cache P carries the slot's scale of the value dims' block
    bf16x8 pa[NH];
    int pa_blk = -1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n0 = dw * (kDV / DW) + nt * 16;
      const int blk = n0 >> 7;
      if (blk != pa_blk) {
        pa_blk = blk;
#pragma unroll
        for (int nh = 0; nh < NH; ++nh) {
          uint32_t pw[4];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            float q4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float sc = 1.0f;
              if constexpr (FP8) sc = scl[(mt * 16 + 4 * g + r) * 4 + blk];
              q4[r] = pv[nh][mt][r] * sc;
            }
            pw[mt * 2] = pack_bf16x2(q4[0], q4[1]);
            pw[mt * 2 + 1] = pack_bf16x2(q4[2], q4[3]);
          }
          const uint4 u = make_uint4(pw[0], pw[1], pw[2], pw[3]);
          pa[nh] = *reinterpret_cast<const bf16x8*>(&u);
        }
      }
      const uint8_t* src = ks + (4 * g + (c >> 2)) * kKsRow + (n0 + 4 * (c & 3)) * 2;
      const v4i16 b0 = read_tr(src);
      const v4i16 b1 = read_tr(src + 16 * kKsRow);
      const v4i16 bb[2] = {b0, b1};
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(bb);
#pragma unroll
      for (int nh = 0; nh < NH; ++nh)
        o[nh][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[nh], b, o[nh][nt], 0, 0, 0);
      if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }

    // ---- stage step + 1 (its rows were issued a step ago)
    __syncthreads();  // all waves are done with ks / ids[buf]
    if (step + 1 < nsteps) nx.store(ks, scl, tid);
    publish_ids((step + 3) & 3, id_ahead);
    id_ahead = load_ids(step + 4);
    __syncthreads();
  };

  for (int step = 0; step < nsteps; ++step) run_step(step);

  // ---- finalize: lane (dim c of tile nt, group g) holds O[head 4g+r][dim]
#pragma unroll
  for (int nh = 0; nh < NH; ++nh) {
    l[nh] += __shfl_xor(l[nh], 16);
    l[nh] += __shfl_xor(l[nh], 32);
    float lr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lr[r] = __shfl(l[nh], 4 * g + r);
    const float lse_val = l[nh] > 0.0f ? (m[nh] + __log2f(l[nh])) * kLn2 : -INFINITY;
    const int hbase = h0 + nh * 16;
    if (p.n_splits == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int dim = dw * (kDV / DW) + nt * 16 + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = lr[r] > 0.0f ? o[nh][nt][r] / lr[r] : 0.0f;
          p.out[(t * p.H + hbase + 4 * g + r) * kDV + dim] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
      if (p.lse && dw == 0 && g == 0) p.lse[t * p.H + hbase + c] = lse_val;
    } else {
      const int64_t base = ((int64_t)split * p.T + t) * p.H;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int dim = dw * (kDV / DW) + nt * 16 + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = lr[r] > 0.0f ? o[nh][nt][r] / lr[r] : 0.0f;
          p.ws_o[(base + hbase + 4 * g + r) * kDV + dim] = v;
        }
      }
      if (dw == 0 && g == 0) p.ws_lse[base + hbase + c] = lse_val;
    }
  }
}

// ---- 64 heads per block (H a multiple of 64, fp8 cache) --------------------
// On gfx950 v_mfma_f32_32x32x16_bf16 runs at twice the rate of
// v_mfma_f32_16x16x32_bf16 (measured), and a 32x32 tile also halves the LDS
// fragment reads per flop, so this kernel works in 32x32 tiles.
// One 256-thread block (4 waves, one per SIMD) per (row, 64 heads, KV
// split), one block per CU. Wave (hg = w % 2, dw = w / 2) owns heads
// 32*hg.. of the block and half dw of the work: S over contraction dims
// 256dw..+256 and rope dims 512+32dw..+32 (18 steps of 16), O over value dims
// 256dw..+256. The two halves of a head group's scores meet in LDS and are
// added in the same order in both waves, so both run an identical softmax.
// The gathered fp8 rows are dequantized to bf16 once per step (code times
// block scale, rounded to nearest even) into a K tile that all four waves
// read. The split's slot ids are loaded into LDS once; absent slots get a
// -inf score bias written with the tile.
// The steps are software-pipelined with one barrier per step: iteration k
// stages the gathered rows of step k+1, computes the partial scores of step
// k and runs softmax and P.V of step k-1 (three K tiles, two score-exchange
// buffers). The gather of step k+3 is issued in iteration k from two
// register stages that alternate (the loop is unrolled by two, so no
// register copy waits on a load in flight).
constexpr int kThreadsW = 256;
constexpr int kIdsCap = 10 * kThreadsW;        // 2560 >= kMaxSplit + 5 steps of overrun


// Gather registers of one thread for one step: slot qd = tid / 8, 16-byte
// code chunks cc + 8k (k = 0..3, chunk k lies in 128-block k), the slot's 4
// block scales and 16 bytes of its rope part.
struct StageF8 {
  uint4 code[4];
  float4 scale;
  uint4 rope;
  bool valid;
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids, int tid) {
    const int qd = tid >> 3, cc = tid & 7;
    const int32_t slot = ids[qd];
    valid = slot >= 0;
    const uint8_t* row = p.kv + (int64_t)(slot >= 0 ? slot : 0) * 656;
#pragma unroll
    for (int k = 0; k < 4; ++k) code[k] = *reinterpret_cast<const uint4*>(row + 16 * (cc + 8 * k));
    scale = *reinterpret_cast<const float4*>(row + 512);
    rope = *reinterpret_cast<const uint4*>(row + 528 + 16 * cc);
  }
  // Staging in five parts (so it can be spread between MFMAs): part k < 4
  // writes bf16(code * scale) of 128-block k, part 4 the rope dims and the
  // score bias. An absent slot stores zeros (scale 0) and a -inf bias.
  __device__ __forceinline__ void store_part(uint8_t* kt, float* bias, int tid, int part) const {
    const int qd = tid >> 3, cc = tid & 7;
    if (part < 4) {
      const float sk = part == 0 ? scale.x : part == 1 ? scale.y : part == 2 ? scale.z : scale.w;
      const float s = valid ? sk : 0.0f;
      const uint32_t w[4] = {code[part].x, code[part].y, code[part].z, code[part].w};
      uint32_t bf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        bf[2 * i] = pack_bf16x2_hw(lo[0] * s, lo[1] * s);
        bf[2 * i + 1] = pack_bf16x2_hw(hi[0] * s, hi[1] * s);
      }
      uint8_t* dst = kt + qd * kKsRow + 32 * (cc + 8 * part);
      *reinterpret_cast<uint4*>(dst) = make_uint4(bf[0], bf[1], bf[2], bf[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(bf[4], bf[5], bf[6], bf[7]);
    } else {
      const uint32_t msk = valid ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<uint4*>(kt + qd * kKsRow + kDV * 2 + 16 * cc) =
          make_uint4(rope.x & msk, rope.y & msk, rope.z & msk, rope.w & msk);
      bias[qd] = valid ? 0.0f : -INFINITY;   // the slot's 8 lanes write the same value
    }
  }
  __device__ __forceinline__ void store(uint8_t* kt, float* bias, int tid) const {
#pragma unroll
    for (int part = 0; part < 5; ++part) store_part(kt, bias, tid, part);
  }
  // Finer staging pieces: piece h < 8 writes 8 codes (half of 128-block
  // h / 2) as 16 bytes of bf16, piece 8 the rope dims and the score bias.
  __device__ __forceinline__ void store_piece(uint8_t* kt, float* bias, int tid, int h) const {
    const int qd = tid >> 3, cc = tid & 7;
    if (h < 8) {
      const int part = h >> 1, half = h & 1;
      const float sk = part == 0 ? scale.x : part == 1 ? scale.y : part == 2 ? scale.z : scale.w;
      const float s = valid ? sk : 0.0f;
      const uint32_t w0 = half == 0 ? code[part].x : code[part].z;
      const uint32_t w1 = half == 0 ? code[part].y : code[part].w;
      uint32_t bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wi = i == 0 ? w0 : w1;
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, true);
        bf[2 * i] = pack_bf16x2_hw(lo[0] * s, lo[1] * s);
        bf[2 * i + 1] = pack_bf16x2_hw(hi[0] * s, hi[1] * s);
      }
      *reinterpret_cast<uint4*>(kt + qd * kKsRow + 32 * (cc + 8 * part) + 16 * half) =
          make_uint4(bf[0], bf[1], bf[2], bf[3]);
    } else {
      store_part(kt, bias, tid, 4);
    }
  }
};

__global__ void __launch_bounds__(kThreadsW, 1)
sparse_mla_h64_kernel(const Params p) {
  constexpr int KS = 18;                     // contraction steps of 16 per wave
  constexpr int ND = 8;                      // value tiles of 32 dims per wave
  __shared__ __attribute__((aligned(16))) uint8_t ks[3][kKsBytes];
  __shared__ __attribute__((aligned(16))) float bias[3][kStep];
  __shared__ int32_t ids[kIdsCap];
  __shared__ __attribute__((aligned(16))) float xch[2][4][4][64][4];   // partial S per wave
  __shared__ int s_ovf;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, kg = lane >> 5;
  const int hg = wave & 1, dw = wave >> 1;

  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int hb = lb % p.n_hb;
  const int split = (lb / p.n_hb) % p.n_splits;
  const int64_t t = lb / (p.n_hb * p.n_splits);
  const int h0 = hb * 64 + hg * 32;          // first head of this wave

  int n_row = p.num_slots > 0 ? p.topk : 0;
  if (p.seqlens) {
    const int sl = p.seqlens[t];
    n_row = sl < 0 ? 0 : (sl < n_row ? sl : n_row);
  }
  const int s_begin = split * p.split_slots;
  const int n = min(s_begin + p.split_slots, n_row) - s_begin;   // may be <= 0
  const int nsteps = n > 0 ? (n + kStep - 1) / kStep : 0;

  // ---- slot ids of the split (validated; -1 past its end)
  {
    const int32_t* irow = p.idx + t * p.idx_stride + s_begin;
    const int last = n > 0 ? n - 1 : 0;
    int32_t v[kIdsCap / kThreadsW];
#pragma unroll
    for (int k = 0; k < kIdsCap / kThreadsW; ++k) v[k] = irow[min(tid + k * kThreadsW, last)];
#pragma unroll
    for (int k = 0; k < kIdsCap / kThreadsW; ++k) {
      const int i = tid + k * kThreadsW;
      const int32_t id = v[k];
      if (i < n && (id < -1 || id >= p.num_slots)) flag_device_error(NSA_DEVERR_SLOT);
      ids[i] = (i < n && id >= 0 && id < p.num_slots) ? id : -1;
    }
  }

  // Q as the B operand of S^T = K.Q^T: lane (head c32, group kg) holds dims
  // 16*kstep + 8kg .. +8 of the wave's 18 steps
  auto kstep_of = [&](int i) { return i < 16 ? dw * 16 + i : 32 + 2 * dw + (i - 16); };
  bf16x8 qb[KS];
  {
    const uint16_t* qh = p.q + t * p.q_tok_stride + (int64_t)(h0 + c32) * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      qb[i] = *reinterpret_cast<const bf16x8*>(qh + kstep_of(i) * 16 + kg * 8);
      asm volatile("" : "+a"(qb[i]));   // Q lives in AGPRs (MFMA reads it there)
    }
  }

  f32x16 o[ND];
  // Softmax without rescaling O: the reference max m of a head is fixed at
  // the first step with a valid slot (O and l are zero until then), and
  // exponents are clamped at kMaxExp, which fp32 O and l absorb (|O| stays
  // far below the fp32 range). A score beyond m + kMaxExp sets `ovf` and the
  // split is run again with m = the true maximum mall (no score exceeds it).
  constexpr float kMaxExp = 64.0f;
  float m, l, mall;
  bool ovf;

  // ---- one pipelined iteration k as explicit instruction groups (separated
  // by scheduling barriers). Group g holds: the MFMA of contraction step g of
  // the partial S^T(k) (g < 18; one accumulator chain, consecutive chain
  // MFMAs separated by other work), the MFMA q = g - 6 of O += P(k-1).V
  // (6 <= g < 22; q = ch * ND + d, so consecutive ones update different value
  // tiles), and a slice of VALU work: the softmax of step k-1 in groups 0..5
  // (P is needed from group 6 on), the staging of step k+1 in groups 6..14,
  // the exchange write of S^T(k) in groups 18..21 and the gather of step k+3
  // in group 21. A wave issues in order and its VALU only partly overlaps its
  // MFMAs, so the slices are kept short. Fragments are read kPf MFMAs ahead
  // into rings of kPf + 2, and a fragment is kept live one MFMA longer, so a
  // read never overwrites the operand of the MFMA just issued. Lane
  // (head c32, kg) element e of S^T holds slot 8(e/4) + 4kg + e%4; O element
  // e of value tile d holds head 8(e/4) + 4kg + e%4 at dim d*32 + c32 of the
  // wave's half.
  constexpr int kPf = 2;                     // fragment prefetch distance
  constexpr int kRing = kPf + 2;
  constexpr int kPv0 = 6;                    // first group with a P.V MFMA
  constexpr int kGroups = kPv0 + 2 * ND;     // 22
  const int grp = lane >> 4, sl = lane & 15;
  auto iter = [&](int k, StageF8& st, int xp, int xc) {
    const uint8_t* ktc = ks[k % 3];          // step k: scores
    const uint8_t* ktp = ks[(k + 2) % 3];    // step k-1: softmax and P.V
    uint8_t* ktn = ks[(k + 1) % 3];          // step k+1: staged now
    const float* bsp = bias[(k + 2) % 3];
    float* bsn = bias[(k + 1) % 3];
    auto kfrag = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(ktc + c32 * kKsRow + (kstep_of(i) * 16 + kg * 8) * 2);
    };
    // V as the B operand: lane (dim, kg) needs the same slots of one value
    // dim; two transposing reads of 4 slot rows each. In each 16-lane group
    // (kg = group / 2, dims 16*(group % 2)..), source lane s points at slot
    // row base + s/4 and dims +4(s%4).
    const uint8_t* vbase = ktp + (4 * kg + (sl >> 2)) * kKsRow +
                           (dw * 256 + 16 * (grp & 1) + 4 * (sl & 3)) * 2;
    auto vfrag = [&](int q) {
      const uint8_t* src = vbase + 16 * (q / ND) * kKsRow + (q % ND) * 64;
      const v4i16 b0 = read_tr(src);
      const v4i16 b1 = read_tr(src + 8 * kKsRow);
      const v4i16 bb[2] = {b0, b1};
      return *reinterpret_cast<const bf16x8*>(bb);
    };
    // exchanged partial scores of step k-1 and the slot bias
    float4 xa[4], xb[4], bi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xa[j] = *reinterpret_cast<const float4*>(&xch[xp][wave][j][lane][0]);
      xb[j] = *reinterpret_cast<const float4*>(&xch[xp][wave ^ 2][j][lane][0]);
      bi[j] = *reinterpret_cast<const float4*>(bsp + 8 * j + 4 * kg);
    }
    bf16x8 fr[kRing], vf[kRing];
#pragma unroll
    for (int i = 0; i < kPf; ++i) { fr[i] = kfrag(i); vf[i] = vfrag(i); }
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    float sc[16];
    float lmx = -INFINITY, m_use = 0.0f;
    bf16x8 pa[2];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g < KS) {
        if (g + kPf < KS) fr[(g + kPf) % kRing] = kfrag(g + kPf);
        if (g > 0) asm volatile("" ::"v"(fr[(g - 1) % kRing]));
      }
      const int q = g - kPv0;
      if (q >= 0) {
        if (q + kPf < 2 * ND) vf[(q + kPf) % kRing] = vfrag(q + kPf);
        if (q > 0) asm volatile("" ::"v"(vf[(q - 1) % kRing]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (g < KS) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[g % kRing], qb[g], acc, 0, 0, 0);
      if (q >= 0)
        o[q % ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[q / ND], vf[q % kRing], o[q % ND], 0, 0, 0);
      if (g < 2) {
        // full scores of step k-1, 8 per group: own half + partner half
        // (a + b == b + a, so both waves of the pair hold identical scores),
        // scaled, plus the bias
#pragma unroll
        for (int j = 2 * g; j < 2 * g + 2; ++j) {
          sc[4 * j] = fmaf(xa[j].x + xb[j].x, p.scale_log2, bi[j].x);
          sc[4 * j + 1] = fmaf(xa[j].y + xb[j].y, p.scale_log2, bi[j].y);
          sc[4 * j + 2] = fmaf(xa[j].z + xb[j].z, p.scale_log2, bi[j].z);
          sc[4 * j + 3] = fmaf(xa[j].w + xb[j].w, p.scale_log2, bi[j].w);
          lmx = fmaxf(lmx, fmaxf(fmaxf(sc[4 * j], sc[4 * j + 1]), fmaxf(sc[4 * j + 2], sc[4 * j + 3])));
        }
        if (g == 1) {
          mall = fmaxf(mall, lmx);
          const float hmx = fmaxf(lmx, __shfl_xor(lmx, 32));   // head c32 in both kg
          m = m == -INFINITY ? hmx : m;                       // first step with a valid slot
          ovf = ovf || lmx > m + kMaxExp;
          m_use = m == -INFINITY ? 0.0f : m;
        }
      } else if (g < kPv0) {
        // weights, 4 per group (a score beyond m + kMaxExp sets ovf and the
        // pass is repeated, so its weight need not be finite)
#pragma unroll
        for (int e = 4 * (g - 2); e < 4 * (g - 1); ++e) {
          sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
          l += sc[e];
        }
        if (g == kPv0 - 1) {
          // P as the A operand for slot chunk ch (slots 16ch..16ch+15): lane
          // (head c32, kg) holds slots 16ch + 4kg + {0..3, 8..11}
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const uint4 u = make_uint4(pack_bf16x2_hw(sc[8 * ch], sc[8 * ch + 1]),
                                       pack_bf16x2_hw(sc[8 * ch + 2], sc[8 * ch + 3]),
                                       pack_bf16x2_hw(sc[8 * ch + 4], sc[8 * ch + 5]),
                                       pack_bf16x2_hw(sc[8 * ch + 6], sc[8 * ch + 7]));
            pa[ch] = *reinterpret_cast<const bf16x8*>(&u);
          }
        }
      } else if (g < kPv0 + 9) {
        st.store_piece(ktn, bsn, tid, g - kPv0);
      } else if (g >= KS) {
        // exchange slice of S^T(k), one float4 per group
        const int j = g - KS;
        *reinterpret_cast<float4*>(&xch[xc][wave][j][lane][0]) =
            make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
        if (g == kGroups - 1) st.load(p, ids + (k + 3) * kStep, tid);   // gather of step k+3
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  // partial scores of step 0 (prologue)
  auto qk0 = [&]() {
    f32x16 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const bf16x8 f = *reinterpret_cast<const bf16x8*>(ks[0] + c32 * kKsRow + (kstep_of(i) * 16 + kg * 8) * 2);
      acc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qb[i], acc[i & 1], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&xch[0][wave][j][lane][0]) =
          make_float4(acc[0][4 * j] + acc[1][4 * j], acc[0][4 * j + 1] + acc[1][4 * j + 1],
                      acc[0][4 * j + 2] + acc[1][4 * j + 2], acc[0][4 * j + 3] + acc[1][4 * j + 3]);
  };
  auto run_pass = [&]() {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
    l = 0.0f;
    if (nsteps > 0) {
      StageF8 sa, sb;
      sa.load(p, ids, tid);
      sb.load(p, ids + kStep, tid);
      sa.store(ks[0], bias[0], tid);
      sa.load(p, ids + 2 * kStep, tid);
      sb.store(ks[1], bias[1], tid);
      sb.load(p, ids + 3 * kStep, tid);
      __syncthreads();
      qk0();
      __syncthreads();
      // steps past nsteps are empty (every bias is -inf): their P is zero
      for (int k = 1; k <= nsteps; k += 2) {
        iter(k, sa, 0, 1);
        iter(k + 1, sb, 1, 0);
      }
    }
  };

  __syncthreads();   // ids
  m = -INFINITY;
  mall = -INFINITY;
  ovf = false;
  run_pass();
  // a score beyond the clamp anywhere in the block: run again with the true
  // maximum as reference (both waves of a head group agree on m and mall)
  if (tid == 0) s_ovf = 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(ovf) != 0 && lane == 0) s_ovf = 1;
  __syncthreads();
  if (s_ovf != 0) {
    m = fmaxf(mall, __shfl_xor(mall, 32));
    ovf = false;
    __syncthreads();
    run_pass();
  }

  // ---- finalize: lane (dim c32 of tile d, group kg) element e holds
  // O[head 8(e/4) + 4kg + e%4][dim]
  l += __shfl_xor(l, 32);
  const float lse_val = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  const int d0 = dw * 256;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int hr = 8 * (e >> 2) + 4 * kg + (e & 3);
    const float lr = __shfl(l, hr);
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    if (p.n_splits == 1) {
      uint16_t* orow = p.out + (t * p.H + h0 + hr) * kDV + d0 + c32;
#pragma unroll
      for (int d = 0; d < ND; ++d) orow[d * 32] = (uint16_t)f32_to_bf16_bits(o[d][e] * inv);
    } else {
      float* orow = p.ws_o + (((int64_t)split * p.T + t) * p.H + h0 + hr) * kDV + d0 + c32;
#pragma unroll
      for (int d = 0; d < ND; ++d) orow[d * 32] = o[d][e] * inv;
    }
  }
  if (dw == 0 && kg == 0) {
    if (p.n_splits == 1) {
      if (p.lse) p.lse[t * p.H + h0 + c32] = lse_val;
    } else {
      p.ws_lse[((int64_t)split * p.T + t) * p.H + h0 + c32] = lse_val;
    }
  }
}

// Merge of KV-split partials, in split order: one wave per (row, head). PT:
// float rows (the 16..64-head kernels) or bf16 rows (the 128-head kernel).
template <typename PT>
__global__ void __launch_bounds__(256)
combine_splits_kernel(const PT* __restrict__ ws_o,
                      const float* __restrict__ ws_lse, int T, int H,
                      int n_splits, uint16_t* __restrict__ out,
                      float* __restrict__ lse) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= (int64_t)T * H) return;
  const int lane = threadIdx.x & 63;
  const int64_t TH = (int64_t)T * H;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ws_lse[s * TH + th]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float den = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float ls = ws_lse[s * TH + th];
      const float wgt = ls == -INFINITY ? 0.0f : __expf(ls - mx);
      den += wgt;
      float4 a, b;
      if constexpr (sizeof(PT) == 4) {
        const float4* src = reinterpret_cast<const float4*>(ws_o + (s * TH + th) * kDV + lane * 8);
        a = src[0]; b = src[1];
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(ws_o + (s * TH + th) * kDV + lane * 8);
        a = make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                        bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
        b = make_float4(bf16_bits_to_f32(u.z & 0xFFFFu), bf16_bits_to_f32(u.z >> 16),
                        bf16_bits_to_f32(u.w & 0xFFFFu), bf16_bits_to_f32(u.w >> 16));
      }
      acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
      acc[4] += wgt * b.x; acc[5] += wgt * b.y; acc[6] += wgt * b.z; acc[7] += wgt * b.w;
    }
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = den > 0.0f ? acc[2 * i] / den : 0.0f;
    const float x1 = den > 0.0f ? acc[2 * i + 1] / den : 0.0f;
    w[i] = pack_bf16x2(x0, x1);
  }
  *reinterpret_cast<uint4*>(out + th * kDV + lane * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  if (lse && lane == 0) lse[th] = den > 0.0f ? mx + __logf(den) : -INFINITY;
}

// Merge of the 128-head kernel's KV-split partials (bf16 rows o_s / l_s and
// lse_s), NS splits known at compile time so that every load of a (row,
// head) is issued before any is used; in split order as above.
template <int NS>
__global__ void __launch_bounds__(256)
combine_bf16_kernel(const uint16_t* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    int T, int H, uint16_t* __restrict__ out, float* __restrict__ lse) {
  // (row, head) pairs in XCD-contiguous order: the attention blocks of a
  // row (and their partials, still in that XCD's L2) run on the same XCD
  const int64_t th = (int64_t)xcd_logical_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (th >= (int64_t)T * H) return;
  const int lane = threadIdx.x & 63;
  const int64_t TH = (int64_t)T * H;
  float ls[NS];
  uint4 u[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ls[s] = ws_lse[s * TH + th];
    u[s] = *reinterpret_cast<const uint4*>(ws_o + (s * TH + th) * kDV + lane * 8);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) mx = fmaxf(mx, ls[s]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float den = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = (mx == -INFINITY || ls[s] == -INFINITY) ? 0.0f : __expf(ls[s] - mx);
    den += wgt;
    const uint32_t w[4] = {u[s].x, u[s].y, u[s].z, u[s].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += wgt * bf16_bits_to_f32(w[i] & 0xFFFFu);
      acc[2 * i + 1] += wgt * bf16_bits_to_f32(w[i] >> 16);
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<uint4*>(out + th * kDV + lane * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  if (lse && lane == 0) lse[th] = den > 0.0f ? mx + __logf(den) : -INFINITY;
}

struct Plan {
  bool h128;   // all 128 heads per block (sparse_mla_h128_kernel)
  bool wide;   // 64 heads per block (sparse_mla_h64_kernel)
  int nh, hw, hb_heads, n_hb, n_splits, split_slots;
};

// Heads per block and KV splits: the 64-head kernel (fp8 caches) runs one
// block per CU, so it aims at 256 blocks (one per CU) and at most kMaxSplit
// slots per block; the narrower kernel runs two blocks per CU.
Plan make_plan(int T, int H, int topk, bool decode, bool fp8) {
  Plan pl;
  // 128 heads over an fp8 cache: the 128-head kernel does more work per
  // second than two 64-head blocks per row (each gathered row is dequantised
  // once for all heads). More than 128 rows fill the CUs with one block per
  // row; fewer rows are split over KV (about 256 blocks, at least 128 slots
  // per split, at most kMaxSplit) and merged by combine_bf16_kernel. Shapes
  // it cannot split that way (tiny topk, topk > 2 kMaxSplit) take the
  // 64-head kernel.
  pl.h128 = fp8 && H == 128 && topk <= 2 * kMaxSplit;
  if (pl.h128) {
    pl.wide = false; pl.nh = 1; pl.hw = 1; pl.hb_heads = 128; pl.n_hb = 1;
    int ns = T > 128 ? 1 : (int)((256 + T - 1) / T);
    const int mx = (topk + 127) / 128;
    ns = ns > mx ? mx : ns;
    int ss = (topk + ns - 1) / ns;
    ss = (ss + kStep - 1) / kStep * kStep;
    ns = (topk + ss - 1) / ss;
    if (ss <= kMaxSplit && (T > 128 || ns > 1)) {
      pl.n_splits = ns; pl.split_slots = ss;
      return pl;
    }
    pl.h128 = false;
  }
  pl.wide = fp8 && H % 64 == 0;
  if (pl.wide) { pl.nh = 1; pl.hw = 4; }
  else if (H % 32 == 0) { pl.nh = 1; pl.hw = 2; }
  else { pl.nh = 1; pl.hw = 1; }
  pl.hb_heads = 16 * pl.nh * pl.hw;
  pl.n_hb = H / pl.hb_heads;
  const int64_t base = (int64_t)T * pl.n_hb;
  const int max_splits = (topk + 127) / 128;   // >= 128 slots per split
  const int min_splits = pl.wide ? (topk + kMaxSplit - 1) / kMaxSplit : 1;
  int ns = 1;
  const int64_t target = (pl.wide || decode) ? 256 : 128;
  if (base < target) ns = (int)((target + base - 1) / base);
  ns = ns < 1 ? 1 : (ns > max_splits ? max_splits : ns);
  ns = ns < min_splits ? min_splits : ns;
  int ss = (topk + ns - 1) / ns;
  ss = (ss + kStep - 1) / kStep * kStep;
  ns = (topk + ss - 1) / ss;
  pl.n_splits = ns;
  pl.split_slots = ss;
  return pl;
}

size_t workspace_bytes(const Plan& pl, int T, int H) {
  if (pl.n_splits <= 1) return 0;
  if (pl.h128)   // bf16 partials + fp32 lse
    return (size_t)pl.n_splits * T * H * (kDV * sizeof(uint16_t) + sizeof(float));
  return (size_t)pl.n_splits * T * H * (kDV + 1) * sizeof(float);
}

int check_args(const char* fn, const void* q, int64_t q_tok_stride,
               int64_t q_head_stride, const void* kv, int kv_dtype,
               int64_t num_slots, const int32_t* idx, int64_t idx_stride,
               int T, int H, int topk, int d_qk, int d_v, const void* out) {
  NSA_REQUIRE(T >= 0 && H > 0 && topk > 0 && num_slots >= 0,
              NSA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  NSA_REQUIRE(d_qk == kDQK && d_v == kDV, NSA_ERR_UNSUPPORTED,
              "%s: d_qk %d / d_v %d (576 / 512 only)", fn, d_qk, d_v);
  NSA_REQUIRE(H % 16 == 0 && H <= 128, NSA_ERR_UNSUPPORTED,
              "%s: H %d (multiple of 16, at most 128)", fn, H);
  NSA_REQUIRE(topk <= 8192, NSA_ERR_UNSUPPORTED, "%s: topk %d > 8192", fn, topk);
  NSA_REQUIRE(kv_dtype == NSA_KV_BF16_576 || kv_dtype == NSA_KV_FP8_656,
              NSA_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  if (T == 0) return NSA_OK;
  NSA_REQUIRE(q && kv && idx && out, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(idx_stride >= topk, NSA_ERR_INVALID_ARG, "%s: idx_stride < topk", fn);
  NSA_REQUIRE(nsa::aligned(q, 16) && q_tok_stride % 8 == 0 && q_head_stride % 8 == 0 &&
                  q_head_stride >= kDQK && q_tok_stride >= (int64_t)H * q_head_stride,
              NSA_ERR_INVALID_ARG,
              "%s: q must be 16-byte aligned with strides multiples of 8 "
              "(head stride >= 576, token stride >= H * head stride)", fn);
  NSA_REQUIRE(nsa::aligned(kv, 16) && nsa::aligned(out, 16), NSA_ERR_INVALID_ARG,
              "%s: kv_cache and out must be 16-byte aligned", fn);
  return NSA_OK;
}

int run(const char* fn, bool decode, const void* q, int64_t q_tok_stride,
        int64_t q_head_stride, const void* kv_cache, int kv_dtype,
        int64_t num_slots, const int32_t* indices, int64_t idx_stride,
        const int32_t* nsa_cache_seqlens, int T, int H, int topk, int d_qk,
        int d_v, float sm_scale, void* out, float* lse, void* workspace,
        size_t ws_bytes, void* stream) {
  int st = check_args(fn, q, q_tok_stride, q_head_stride, kv_cache, kv_dtype,
                      num_slots, indices, idx_stride, T, H, topk, d_qk, d_v, out);
  if (st != NSA_OK) return st;
  if (T == 0) return nsa::ok();
  const bool fp8 = kv_dtype == NSA_KV_FP8_656;
  const Plan pl = make_plan(T, H, topk, decode, fp8);
  const size_t need = workspace_bytes(pl, T, H);
  NSA_REQUIRE(need == 0 || (workspace && ws_bytes >= need), NSA_ERR_WORKSPACE,
              "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  NSA_REQUIRE(need == 0 || nsa::aligned(workspace, 16), NSA_ERR_INVALID_ARG,
              "%s: workspace must be 16-byte aligned", fn);
  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.q_tok_stride = q_tok_stride;
  p.q_head_stride = q_head_stride;
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.num_slots = num_slots;
  p.idx = indices;
  p.idx_stride = idx_stride;
  p.seqlens = nsa_cache_seqlens;
  p.T = T;
  p.H = H;
  p.topk = topk;
  p.scale_log2 = sm_scale * kLog2e;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.ws_o = pl.n_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  p.ws_lse = pl.n_splits > 1
                 ? (pl.h128 ? reinterpret_cast<float*>(static_cast<uint16_t*>(workspace) +
                                                       (size_t)pl.n_splits * T * H * kDV)
                            : static_cast<float*>(workspace) + (size_t)pl.n_splits * T * H * kDV)
                 : nullptr;
  p.n_splits = pl.n_splits;
  p.split_slots = pl.split_slots;
  p.n_hb = pl.n_hb;
  const int64_t blocks = (int64_t)T * pl.n_hb * pl.n_splits;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks), block(pl.wide ? kThreadsW : kThreads);
#define NSA_MLA_LAUNCH(NH, HW)                                                      \
  do {                                                                            \
    if (fp8) hipLaunchKernelGGL((sparse_mla_kernel<NH, HW, true>), grid, block, 0, s, p); \
    else hipLaunchKernelGGL((sparse_mla_kernel<NH, HW, false>), grid, block, 0, s, p);    \
  } while (0)
  if (pl.h128) {
    launch_sparse_mla_h128(p, (unsigned)blocks, s);
  } else if (pl.wide) {
    hipLaunchKernelGGL(sparse_mla_h64_kernel, grid, block, 0, s, p);
  } else if (pl.hw == 2) {
    NSA_MLA_LAUNCH(1, 2);
  } else {
    NSA_MLA_LAUNCH(1, 1);
  }
#undef NSA_MLA_LAUNCH
  st = nsa::check_launch(fn);
  if (st != NSA_OK || pl.n_splits == 1) return st;
  const int64_t cb = ((int64_t)T * H + 3) / 4;
  const uint16_t* wsb = reinterpret_cast<const uint16_t*>(p.ws_o);
  if (pl.h128 && pl.n_splits == 2)
    hipLaunchKernelGGL(combine_bf16_kernel<2>, dim3((unsigned)cb), dim3(256), 0, s, wsb,
                       p.ws_lse, T, H, p.out, lse);
  else if (pl.h128 && pl.n_splits == 4)
    hipLaunchKernelGGL(combine_bf16_kernel<4>, dim3((unsigned)cb), dim3(256), 0, s, wsb,
                       p.ws_lse, T, H, p.out, lse);
  else if (pl.h128)
    hipLaunchKernelGGL(combine_splits_kernel<uint16_t>, dim3((unsigned)cb), dim3(256), 0, s,
                       wsb, p.ws_lse, T, H, pl.n_splits, p.out, lse);
  else
    hipLaunchKernelGGL(combine_splits_kernel<float>, dim3((unsigned)cb), dim3(256), 0, s,
                       p.ws_o, p.ws_lse, T, H, pl.n_splits, p.out, lse);
  return nsa::check_launch(fn);
}

// ---- allocation-free variant: the workspace is a file-scope device array
// (one copy per GPU, allocated when the code object loads). Host code never
// passes the array's name to a kernel: its device address comes from
// hipGetSymbolAddress, taken once per device and cached.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  NSA_REQUIRE(e == hipSuccess, NSA_ERR_LAUNCH, "%s: hipGetDevice: %s", fn,
              hipGetErrorString(e));
  NSA_REQUIRE(dev >= 0 && dev < kMaxDevices, NSA_ERR_UNSUPPORTED,
              "%s: device %d >= %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    NSA_REQUIRE(e == hipSuccess && p != nullptr, NSA_ERR_LAUNCH,
                "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return NSA_OK;
}

}  // namespace

extern "C" int nsa_sparse_mla_decode_noalloc(
    const void* q, int64_t q_tok_stride, int64_t q_head_stride,
    const void* kv_cache, int kv_dtype, int64_t num_slots,
    const int32_t* indices, int64_t idx_stride,
    const int32_t* nsa_cache_seqlens, int T, int H, int topk, int d_qk,
    int d_v, float sm_scale, void* out, float* lse, void* stream) {
  const char* fn = "nsa_sparse_mla_decode_noalloc";
  int st = check_args(fn, q, q_tok_stride, q_head_stride, kv_cache, kv_dtype,
                      num_slots, indices, idx_stride, T, H, topk, d_qk, d_v, out);
  if (st != NSA_OK) return st;
  if (T == 0) return nsa::ok();
  const size_t need =
      workspace_bytes(make_plan(T, H, topk, true, kv_dtype == NSA_KV_FP8_656), T, H);
  NSA_REQUIRE(need <= kScratchBytes, NSA_ERR_WORKSPACE,
              "%s: this shape needs %zu bytes of scratch, the static array holds %zu",
              fn, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(fn, &ws);
    if (st != NSA_OK) return st;
  }
  return run(fn, true, q, q_tok_stride, q_head_stride, kv_cache, kv_dtype,
             num_slots, indices, idx_stride, nsa_cache_seqlens, T, H, topk, d_qk,
             d_v, sm_scale, out, lse, ws, ws ? kScratchBytes : 0, stream);
}

extern "C" int nsa_sparse_mla_workspace_size(int T, int H, int topk, int d_v,
                                             size_t* bytes) {
  NSA_REQUIRE(bytes != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_sparse_mla_workspace_size: null output");
  NSA_REQUIRE(T >= 0 && H > 0 && H % 16 == 0 && topk > 0 && d_v == kDV,
              NSA_ERR_INVALID_ARG, "nsa_sparse_mla_workspace_size: bad sizes");
  // the largest of the decode and extend plans for either cache format, so
  // one buffer serves every call
  size_t w = 0;
  for (int dec = 0; dec < 2; ++dec)
    for (int f8 = 0; f8 < 2; ++f8) {
      const size_t b = workspace_bytes(make_plan(T, H, topk, dec != 0, f8 != 0), T, H);
      w = b > w ? b : w;
    }
  *bytes = w;
  return nsa::ok();
}

extern "C" int nsa_sparse_mla_decode(
    const void* q, int64_t q_tok_stride, int64_t q_head_stride,
    const void* kv_cache, int kv_dtype, int64_t num_slots,
    const int32_t* indices, int64_t idx_stride,
    const int32_t* nsa_cache_seqlens, int T, int H, int topk, int d_qk,
    int d_v, float sm_scale, void* out, float* lse, void* workspace,
    size_t ws_bytes, void* stream) {
  return run("nsa_sparse_mla_decode", true, q, q_tok_stride, q_head_stride,
             kv_cache, kv_dtype, num_slots, indices, idx_stride,
             nsa_cache_seqlens, T, H, topk, d_qk, d_v, sm_scale, out, lse,
             workspace, ws_bytes, stream);
}

extern "C" int nsa_sparse_mla_extend(
    const void* q, int64_t q_tok_stride, int64_t q_head_stride,
    const void* kv_cache, int kv_dtype, int64_t num_slots,
    const int32_t* indices, int64_t idx_stride,
    const int32_t* nsa_cache_seqlens, int T, int H, int topk, int d_qk,
    int d_v, float sm_scale, void* out, float* lse, void* workspace,
    size_t ws_bytes, void* stream) {
  return run("nsa_sparse_mla_extend", false, q, q_tok_stride, q_head_stride,
             kv_cache, kv_dtype, num_slots, indices, idx_stride,
             nsa_cache_seqlens, T, H, topk, d_qk, d_v, sm_scale, out, lse,
             workspace, ws_bytes, stream);
}
