// a4 / a5: MLA attention over the selected KV slots of a shared 576-wide
// latent cache (512 no-rope + 64 rope; value = the first 512).
//
// Semantics ("nsa_backend.py (EngineX-Hygon sglang fork)", _forward_fa3 and
// the FlashMLA routes): per query row t and head h, over the valid slots I_t
// of the row's index list (first nsa_cache_seqlens[t] entries, -1 skipped),
//   s_i = sm_scale * q[t,h,:576] . K_i[:576],  o = softmax(s) . K[:, :512],
//   lse = log sum_i exp(s_i).
//
// MI355X design (one 256-thread block = 4 waves):
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
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 32;                 // slots per step
constexpr int kDQK = 576, kDV = 512;
constexpr int kKsStride = kDQK + 8;       // bf16 elements per staged K row
constexpr int kKsRow = kKsStride * 2;     // bytes per staged K row (1168)
constexpr int kKsBytes = kStep * kKsRow;  // 37376
constexpr int kKSteps = kDQK / 32;        // 18 contraction steps of 32 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;             // log2 headroom before O is rescaled

struct Params {
  const uint16_t* q;
  int64_t q_tok_stride, q_head_stride;
  const uint8_t* kv;
  int64_t num_slots;
  const int32_t* idx;
  int64_t idx_stride;
  const int32_t* seqlens;  // nullable
  int T, H, topk;
  float scale_log2;
  uint16_t* out;
  float* lse;              // nullable
  float* ws_o;             // [n_splits][T][H][512] when n_splits > 1
  float* ws_lse;           // [n_splits][T][H]
  int n_splits, split_slots, n_hb;
};

__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t bid, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = bid % 8;
  return x * q + (x < r ? x : r) + bid / 8;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 4 bf16 of one value dim across 4 slot rows (see the design note above).
__device__ __forceinline__ v4i16 read_tr(const uint8_t* lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) uint8_t*)lds_byte_addr);
}

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

// ---- 64 heads per block (H a multiple of 64) --------------------------------
// One 512-thread block (8 waves) per (row, 64 heads, KV split), one block per
// CU. Wave (ht = w % 4, dw = w / 4) owns heads 16*ht.. of the block and half
// dw of the work: contraction dims of 128-blocks 2dw, 2dw+1 plus rope step
// 16+dw for S, and value dims 256*dw.. for O. The two halves of a head
// tile's scores meet in LDS and are added in the same order in both waves,
// so both run an identical softmax. The split's slot ids and per-step valid
// masks are loaded into LDS once; the bf16 K tile is double-buffered (two
// barriers per step: score exchange and tile swap); the gather of step s+3
// is issued while step s is computed, from two register stages that
// alternate (the step loop is unrolled by two, so no register copy waits on
// a load in flight).
constexpr int kThreadsW = 512;
constexpr int kMaxSplit = 2048;                // slots per block
constexpr int kIdsCap = 5 * kThreadsW;         // 2560 >= kMaxSplit + 4 steps of overrun
constexpr int kMaskCap = kIdsCap / kStep;      // 80 steps

// Gather registers of one thread of a 512-thread block for one step: slot
// qd = tid / 16 of the step, 16-byte chunks cc and cc + 16 of its value part
// and 8 bytes of its rope part.
template <bool FP8>
struct StageW;

template <>
struct StageW<true> {   // 656-byte rows
  uint2 code[4];         // codes 8cc + 128k .. +8 (block k)
  float scale;           // block scale cc % 4 of the slot
  uint2 rope;
  bool valid;
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids, int tid) {
    const int qd = tid >> 4, cc = tid & 15;
    const int32_t slot = ids[qd];
    valid = slot >= 0;
    const uint8_t* row = p.kv + (int64_t)(slot >= 0 ? slot : 0) * 656;
#pragma unroll
    for (int k = 0; k < 4; ++k) code[k] = *reinterpret_cast<const uint2*>(row + 8 * cc + 128 * k);
    scale = *reinterpret_cast<const float*>(row + 512 + 4 * (cc & 3));
    rope = *reinterpret_cast<const uint2*>(row + 528 + 8 * cc);
  }
  // exact fp8 -> bf16 (every e4m3 value is a bf16 value: the upper halves of
  // the fp32 images); the block scales go to LDS and are applied to the
  // scores and to P. Consecutive lanes write consecutive 16-byte pieces.
  __device__ __forceinline__ void store(uint8_t* kt, float* scl, int tid) const {
    const int qd = tid >> 4, cc = tid & 15;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint2 cs = valid ? code[k] : make_uint2(0, 0);
      uint32_t bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wi = i == 0 ? cs.x : cs.y;
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wi, true);
        bf[2 * i] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
        bf[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
      }
      *reinterpret_cast<uint4*>(kt + qd * kKsRow + 16 * cc + 256 * k) =
          make_uint4(bf[0], bf[1], bf[2], bf[3]);
    }
    // 4 lanes of the slot write each block scale (identical values)
    scl[qd * 4 + (cc & 3)] = valid ? scale : 0.0f;
    *reinterpret_cast<uint2*>(kt + qd * kKsRow + kDV * 2 + 8 * cc) =
        valid ? rope : make_uint2(0, 0);
  }
};

template <>
struct StageW<false> {  // 576 bf16 rows
  uint4 v[4];
  uint2 rope;
  bool valid;
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids, int tid) {
    const int qd = tid >> 4, cc = tid & 15;
    const int32_t slot = ids[qd];
    valid = slot >= 0;
    const uint8_t* row = p.kv + (int64_t)(slot >= 0 ? slot : 0) * (kDQK * 2);
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = *reinterpret_cast<const uint4*>(row + 16 * (cc + 16 * h));
    rope = *reinterpret_cast<const uint2*>(row + kDV * 2 + 8 * cc);
  }
  __device__ __forceinline__ void store(uint8_t* kt, float*, int tid) const {
    const int qd = tid >> 4, cc = tid & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<uint4*>(kt + qd * kKsRow + 16 * (cc + 16 * h)) =
          valid ? v[h] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint2*>(kt + qd * kKsRow + kDV * 2 + 8 * cc) =
        valid ? rope : make_uint2(0, 0);
  }
};

template <bool FP8>
__global__ void __launch_bounds__(kThreadsW, 1)
sparse_mla_h64_kernel(const Params p) {
  constexpr int NT = kDV / 2 / 16;           // 16 value-dim tiles per wave
  constexpr int KS = kKSteps / 2;            // 9 contraction steps per wave
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][kKsBytes];
  __shared__ __attribute__((aligned(16))) float scl[2][FP8 ? kStep * 4 : 4];
  __shared__ int32_t ids[kIdsCap];
  __shared__ uint32_t vmask[kMaskCap];
  __shared__ float xch[8][8][64];            // partial scores per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ht = wave & 3, dw = wave >> 2;

  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int hb = lb % p.n_hb;
  const int split = (lb / p.n_hb) % p.n_splits;
  const int64_t t = lb / (p.n_hb * p.n_splits);
  const int h0 = hb * 64 + ht * 16;          // first head of this wave

  int n_row = p.num_slots > 0 ? p.topk : 0;
  if (p.seqlens) {
    const int sl = p.seqlens[t];
    n_row = sl < 0 ? 0 : (sl < n_row ? sl : n_row);
  }
  const int s_begin = split * p.split_slots;
  const int n = min(s_begin + p.split_slots, n_row) - s_begin;   // may be <= 0
  const int nsteps = n > 0 ? (n + kStep - 1) / kStep : 0;

  // ---- slot ids of the split (validated; -1 past its end) and step masks
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
      ids[i] = (i < n && id >= 0 && id < p.num_slots) ? id : -1;
    }
  }
  __syncthreads();
  for (int k = wave; k < kMaskCap; k += 8) {
    const bool ok = lane < kStep && ids[k * kStep + (lane & (kStep - 1))] >= 0;
    const unsigned long long b = __ballot(ok);
    if (lane == 0) vmask[k] = (uint32_t)b;
  }

  // Q as the B operand of S^T = K.Q^T: lane (head c, group g) holds dims
  // kstep*32 + 8g .. +8 of the wave's 9 contraction steps (blocks 2dw, 2dw+1
  // and rope step 16 + dw)
  bf16x8 qb[KS];
  {
    const uint16_t* qh = p.q + t * p.q_tok_stride + (int64_t)(h0 + c) * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int kstep = i < 8 ? dw * 8 + i : 16 + dw;
      qb[i] = *reinterpret_cast<const bf16x8*>(qh + kstep * 32 + g * 8);
    }
  }

  f32x4 o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;   // reference max (log2 domain) and sum of head c

  // one step over the staged tile `kt` (block scales `sc` for an fp8 cache)
  auto compute = [&](const uint8_t* kt, const float* sc, uint32_t valid) {
    auto kfrag = [&](int mt, int kstep) {
      return *reinterpret_cast<const bf16x8*>(kt + (mt * 16 + c) * kKsRow + (kstep * 32 + g * 8) * 2);
    };
    // ---- partial S^T over this wave's steps: two 128-dim blocks (fp8: each
    // its own accumulator, scaled by the slot's block scale) and one rope
    // step. The fragments of step kk+1 are read while step kk is multiplied;
    // consecutive MFMAs go to independent accumulators.
    f32x4 tb[3][2];
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) tb[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fr[2][2][2];   // [buffer][u][mt]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) fr[0][u][mt] = kfrag(mt, dw * 8 + u * 4);
#pragma unroll
    for (int kk = 0; kk < 5; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk < 3) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) fr[nxt][u][mt] = kfrag(mt, dw * 8 + u * 4 + kk + 1);
      } else if (kk == 3) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) fr[nxt][0][mt] = kfrag(mt, 16 + dw);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 4) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            tb[u][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[cur][u][mt], qb[u * 4 + kk], tb[u][mt], 0, 0, 0);
      } else {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          tb[2][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[cur][0][mt], qb[8], tb[2][mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (head c, group g) holds slots mt*16 + 4g + r
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float part;
        if constexpr (FP8) {
          const float2 s2 = *reinterpret_cast<const float2*>(sc + (mt * 16 + 4 * g + r) * 4 + 2 * dw);
          part = fmaf(s2.x, tb[0][mt][r], fmaf(s2.y, tb[1][mt][r], tb[2][mt][r]));
        } else {
          part = (tb[0][mt][r] + tb[1][mt][r]) + tb[2][mt][r];
        }
        xch[wave][mt * 4 + r][lane] = part;
      }
    __syncthreads();
    // full scores: own half + partner half (a + b == b + a, so both waves of
    // the pair hold identical scores); absent slots get -inf by adding it
    float pv[2][4];
    float lmx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sfull = xch[wave][mt * 4 + r][lane] + xch[wave ^ 4][mt * 4 + r][lane];
        const int j = mt * 16 + 4 * g + r;
        const float off = ((valid >> j) & 1u) ? 0.0f : -INFINITY;
        pv[mt][r] = fmaf(sfull, p.scale_log2, off);
        lmx = fmaxf(lmx, pv[mt][r]);
      }

    // ---- online softmax with a lazily raised reference max: O is rescaled
    // only in the rare step where a score of a head exceeds its reference
    // max by more than kLazy; l is kept per lane and summed at the end
    if (__builtin_amdgcn_ballot_w64(lmx > m + kLazy) != 0) {
      float mx = lmx;
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool upd = mx > m + kLazy;        // same in the head's 4 lanes
      const float alpha = upd ? exp2f(m - mx) : 1.0f;   // m = -inf -> 0
      if (upd) m = mx;
      l *= alpha;
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nt][r] *= al[r];
    }
    // exponents are at most kLazy; weights below 2^-126 may flush to zero
    const float m_use = m == -INFINITY ? 0.0f : m;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[mt][r] = __builtin_amdgcn_exp2f(pv[mt][r] - m_use);
        l += pv[mt][r];
      }
    __builtin_amdgcn_sched_barrier(0);

    // ---- P . V over this wave's two value blocks; for an fp8 cache P
    // carries the slot's scale of the block. The B fragments of tile j+1 are
    // read while tile j is multiplied.
    auto vfrag = [&](int vb, int j) {
      const uint8_t* src = kt + (4 * g + (c >> 2)) * kKsRow + (vb * 128 + j * 16 + 4 * (c & 3)) * 2;
      const v4i16 b0 = read_tr(src);
      const v4i16 b1 = read_tr(src + 16 * kKsRow);
      const v4i16 bb[2] = {b0, b1};
      return *reinterpret_cast<const bf16x8*>(bb);
    };
    bf16x8 vf[2];
    vf[0] = vfrag(dw * 2, 0);
#pragma unroll
    for (int vh = 0; vh < 2; ++vh) {
      const int vb = dw * 2 + vh;
      bf16x8 pa;
      {
        float q8[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = 1.0f;
            if constexpr (FP8) s = sc[(mt * 16 + 4 * g + r) * 4 + vb];
            q8[mt][r] = pv[mt][r] * s;
          }
        const uint4 u = make_uint4(pack_bf16x2_hw(q8[0][0], q8[0][1]), pack_bf16x2_hw(q8[0][2], q8[0][3]),
                                   pack_bf16x2_hw(q8[1][0], q8[1][1]), pack_bf16x2_hw(q8[1][2], q8[1][3]));
        pa = *reinterpret_cast<const bf16x8*>(&u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = vh * 8 + j;             // tile index within the wave
        if (q + 1 < NT) vf[(q + 1) & 1] = vfrag(dw * 2 + (q + 1) / 8, (q + 1) % 8);
        __builtin_amdgcn_sched_barrier(0);
        o[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vf[q & 1], o[q], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (nsteps > 0) {
    StageW<FP8> sa, sb;
    sa.load(p, ids, tid);
    sb.load(p, ids + kStep, tid);
    sa.store(ks[0], scl[0], tid);
    sa.load(p, ids + 2 * kStep, tid);
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
      sb.store(ks[1], scl[1], tid);                 // step s + 1
      sb.load(p, ids + (s + 3) * kStep, tid);       // step s + 3
      __builtin_amdgcn_sched_barrier(0);
      compute(ks[0], scl[0], vmask[s]);
      __syncthreads();
      sa.store(ks[0], scl[0], tid);                 // step s + 2
      sa.load(p, ids + (s + 4) * kStep, tid);       // step s + 4
      __builtin_amdgcn_sched_barrier(0);
      compute(ks[1], scl[1], vmask[s + 1]);         // empty when s + 1 == nsteps
      __syncthreads();
    }
  }

  // ---- finalize: lane (dim c of tile nt, group g) holds O[head 4g+r][dim]
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lr[r] = __shfl(l, 4 * g + r);
  const float lse_val = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  const int d0 = dw * (kDV / 2);
  if (p.n_splits == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = lr[r] > 0.0f ? o[nt][r] / lr[r] : 0.0f;
        p.out[(t * p.H + h0 + 4 * g + r) * kDV + d0 + nt * 16 + c] = (uint16_t)f32_to_bf16_bits(v);
      }
    if (p.lse && dw == 0 && g == 0) p.lse[t * p.H + h0 + c] = lse_val;
  } else {
    const int64_t base = ((int64_t)split * p.T + t) * p.H;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = lr[r] > 0.0f ? o[nt][r] / lr[r] : 0.0f;
        p.ws_o[(base + h0 + 4 * g + r) * kDV + d0 + nt * 16 + c] = v;
      }
    if (dw == 0 && g == 0) p.ws_lse[base + h0 + c] = lse_val;
  }
}

// Merge of KV-split partials, in split order: one wave per (row, head).
__global__ void __launch_bounds__(256)
combine_splits_kernel(const float* __restrict__ ws_o,
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
      const float4* src = reinterpret_cast<const float4*>(ws_o + (s * TH + th) * kDV + lane * 8);
      const float4 a = src[0], b = src[1];
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

struct Plan {
  bool wide;   // 64 heads per block (sparse_mla_h64_kernel)
  int nh, hw, hb_heads, n_hb, n_splits, split_slots;
};

// Heads per block and KV splits: the 64-head kernel runs one block per CU,
// so it aims at 256 blocks (one per CU) and at most kMaxSplit slots per
// block; the narrower kernel runs two blocks per CU.
Plan make_plan(int T, int H, int topk, bool decode) {
  Plan pl;
  pl.wide = H % 64 == 0;
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
  const Plan pl = make_plan(T, H, topk, decode);
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
                 ? static_cast<float*>(workspace) + (size_t)pl.n_splits * T * H * kDV
                 : nullptr;
  p.n_splits = pl.n_splits;
  p.split_slots = pl.split_slots;
  p.n_hb = pl.n_hb;
  const int64_t blocks = (int64_t)T * pl.n_hb * pl.n_splits;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  hipStream_t s = (hipStream_t)stream;
  const bool fp8 = kv_dtype == NSA_KV_FP8_656;
  const dim3 grid((unsigned)blocks), block(pl.wide ? kThreadsW : kThreads);
#define NSA_MLA_LAUNCH(NH, HW)                                                      \
  do {                                                                            \
    if (fp8) hipLaunchKernelGGL((sparse_mla_kernel<NH, HW, true>), grid, block, 0, s, p); \
    else hipLaunchKernelGGL((sparse_mla_kernel<NH, HW, false>), grid, block, 0, s, p);    \
  } while (0)
  if (pl.wide) {
    if (fp8) hipLaunchKernelGGL(sparse_mla_h64_kernel<true>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(sparse_mla_h64_kernel<false>, grid, block, 0, s, p);
  } else if (pl.hw == 2) {
    NSA_MLA_LAUNCH(1, 2);
  } else {
    NSA_MLA_LAUNCH(1, 1);
  }
#undef NSA_MLA_LAUNCH
  st = nsa::check_launch(fn);
  if (st != NSA_OK || pl.n_splits == 1) return st;
  const int64_t cb = ((int64_t)T * H + 3) / 4;
  hipLaunchKernelGGL(combine_splits_kernel, dim3((unsigned)cb), dim3(256), 0, s,
                     p.ws_o, p.ws_lse, T, H, pl.n_splits, p.out, lse);
  return nsa::check_launch(fn);
}

}  // namespace

extern "C" int nsa_sparse_mla_workspace_size(int T, int H, int topk, int d_v,
                                             size_t* bytes) {
  NSA_REQUIRE(bytes != nullptr, NSA_ERR_INVALID_ARG,
              "nsa_sparse_mla_workspace_size: null output");
  NSA_REQUIRE(T >= 0 && H > 0 && H % 16 == 0 && topk > 0 && d_v == kDV,
              NSA_ERR_INVALID_ARG, "nsa_sparse_mla_workspace_size: bad sizes");
  // the larger of the decode and extend plans, so one buffer serves both
  const Plan a = make_plan(T, H, topk, true), b = make_plan(T, H, topk, false);
  const size_t wa = workspace_bytes(a, T, H), wb = workspace_bytes(b, T, H);
  *bytes = wa > wb ? wa : wb;
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
