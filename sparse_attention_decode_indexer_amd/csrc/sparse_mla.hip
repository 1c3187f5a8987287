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
//   * a block owns one query row, HB = 16*HW heads and one KV split; wave w
//     owns head tile w % HW and dim slice w / HW of DW = 4 / HW slices (so
//     16-head models use all 4 waves by splitting the 576 contraction dims
//     in QK and the 512 value dims in PV);
//   * per step, 32 selected slots are gathered with 16-byte loads (issued
//     one step ahead), dequantised to bf16 if the cache is fp8, and staged
//     in LDS twice: row-major for Q.K (A operand = keys, 16 slots x 32 dims
//     per v_mfma_f32_16x16x32_bf16) and transposed for P.V (B operand = 8
//     slots of one value dim);
//   * S^T = K.Q^T puts one head per lane column, so P is already in the A
//     layout of P.V (heads x slots) and needs no shuffles; the online
//     softmax runs in the log2 domain in fp32;
//   * KV splits write (o / l, lse) partials to the workspace and a second
//     kernel merges them in split order (bit-reproducible).
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 32;                 // slots per step
constexpr int kDQK = 576, kDV = 512;
constexpr int kKsStride = kDQK + 8;       // bf16 elements per staged K row
constexpr int kVtStride = kStep + 4;      // bf16 elements per staged V^T row
constexpr int kKsBytes = kStep * kKsStride * 2;   // 37376
constexpr int kVtBytes = kDV * kVtStride * 2;     // 36864
constexpr int kKSteps = kDQK / 32;        // 18 contraction steps of 32 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

// bf16 pair selection: lo halves of a and b -> (a.lo, b.lo); hi halves.
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Prefetch registers of one thread for one step.
template <bool FP8>
struct Stage;

// bf16 cache: two (4 slots x 8 dims) pieces of the value part + one rope
// piece of 8 dims.
template <>
struct Stage<false> {
  uint4 v[2][4];
  uint4 rope;
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids,
                                       int tid) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + it * kThreads;
      const int qd = item >> 6, ch = item & 63;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int32_t slot = ids[qd * 4 + s];
        if (slot >= 0)
          v[it][s] = *reinterpret_cast<const uint4*>(
              p.kv + (int64_t)slot * (kDQK * 2) + ch * 16);
        else
          v[it][s] = make_uint4(0, 0, 0, 0);
      }
    }
    const int32_t slot = ids[tid >> 3];
    rope = slot >= 0 ? *reinterpret_cast<const uint4*>(
                           p.kv + (int64_t)slot * (kDQK * 2) + kDV * 2 + (tid & 7) * 16)
                     : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(uint8_t* ks, uint8_t* vt, int tid) const {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + it * kThreads;
      const int qd = item >> 6, ch = item & 63;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(ks + (qd * 4 + s) * (kKsStride * 2) + ch * 16) = v[it][s];
      // transpose 4 slots x 8 dims -> 8 dims x 4 slots
      const uint32_t a[4] = {v[it][0].x, v[it][0].y, v[it][0].z, v[it][0].w};
      const uint32_t b[4] = {v[it][1].x, v[it][1].y, v[it][1].z, v[it][1].w};
      const uint32_t c[4] = {v[it][2].x, v[it][2].y, v[it][2].z, v[it][2].w};
      const uint32_t d[4] = {v[it][3].x, v[it][3].y, v[it][3].z, v[it][3].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dim = ch * 8 + 2 * e;
        uint2 w0 = make_uint2(lo_pair(a[e], b[e]), lo_pair(c[e], d[e]));
        uint2 w1 = make_uint2(hi_pair(a[e], b[e]), hi_pair(c[e], d[e]));
        *reinterpret_cast<uint2*>(vt + dim * (kVtStride * 2) + qd * 8) = w0;
        *reinterpret_cast<uint2*>(vt + (dim + 1) * (kVtStride * 2) + qd * 8) = w1;
      }
    }
    *reinterpret_cast<uint4*>(ks + (tid >> 3) * (kKsStride * 2) + kDV * 2 + (tid & 7) * 16) = rope;
  }
};

// fp8 cache (656-byte rows): one (4 slots x 16 codes) piece with the 4
// block scales + one rope piece of 8 dims.
template <>
struct Stage<true> {
  uint4 code[4];
  float scale[4];
  uint4 rope;
  __device__ __forceinline__ void load(const Params& p, const int32_t* ids,
                                       int tid) {
    const int qd = tid >> 5, cc = tid & 31;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int32_t slot = ids[qd * 4 + s];
      if (slot >= 0) {
        const uint8_t* row = p.kv + (int64_t)slot * 656;
        code[s] = *reinterpret_cast<const uint4*>(row + cc * 16);
        scale[s] = *reinterpret_cast<const float*>(row + 512 + 4 * (cc >> 3));
      } else {
        code[s] = make_uint4(0, 0, 0, 0);
        scale[s] = 0.0f;
      }
    }
    const int32_t slot = ids[tid >> 3];
    rope = slot >= 0 ? *reinterpret_cast<const uint4*>(p.kv + (int64_t)slot * 656 +
                                                       528 + (tid & 7) * 16)
                     : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(uint8_t* ks, uint8_t* vt, int tid) const {
    const int qd = tid >> 5, cc = tid & 31;
    uint32_t bf[4][8];  // [slot][dim pair]: 16 dims as 8 bf16 pairs
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w[4] = {code[s].x, code[s].y, code[s].z, code[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        bf[s][2 * i] = pack_bf16x2(lo[0] * scale[s], lo[1] * scale[s]);
        bf[s][2 * i + 1] = pack_bf16x2(hi[0] * scale[s], hi[1] * scale[s]);
      }
      uint8_t* dst = ks + (qd * 4 + s) * (kKsStride * 2) + cc * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(bf[s][0], bf[s][1], bf[s][2], bf[s][3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(bf[s][4], bf[s][5], bf[s][6], bf[s][7]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dim = cc * 16 + 2 * e;
      uint2 w0 = make_uint2(lo_pair(bf[0][e], bf[1][e]), lo_pair(bf[2][e], bf[3][e]));
      uint2 w1 = make_uint2(hi_pair(bf[0][e], bf[1][e]), hi_pair(bf[2][e], bf[3][e]));
      *reinterpret_cast<uint2*>(vt + dim * (kVtStride * 2) + qd * 8) = w0;
      *reinterpret_cast<uint2*>(vt + (dim + 1) * (kVtStride * 2) + qd * 8) = w1;
    }
    *reinterpret_cast<uint4*>(ks + (tid >> 3) * (kKsStride * 2) + kDV * 2 + (tid & 7) * 16) = rope;
  }
};

template <int HW, bool FP8>
__global__ void __launch_bounds__(kThreads, (HW == 4 ? 1 : 2))
sparse_mla_kernel(const Params p) {
  constexpr int DW = 4 / HW;                 // dim slices
  constexpr int KSW = (kKSteps + DW - 1) / DW;
  constexpr int NT = kDV / DW / 16;          // value-dim tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t ks[kKsBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kVtBytes];
  __shared__ int32_t ids[2][kStep];
  __shared__ uint32_t vmask[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hw = wave % HW, dw = wave / HW;

  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int hb = lb % p.n_hb;
  const int split = (lb / p.n_hb) % p.n_splits;
  const int64_t t = lb / (p.n_hb * p.n_splits);
  const int h0 = hb * (16 * HW) + hw * 16;   // first head of this wave

  int n_row = p.topk;
  if (p.seqlens) {
    const int sl = p.seqlens[t];
    n_row = sl < 0 ? 0 : (sl < n_row ? sl : n_row);
  }
  const int s_begin = split * p.split_slots;
  const int s_end = min(s_begin + p.split_slots, n_row);
  const int nsteps = s_end > s_begin ? (s_end - s_begin + kStep - 1) / kStep : 0;
  const int32_t* irow = p.idx + t * p.idx_stride;

  // Q as the B operand of S^T = K.Q^T: lane (head c, group g) holds dims
  // ks*32 + 8g .. +8 of its head for the wave's contraction steps
  bf16x8 qb[KSW];
  {
    const uint16_t* qh = p.q + t * p.q_tok_stride + (int64_t)(h0 + c) * p.q_head_stride;
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int kstep = dw + DW * i;
      if (kstep < kKSteps)
        qb[i] = *reinterpret_cast<const bf16x8*>(qh + kstep * 32 + g * 8);
    }
  }

  auto load_ids = [&](int step) -> int32_t {
    // thread j < 32: id of slot j of `step` (-1 when absent or invalid)
    const int pos = s_begin + step * kStep + tid;
    int32_t id = -1;
    if (tid < kStep && step < nsteps && pos < s_end) {
      id = irow[pos];
      if (id < 0 || id >= p.num_slots) id = -1;
    }
    return id;
  };
  auto publish_ids = [&](int buf, int32_t id) {
    if (tid < kStep) ids[buf][tid] = id;
    if (wave == 0) {
      const unsigned long long b = __ballot(tid < kStep && id >= 0);
      if (lane == 0) vmask[buf] = (uint32_t)b;
    }
  };

  f32x4 o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;

  Stage<FP8> st;
  if (nsteps > 0) {
    publish_ids(0, load_ids(0));
    publish_ids(1, load_ids(1));
    __syncthreads();
    st.load(p, ids[0], tid);
    st.store(ks, vt, tid);
    __syncthreads();
  }
  int32_t id_ahead = load_ids(2);

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) st.load(p, ids[buf ^ 1], tid);   // next step's slots

    // ---- S^T = K . Q^T (partial over this wave's contraction steps)
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int kstep = dw + DW * i;
      if (kstep < kKSteps) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              ks + (mt * 16 + c) * (kKsStride * 2) + (kstep * 32 + g * 8) * 2);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], acc[mt], 0, 0, 0);
        }
      }
    }
    if constexpr (DW > 1) {
      // sum the DW partial scores of this head tile, in slice order
      float* red = reinterpret_cast<float*>(ks);
      __syncthreads();  // every wave has finished reading ks
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * 2 + mt) * 4 + r) * 64 + lane] = acc[mt][r];
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < DW; ++j)
            s += red[(((j * HW + hw) * 2 + mt) * 4 + r) * 64 + lane];
          acc[mt][r] = s;
        }
    }

    // ---- online softmax: lane (head c, group g) holds slots mt*16+4g+r
    const uint32_t valid = vmask[buf];
    float sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = mt * 16 + 4 * g + r;
        sv[mt][r] = ((valid >> j) & 1u) ? acc[mt][r] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[mt][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m - m_use);
    float psum = 0.0f;
    uint32_t pw[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = exp2f(sv[mt][r] - m_use);
        psum += pr[r];
      }
      pw[mt * 2] = pack_bf16x2(pr[0], pr[1]);
      pw[mt * 2 + 1] = pack_bf16x2(pr[2], pr[3]);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l = l * alpha + psum;
    m = m_new;
    bf16x8 pa;
    {
      const uint4 u = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      pa = *reinterpret_cast<const bf16x8*>(&u);
    }

    // ---- rescale O rows (heads 4g + r) and accumulate P . V
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[nt][r] *= al[r];
      const int dim = dw * (kDV / DW) + nt * 16 + c;
      const uint8_t* vrow = vt + dim * (kVtStride * 2);
      const uint2 b0 = *reinterpret_cast<const uint2*>(vrow + g * 8);
      const uint2 b1 = *reinterpret_cast<const uint2*>(vrow + 32 + g * 8);
      const uint4 bu = make_uint4(b0.x, b0.y, b1.x, b1.y);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&bu);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[nt], 0, 0, 0);
    }

    // ---- stage the next step
    __syncthreads();  // all waves are done with ks / vt / ids[buf]
    if (more) st.store(ks, vt, tid);
    publish_ids(buf, id_ahead);     // ids of step + 2
    id_ahead = load_ids(step + 3);
    __syncthreads();
  }

  // ---- finalize: lane (dim c of tile nt, group g) holds O[head 4g+r][dim]
  float lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lr[r] = __shfl(l, 4 * g + r);
  const float lse_val = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  if (p.n_splits == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int dim = dw * (kDV / DW) + nt * 16 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = lr[r] > 0.0f ? o[nt][r] / lr[r] : 0.0f;
        p.out[(t * p.H + h0 + 4 * g + r) * kDV + dim] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
    if (p.lse && dw == 0 && g == 0) p.lse[t * p.H + h0 + c] = lse_val;
  } else {
    const int64_t base = ((int64_t)split * p.T + t) * p.H;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int dim = dw * (kDV / DW) + nt * 16 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = lr[r] > 0.0f ? o[nt][r] / lr[r] : 0.0f;
        p.ws_o[(base + h0 + 4 * g + r) * kDV + dim] = v;
      }
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
  int hb_heads, n_hb, n_splits, split_slots;
};

Plan make_plan(int T, int H, int topk, bool decode) {
  Plan pl;
  pl.hb_heads = (H % 64 == 0) ? 64 : ((H % 32 == 0) ? 32 : 16);
  pl.n_hb = H / pl.hb_heads;
  const int64_t base = (int64_t)T * pl.n_hb;
  const int max_splits = (topk + 127) / 128;   // >= 128 slots per split
  int ns = 1;
  const int64_t target = decode ? 512 : 256;
  if (base < target) ns = (int)((target + base - 1) / base);
  ns = ns < 1 ? 1 : (ns > max_splits ? max_splits : ns);
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
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (pl.hb_heads == 64) {
    if (fp8) hipLaunchKernelGGL((sparse_mla_kernel<4, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((sparse_mla_kernel<4, false>), grid, block, 0, s, p);
  } else if (pl.hb_heads == 32) {
    if (fp8) hipLaunchKernelGGL((sparse_mla_kernel<2, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((sparse_mla_kernel<2, false>), grid, block, 0, s, p);
  } else {
    if (fp8) hipLaunchKernelGGL((sparse_mla_kernel<1, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((sparse_mla_kernel<1, false>), grid, block, 0, s, p);
  }
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
