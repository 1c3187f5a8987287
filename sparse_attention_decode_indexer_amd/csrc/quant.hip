// a6: bf16 latent cache -> fp8 e4m3fn block-scaled cache (656 bytes / slot).
//
// "nsa_backend.py (EngineX-Hygon sglang fork)", _forward_flashmla_decode, and
// "dsa_backend.py (sglang main)", _forward_flashmla_kv, call
// quantize_k_cache(kv_cache) to produce the fp8 cache the sparse decode reads.
// The byte layout and rounding (not on the pages) are the reading stated in
// nsa.h: 512 codes in 4 blocks of 128, 4 fp32 scales amax/448, 64 bf16 rope.
//
// The same encoder also runs as quantize-on-write: "dsa_backend.py (sglang
// main)", forward_extend / forward_decode, store the new tokens' latent rows
// with token_to_kv_pool.set_mla_kv_buffer(layer, cache_loc, k, k_rope);
// nsa_set_mla_kv_buffer writes row i to slot cache_loc[i], encoded in the
// cache's own format (fp8 rows exactly as quantize_k_cache makes them, bf16
// rows copied).
//
// One wave per row: lane l owns no-rope elements 8l..8l+7 (block l/16), so a
// block's amax is a 16-lane reduction; lane l also copies rope element l.
// The encoder is written from the e4m3fn definition (bias 7, 3 mantissa bits,
// subnormals below 2^-6, largest finite 448) with round-to-nearest-even and
// saturation; the quotient x/scale is an IEEE fp32 division.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kSlotsPerBlock = kThreads / 64;

// e4m3fn code of a finite float: RNE, saturating at +-448.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9
    // a * 512 is exact (power-of-two scaling); rint rounds half to even.
    // A result of 8 is the smallest normal, whose code is also 8.
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;           // -6 .. 8
    uint32_t m = (au >> 20) & 0x7u;          // top 3 mantissa bits
    const uint32_t rest = au & 0xFFFFFu;     // the 20 bits rounded away
    const uint32_t half = 0x80000u;
    if (rest > half || (rest == half && (m & 1u))) {
      m += 1;
      if (m == 8) { m = 0; e += 1; }
    }
    code = ((uint32_t)(e + 7) << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;          // cannot happen below 448
  }
  return sign | code;
}

// Latent rows i = 0..n-1: 512 no-rope bf16 at nope + i * nope_stride, 64
// rope bf16 at rope + i * rope_stride (elements).
struct Rows {
  const uint16_t* nope;
  int64_t nope_stride;
  const uint16_t* rope;
  int64_t rope_stride;
};

// Destination slot of row i: i itself (whole-cache conversion) or
// cache_loc[i]; a slot outside [0, num_slots) is skipped.
template <bool SCATTER>
__device__ __forceinline__ int64_t dest_slot(const int32_t* cache_loc, int64_t i,
                                             int64_t num_slots) {
  if constexpr (SCATTER) {
    const int64_t s = cache_loc[i];
    if (s >= 0 && s < num_slots) return s;
    flag_device_error(NSA_DEVERR_SLOT);
    return -1;
  } else {
    return i;
  }
}

template <bool SCATTER>
__global__ void __launch_bounds__(kThreads)
quantize_rows_kernel(Rows src, int64_t n, const int32_t* __restrict__ cache_loc,
                     int64_t num_slots, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kSlotsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t slot = dest_slot<SCATTER>(cache_loc, i, num_slots);
  if (slot < 0) return;
  const uint16_t* row = src.nope + i * src.nope_stride;
  uint8_t* orow = out + slot * 656;

  const uint4 raw = *reinterpret_cast<const uint4*>(row + lane * 8);
  float x[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;

  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= encode_e4m3(x[i] / scale) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= encode_e4m3(x[4 + i] / scale) << (8 * i);
  *reinterpret_cast<uint2*>(orow + lane * 8) = make_uint2(lo, hi);
  if ((lane & 15) == 0)
    *reinterpret_cast<float*>(orow + 512 + 4 * (lane >> 4)) = scale;
  reinterpret_cast<uint16_t*>(orow + 528)[lane] = src.rope[i * src.rope_stride + lane];
}

// bf16 cache rows: 512 + 64 values copied into the 1152-byte slot row (lane l
// copies no-rope bytes 16l..16l+15; lanes 0..7 the rope bytes).
__global__ void __launch_bounds__(kThreads)
copy_rows_kernel(Rows src, int64_t n, const int32_t* __restrict__ cache_loc,
                 int64_t num_slots, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kSlotsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t slot = dest_slot<true>(cache_loc, i, num_slots);
  if (slot < 0) return;
  uint8_t* orow = out + slot * (NSA_D_QK * 2);
  *reinterpret_cast<uint4*>(orow + 16 * lane) =
      *reinterpret_cast<const uint4*>(src.nope + i * src.nope_stride + 8 * lane);
  if (lane < 8)
    *reinterpret_cast<uint4*>(orow + 1024 + 16 * lane) =
        *reinterpret_cast<const uint4*>(src.rope + i * src.rope_stride + 8 * lane);
}

// The RAGGED extend route's dequantize_k_cache_paged ("dsa_backend.py
// (sglang main)", forward_extend): row i of the output is the bf16 latent row
// of slot slots[i] -- each no-rope value the fp32 product of its e4m3 code and
// its block scale, rounded to bf16 (nearest even), the rope values copied; a
// slot outside the cache gives a zero row. One wave per row; lane l decodes
// values 8l..8l+7 (block l / 16) and lanes 0..7 copy 16 rope bytes each.
__global__ void __launch_bounds__(kThreads)
dequantize_paged_kernel(const uint8_t* __restrict__ cache, int64_t num_slots,
                        const int32_t* __restrict__ slots, int64_t n,
                        uint16_t* __restrict__ out, int64_t out_stride) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kSlotsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t slot = slots[i];
  const bool ok = slot >= 0 && slot < num_slots;
  if (!ok && lane == 0) flag_device_error(NSA_DEVERR_SLOT);
  const uint8_t* row = cache + (ok ? slot : 0) * 656;
  uint16_t* orow = out + i * out_stride;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (ok) {
    const uint2 codes = *reinterpret_cast<const uint2*>(row + 8 * lane);
    const float scale = *reinterpret_cast<const float*>(row + 512 + 4 * (lane >> 4));
    const uint32_t w[2] = {codes.x, codes.y};
    uint32_t bf[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
      bf[2 * k] = pack_bf16x2(lo[0] * scale, lo[1] * scale);
      bf[2 * k + 1] = pack_bf16x2(hi[0] * scale, hi[1] * scale);
    }
    v = make_uint4(bf[0], bf[1], bf[2], bf[3]);
  }
  *reinterpret_cast<uint4*>(orow + 8 * lane) = v;
  if (lane < 8)
    *reinterpret_cast<uint4*>(orow + 512 + 8 * lane) =
        ok ? *reinterpret_cast<const uint4*>(row + 528 + 16 * lane) : make_uint4(0, 0, 0, 0);
}

}  // namespace

extern "C" int nsa_dequantize_k_cache_paged(const void* kv_fp8, int64_t num_slots,
                                            const int32_t* slots, int64_t n,
                                            void* out, int64_t out_stride,
                                            void* stream) {
  const char* fn = "nsa_dequantize_k_cache_paged";
  NSA_REQUIRE(n >= 0 && num_slots >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n == 0) return nsa::ok();
  NSA_REQUIRE(slots && out && (kv_fp8 || num_slots == 0), NSA_ERR_INVALID_ARG,
              "%s: null pointer", fn);
  NSA_REQUIRE(out_stride >= NSA_D_QK && out_stride % 8 == 0, NSA_ERR_INVALID_ARG,
              "%s: out_stride must be >= 576 and a multiple of 8", fn);
  NSA_REQUIRE(nsa::aligned(out, 16) && nsa::aligned(kv_fp8, 16), NSA_ERR_INVALID_ARG,
              "%s: out and kv_fp8 must be 16-byte aligned", fn);
  const int64_t blocks = (n + kSlotsPerBlock - 1) / kSlotsPerBlock;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  hipLaunchKernelGGL(dequantize_paged_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, static_cast<const uint8_t*>(kv_fp8),
                     num_slots, slots, n, static_cast<uint16_t*>(out), out_stride);
  return nsa::check_launch(fn);
}

extern "C" int nsa_quantize_k_cache(const void* kv_bf16, int64_t num_slots,
                                    int64_t in_stride, void* out,
                                    void* stream) {
  const char* fn = "nsa_quantize_k_cache";
  NSA_REQUIRE(num_slots >= 0, NSA_ERR_INVALID_ARG, "%s: negative num_slots", fn);
  if (num_slots == 0) return nsa::ok();
  NSA_REQUIRE(kv_bf16 && out, NSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  NSA_REQUIRE(in_stride >= NSA_D_QK && in_stride % 8 == 0, NSA_ERR_INVALID_ARG,
              "%s: in_stride must be >= 576 and a multiple of 8", fn);
  NSA_REQUIRE(nsa::aligned(kv_bf16, 16) && nsa::aligned(out, 16),
              NSA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  const int64_t blocks = (num_slots + kSlotsPerBlock - 1) / kSlotsPerBlock;
  NSA_REQUIRE(blocks < (1ll << 31), NSA_ERR_UNSUPPORTED, "%s: too many slots", fn);
  const uint16_t* kv = static_cast<const uint16_t*>(kv_bf16);
  const Rows src{kv, in_stride, kv + 512, in_stride};
  hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3((unsigned)blocks),
                     dim3(kThreads), 0, (hipStream_t)stream, src, num_slots,
                     nullptr, num_slots, static_cast<uint8_t*>(out));
  return nsa::check_launch(fn);
}

extern "C" int nsa_set_mla_kv_buffer(const void* k_nope, int64_t nope_stride,
                                     const void* k_rope, int64_t rope_stride,
                                     const int32_t* cache_loc, int n,
                                     void* kv_cache, int kv_dtype,
                                     int64_t num_slots, void* stream) {
  const char* fn = "nsa_set_mla_kv_buffer";
  NSA_REQUIRE(n >= 0 && num_slots >= 0, NSA_ERR_INVALID_ARG, "%s: negative size", fn);
  NSA_REQUIRE(kv_dtype == NSA_KV_BF16_576 || kv_dtype == NSA_KV_FP8_656,
              NSA_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  if (n == 0 || num_slots == 0) return nsa::ok();
  NSA_REQUIRE(k_nope && k_rope && cache_loc && kv_cache, NSA_ERR_INVALID_ARG,
              "%s: null pointer", fn);
  NSA_REQUIRE(nope_stride >= NSA_D_V && nope_stride % 8 == 0 && nsa::aligned(k_nope, 16),
              NSA_ERR_INVALID_ARG,
              "%s: k_nope must be 16-byte aligned with a row stride >= 512 "
              "and a multiple of 8", fn);
  NSA_REQUIRE(rope_stride >= NSA_D_QK - NSA_D_V, NSA_ERR_INVALID_ARG,
              "%s: rope_stride < 64", fn);
  if (kv_dtype == NSA_KV_BF16_576)
    NSA_REQUIRE(rope_stride % 8 == 0 && nsa::aligned(k_rope, 16), NSA_ERR_INVALID_ARG,
                "%s: for a bf16 cache k_rope must be 16-byte aligned with a row "
                "stride that is a multiple of 8", fn);
  else
    NSA_REQUIRE(nsa::aligned(k_rope, 2), NSA_ERR_INVALID_ARG,
                "%s: k_rope must be 2-byte aligned", fn);
  NSA_REQUIRE(nsa::aligned(kv_cache, 16), NSA_ERR_INVALID_ARG,
              "%s: kv_cache must be 16-byte aligned", fn);
  const int64_t blocks = ((int64_t)n + kSlotsPerBlock - 1) / kSlotsPerBlock;
  const Rows src{static_cast<const uint16_t*>(k_nope), nope_stride,
                 static_cast<const uint16_t*>(k_rope), rope_stride};
  uint8_t* dst = static_cast<uint8_t*>(kv_cache);
  if (kv_dtype == NSA_KV_FP8_656)
    hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3((unsigned)blocks),
                       dim3(kThreads), 0, (hipStream_t)stream, src, (int64_t)n,
                       cache_loc, num_slots, dst);
  else
    hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, src, (int64_t)n, cache_loc, num_slots, dst);
  return nsa::check_launch(fn);
}
