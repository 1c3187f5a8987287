// a6: bf16 latent cache -> fp8 e4m3fn block-scaled cache (656 bytes / slot).
//
// "nsa_backend.py (EngineX-Hygon sglang fork)", _forward_flashmla_decode, and
// "dsa_backend.py (sglang main)", _forward_flashmla_kv, call
// quantize_k_cache(kv_cache) to produce the fp8 cache the sparse decode reads.
// The byte layout and rounding (not on the pages) are the reading stated in
// nsa.h: 512 codes in 4 blocks of 128, 4 fp32 scales amax/448, 64 bf16 rope.
//
// One wave per slot: lane l owns no-rope elements 8l..8l+7 (block l/16), so a
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

__global__ void __launch_bounds__(kThreads)
quantize_k_cache_kernel(const uint16_t* __restrict__ kv, int64_t num_slots,
                        int64_t in_stride, uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t slot = (int64_t)blockIdx.x * kSlotsPerBlock + (threadIdx.x >> 6);
  if (slot >= num_slots) return;
  const uint16_t* row = kv + slot * in_stride;
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
  reinterpret_cast<uint16_t*>(orow + 528)[lane] = row[512 + lane];
}

}  // namespace

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
  hipLaunchKernelGGL(quantize_k_cache_kernel, dim3((unsigned)blocks),
                     dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(kv_bf16), num_slots,
                     in_stride, static_cast<uint8_t*>(out));
  return nsa::check_launch(fn);
}
