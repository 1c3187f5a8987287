// Internal helpers shared by the library's translation units: status and
// last-error handling, host-side argument checks, small device utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <cstdarg>
#include <cstdio>

#include "nsa.h"

namespace nsa {

// Records a formatted message as this thread's last error and returns code.
int set_error(int code, const char* fmt, ...);
// Clears this thread's last error and returns NSA_OK.
int ok();

// Translates the result of the launch just issued into a status.
inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(NSA_ERR_LAUNCH, "%s: launch failed: %s", what,
                     hipGetErrorString(e));
  return ok();
}

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace nsa

// ---- device-side error word -----------------------------------------------
// Ids the host cannot see (page ids, slots, request indices, pool rows) are
// checked in the kernels; an out-of-range one is treated as absent and its
// NSA_DEVERR_* bit is OR-ed into a word in device memory with a vector
// atomic. The library is built without relocatable device code, so every
// translation unit has its own word; each unit registers a reader at load
// time and nsa_check_device_errors() combines (and clears) them all.
static __device__ uint32_t nsa_device_error_word;

__device__ __forceinline__ void flag_device_error(uint32_t bits) {
  atomicOr(&nsa_device_error_word, bits);
}

namespace nsa {
typedef int (*ErrorReader)(hipStream_t, uint32_t*);
// Adds a reader to the library's list; returns its index.
int register_error_reader(ErrorReader f);
}  // namespace nsa

// Reads and clears this unit's word on the current device (synchronises s).
static int nsa_take_unit_errors(hipStream_t s, uint32_t* bits) {
  uint32_t v = 0;
  const uint32_t zero = 0;
  if (hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(nsa_device_error_word), sizeof(v), 0,
                               hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return -1;
  if (v != 0 && (hipMemcpyToSymbolAsync(HIP_SYMBOL(nsa_device_error_word), &zero,
                                        sizeof(zero), 0, hipMemcpyHostToDevice, s) != hipSuccess ||
                 hipStreamSynchronize(s) != hipSuccess))
    return -1;
  *bits = v;
  return 0;
}
__attribute__((used)) static const int nsa_unit_reader_index =
    nsa::register_error_reader(nsa_take_unit_errors);

#define NSA_REQUIRE(cond, code, ...)              \
  do {                                            \
    if (!(cond)) return nsa::set_error(code, __VA_ARGS__); \
  } while (0)

// ---- device helpers --------------------------------------------------------

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Packs two floats into one dword of two bfloat16 (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Order-preserving image of a float in uint32: NaN ranks lowest and -0.0
// equals +0.0 (so equal values tie and are broken by position). The top-k
// histograms count its top 12 bits (kKeyBins bins).
constexpr int kKeyBins = 4096;
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = x == 0.0f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Same packing in one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
