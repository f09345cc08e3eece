// Shared device helpers and host-side argument checks of libmoe (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
// bf16 values travel as raw 16-bit patterns; arithmetic is binary32.
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// binary32 -> bf16 by gfx950's v_cvt_pk_bf16_f32: round to nearest even,
// subnormals kept, a NaN becomes the quiet NaN (bits >> 16) | 0x40. Checked
// on the device against that rule written out in integer arithmetic, for
// every one of the 2^32 binary32 patterns: no difference.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

MOE_DEV uint16_t f32_to_bf16(float f) { return static_cast<uint16_t>(pack_bf16x2(f, 0.0f)); }

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static MOE_DEV float load(const float* p, size_t i) { return p[i]; }
  static MOE_DEV void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static MOE_DEV float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static MOE_DEV void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 16-byte vectors: 8 bf16 or 4 binary32 elements.
struct alignas(16) V16 { uint32_t w[4]; };

MOE_DEV void unpack(const V16& v, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(v.w[i] << 16);
    o[2 * i + 1] = __uint_as_float(v.w[i] & 0xffff0000u);
  }
}
MOE_DEV void unpack(const V16& v, float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v.w[i]);
}
MOE_DEV V16 pack(const float (&o)[8]) {
  V16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
  return v;
}
MOE_DEV V16 pack(const float (&o)[4]) {
  V16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = __float_as_uint(o[i]);
  return v;
}

// V16 that is v when ok, else zero (word by word: a select of whole vectors
// can be compiled through scratch memory)
MOE_DEV V16 keep_if(bool ok, const V16& v) {
  V16 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.w[i] = ok ? v.w[i] : 0u;
  return o;
}

// Elements per 16-byte vector.
template <typename T> constexpr int kVec = 16 / sizeof(T);

MOE_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }
MOE_DEV float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Wave-wide sum (fixed butterfly order: deterministic).
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace moe

// ------------------------------------------------------------------ host checks
namespace moe {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
inline size_t dtype_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe

#define MOE_CHECK_ARG(cond)                    \
  do {                                         \
    if (!(cond)) return MOE_ERR_INVALID_ARG;   \
  } while (0)
#define MOE_CHECK_SUPPORTED(cond)              \
  do {                                         \
    if (!(cond)) return MOE_ERR_UNSUPPORTED;   \
  } while (0)
