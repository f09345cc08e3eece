// MXFP8 element and block encoders shared by the quantiser (mx_quant.hip) and
// the grouped-GEMM epilogues that quantise their outputs (gemm_epilogue.h).
// The format follows the public OCP Microscaling Formats v1.0 specification
// (the pages name MXFP8 only: bigchange.ai pt-BR, "Três números, três
// denominadores"): blocks of 32 values share the scale 2^X with
// X = floor(log2 amax) - 8, clamped to [-127, 127] (X = -127 for an all-zero
// block); elements are v * 2^-X rounded to nearest-even E4M3, saturated to
// +-448, sign kept. Inputs are finite bf16 values.
#pragma once

#include "common.h"

namespace moe {

constexpr float kE4M3Max = 448.0f;

// Block scale exponent from the largest magnitude of the block (a
// non-negative binary32 value that is a bf16 value): the biased exponent
// field gives floor(log2 amax) for normal values; subnormal and zero amax
// clamp to -127 either way.
MOE_DEV int mx_exponent(float amax) {
  const int x = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
  return x < -127 ? -127 : x;
}

// 2^n as binary32 for -126 <= n <= 127.
MOE_DEV float pow2(int n) { return __uint_as_float(static_cast<uint32_t>(n + 127) << 23); }

// Four E4M3 bytes (v0 lowest) of v * 2^-X, inv = 2^-X. v * inv is exact (a
// power-of-two scaling of a bf16 value) unless it falls below binary32's
// normal range, where it rounds to zero in E4M3 anyway. The clamp to +-448
// is the format's saturation (values from 448 up round to 448, never to
// NaN); the conversion itself is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3,
// round to nearest even, subnormals, sign of zero kept).
MOE_DEV uint32_t e4m3_word(float v0, float v1, float v2, float v3, float inv) {
  auto sat = [&](float v) { return __builtin_amdgcn_fmed3f(v * inv, -kE4M3Max, kE4M3Max); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v0), sat(v1), 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(sat(v2), sat(v3), lo, true));
}

// Codes of one 32-value block (bytes of two 16-byte words) and its scale code.
MOE_DEV uint32_t quantize_block(const float (&v)[32], V16 (&out)[2]) {
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(v[r]));
  const int x = mx_exponent(amax);
  const float inv = pow2(-x);
#pragma unroll
  for (int w = 0; w < 8; ++w)
    out[w >> 2].w[w & 3] = e4m3_word(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3], inv);
  return static_cast<uint32_t>(x + 127);
}

}  // namespace moe
