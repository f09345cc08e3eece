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

// ---------------------------------------------------------------- packed bf16
// The quantiser works on words holding two bf16 values (low half first) and
// never widens them to binary32: the block maximum comes from packed 16-bit
// integer maxima of the magnitudes (for finite non-negative bf16 values the
// order of the bit patterns is the order of the values), saturation is a
// packed integer clamp of the magnitudes, and gfx950's scaled conversion
// v_cvt_scalef32_pk_fp8_bf16 turns two values into two E4M3 bytes. That
// instruction divides by 2^e, e the unbiased exponent field of its binary32
// scale operand (a subnormal operand counts as 2^-127), exactly, then rounds
// to nearest even with subnormals and the sign of zero kept; magnitudes from
// 464 up become NaN, which the clamp before it rules out (values in
// (448, 464] round to 448 either way, so clamping them to 448 changes no code).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short cvt16x2 __attribute__((ext_vector_type(2)));

// Packed maximum of two words of non-negative bf16 patterns.
MOE_DEV uint32_t max2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
// Running maximum of the magnitudes of the two values of w.
MOE_DEV uint32_t mag_max2(uint32_t acc, uint32_t w) { return max2(acc, w & 0x7fff7fffu); }
// The larger half of a word of two magnitudes.
MOE_DEV uint32_t max_half(uint32_t m) { return max(m & 0xffffu, m >> 16); }

// X from the bf16 pattern of a block's largest magnitude: its biased
// exponent field gives floor(log2 amax) for normal values; subnormal and zero
// maxima clamp to -127 either way.
MOE_DEV int mx_exponent_bf16(uint32_t amax) {
  const int x = static_cast<int>(amax >> 7) - 127 - 8;
  return x < -127 ? -127 : x;
}
// Both halves: the bf16 pattern of 448 * 2^X (1.75 * 2^(X+8); X + 8 + 127 is
// in [8, 254] for X in [-127, 119], the range a finite bf16 block gives).
MOE_DEV uint32_t sat_limit(int x) { return static_cast<uint32_t>(x + 135) << 7 | 0x60u; }
// Scale operand of the conversion for 2^X: exponent field X + 127 (a
// subnormal for X = -127); the low mantissa bit set keeps it non-zero.
MOE_DEV float cvt_scale(int x) { return __uint_as_float(static_cast<uint32_t>(x + 127) << 23 | 0x400000u); }

// Clamp both values of w to +-lim (lim2: the magnitude pattern in both
// halves). Negative values are the patterns from 0x8000 up, so an unsigned
// minimum against lim | 0x8000 clamps them and leaves positive ones alone;
// as signed 16-bit integers negative values are below every positive limit,
// so a signed minimum against lim then clamps the positive ones.
MOE_DEV uint32_t sat2(uint32_t w, uint32_t lim2) {
  const u16x2 a = __builtin_elementwise_min(__builtin_bit_cast(u16x2, w), __builtin_bit_cast(u16x2, lim2 | 0x80008000u));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2, a),
                                                                __builtin_bit_cast(i16x2, lim2)));
}

// Four E4M3 bytes (lowest from the low half of w01) of saturated values.
MOE_DEV uint32_t e4m3_quad(uint32_t w01, uint32_t w23, float scale) {
  cvt16x2 o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(bf16x2, w01), scale, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(bf16x2, w23), scale, true);
  return __builtin_bit_cast(uint32_t, o);
}

// Scale state of one block from its packed magnitude maximum.
struct BlockScale {
  int x;          // X
  uint32_t lim2;  // saturation limit, both halves
  float scale;    // conversion operand
};
MOE_DEV BlockScale block_scale(uint32_t amax) {
  BlockScale b;
  b.x = mx_exponent_bf16(amax);
  b.lim2 = sat_limit(b.x) * 0x10001u;
  b.scale = cvt_scale(b.x);
  return b;
}
// Four codes of words w01, w23 under block scale b.
MOE_DEV uint32_t encode_quad(uint32_t w01, uint32_t w23, const BlockScale& b) {
  return e4m3_quad(sat2(w01, b.lim2), sat2(w23, b.lim2), b.scale);
}

// Codes of one 32-value block given as 16 words (bytes of two 16-byte words)
// and its scale code.
MOE_DEV uint32_t quantize_block_bf16(const uint32_t* w, V16 (&out)[2]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = mag_max2(m, w[i]);
  const BlockScale b = block_scale(max_half(m));
#pragma unroll
  for (int q = 0; q < 8; ++q) out[q >> 2].w[q & 3] = encode_quad(w[2 * q], w[2 * q + 1], b);
  return static_cast<uint32_t>(b.x + 127);
}

}  // namespace moe
