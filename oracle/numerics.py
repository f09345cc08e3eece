"""Number formats used by the layer, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16: 1 sign, 8 exponent, 7 fraction bits, the top half of an IEEE binary32;
rounding is to nearest, ties to even.

E4M3 and E8M0 follow the OCP 8-bit floating point and OCP Microscaling (MX)
v1.0 specifications, which the pages name only as "MXFP8" (bigchange.ai pt-BR,
"Três números, três denominadores"):
  E4M3 ("FN" flavour): exponent bias 7, no infinities, S.1111.111 is NaN,
       largest finite 448 = 1.75 * 2^8, subnormals m * 2^-9 (m = 1..7).
  E8M0: an unsigned biased exponent, value 2^(code - 127), code 0xFF is NaN.
  MX block: 32 elements share one E8M0 scale X; elements are stored as
       E4M3 of v / 2^X.
Readings where the MX specification leaves a choice (recorded once here):
  * X = floor(log2(max|v|)) - 8 (8 is the E4M3 largest normal exponent),
    clamped to [-127, 127]; an all-zero block takes X = -127 (code 0).
  * elements are rounded to nearest-even and saturated to +-448; the sign of
    a value that rounds to zero is kept (code 0x80 for negative ones).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.ldexp(255.0, 120))      # (2 - 2^-7) * 2^127
E4M3_MAX = 448.0
MX_BLOCK = 32


# ----------------------------------------------------------------------------- bf16
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    A finite value a = r * 2^q with an integer r of at most 8 significant bits;
    q = exponent(a) - 7 for normal results and -133 below 2^-126 (bf16
    subnormals share binary32's exponent range)."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                       # a = m * 2^e, 0.5 <= |m| < 1
    q = np.where(e - 1 >= -126, e - 8, -133)
    r = np.rint(np.ldexp(a, -q))             # numpy rint: half to even
    out = np.ldexp(r, q)
    out = np.where(np.abs(out) > BF16_MAX, np.copysign(np.inf, a), out)
    return np.where(np.isfinite(a), out, a)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round to bf16 and return the bit patterns (uint16)."""
    v = round_bf16(a).astype(np.float32)     # exact: bf16 is a subset of binary32
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(a) -> np.ndarray:
    """Round float64 values to binary32 (nearest-even), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def storer(dtype: str):
    """The rounding applied when a tensor is written in the layer's storage
    type: 'bf16', 'f32', or 'f64' (no rounding, for exact algebraic checks)."""
    if dtype == "bf16" or dtype == "mxfp8":
        return round_bf16
    if dtype == "f32":
        return round_f32
    if dtype == "f64":
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- E4M3
def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) from its sign, exponent and fraction fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m.astype(np.float64), -9)
    v = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_encode(v) -> np.ndarray:
    """Round float64 values to E4M3 codes: nearest-even, saturating at 448,
    keeping the sign bit (also for results that round to zero)."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, e = np.frexp(a)                       # a = m * 2^e
    q = np.maximum(e - 1, -6) - 3            # quantum: 2^(exp-3), subnormal 2^-9
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E4M3_MAX)
    # encode the rounded magnitude
    _, er = np.frexp(r)
    is_norm = r >= 2.0 ** -6
    exp_field = np.where(is_norm, er - 1 + 7, 0)
    man = np.where(is_norm, np.ldexp(r, -(er - 1)) * 8.0 - 8.0, np.ldexp(r, 9))
    code = (exp_field.astype(np.int64) << 3) | np.rint(man).astype(np.int64)
    code = np.where(r == 0, 0, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


# ----------------------------------------------------------------------------- MX
def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent X of a block from its largest magnitude (see the reading
    in the module docstring)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    x = np.where(amax > 0, (e - 1) - 8, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def mx_quantize(v: np.ndarray):
    """MX-quantise a 2-D array in blocks of 32 along its last axis.

    A trailing partial block is treated as if padded with zeros (which cannot
    change its largest magnitude). Returns (codes uint8 [rows, K],
    scales uint8 [rows, ceil(K/32)])."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    nb = -(-K // MX_BLOCK)
    pad = np.zeros((rows, nb * MX_BLOCK))
    pad[:, :K] = v
    blocks = pad.reshape(rows, nb, MX_BLOCK)
    x = mx_scale_exponent(np.max(np.abs(blocks), axis=2))        # [rows, nb]
    codes = e4m3_encode(np.ldexp(blocks, -x[:, :, None]))
    return codes.reshape(rows, nb * MX_BLOCK)[:, :K], (x + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Float64 values of MX-quantised data (blocks of 32 along the last axis)."""
    rows, K = codes.shape
    x = scales.astype(np.int64) - 127
    xs = np.repeat(x, MX_BLOCK, axis=1)[:, :K]
    return np.ldexp(e4m3_decode(codes), xs)


def mx_roundtrip(v: np.ndarray) -> np.ndarray:
    """The values an MX-quantised operand carries into a GEMM."""
    return mx_dequantize(*mx_quantize(v))
