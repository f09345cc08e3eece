"""Pins of the oracle's number formats against things other than itself:
torch's own bf16 / float8 casts (independent library code), the OCP format
tables written out by hand, and exhaustive sweeps of every bit pattern."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.numerics import (
    bf16_bits_to_f64, e4m3_decode, e4m3_encode, f64_to_bf16_bits, mx_dequantize,
    mx_quantize, mx_scale_exponent, round_bf16,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse(s):
    s = s.strip()
    if s == "nan":
        return float("nan")
    if s == "-0":
        return -0.0
    if "^" in s:
        coef = 1.0
        if "*" in s:
            c, s = s.split("*")
            coef = float(c)
        b, e = s.split("^")
        return coef * float(b) ** int(e)
    return float(s)


def test_bf16_round_matches_torch_on_random_f32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f.astype(np.float64))
    # torch rounds huge finite values to inf exactly like round-to-nearest-even does
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even_and_subnormals():
    one = 1.0
    ulp = 2.0 ** -7
    assert round_bf16(one + ulp / 2) == one                      # tie -> even (1.0)
    assert round_bf16(one + 3 * ulp / 2) == one + 2 * ulp        # tie -> even (up)
    assert round_bf16(one + ulp / 2 + 2.0 ** -30) == one + ulp   # above tie
    sub = 2.0 ** -133
    assert round_bf16(sub * 0.5) == 0.0                          # tie -> even (0)
    assert round_bf16(sub * 0.75) == sub
    assert round_bf16(-0.0) == 0.0 and np.signbit(round_bf16(-0.0))
    assert math.isinf(round_bf16(2.0 ** 128))


def test_bf16_decode_every_pattern_matches_torch():
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    got = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    # and bits -> value -> bits round-trips for every non-NaN pattern
    keep = ~np.isnan(got)
    assert np.array_equal(f64_to_bf16_bits(got[keep]), bits[keep])


def test_e4m3_table_values():
    tab = json.load(open(os.path.join(GOLDEN, "ocp_formats.json")))
    for code, val in tab["e4m3"]:
        v = e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = _parse(val)
        if math.isnan(want):
            assert math.isnan(v), code
        else:
            assert v == want and np.signbit(v) == np.signbit(want), code


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("scale_exp", [-8, -3, 0, 5, 20, -20])
def test_e4m3_encode_every_bf16_pattern_matches_torch(scale_exp):
    """All 65,536 bf16 patterns, scaled by a power of two, rounded to E4M3:
    inside +-448 the codes must equal torch's nearest-even cast bit for bit;
    beyond it the oracle saturates to +-448."""
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    v = v[np.isfinite(v)]
    v = np.ldexp(v, scale_exp)
    got = e4m3_encode(v)
    inside = np.abs(v) <= 448.0
    ref = torch.from_numpy(v[inside].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # ldexp of a bf16 value by a power of two is exact in float32 unless it underflows
    # below 2^-149, where both sides give a signed zero
    assert np.array_equal(got[inside], ref)
    out = ~inside
    assert np.all(e4m3_decode(got[out]) == np.copysign(448.0, v[out]))


def test_e4m3_encode_roundtrips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    keep = ~np.isnan(vals)
    assert np.array_equal(e4m3_encode(vals[keep]), codes[keep])


def test_mx_golden_blocks():
    tab = json.load(open(os.path.join(GOLDEN, "ocp_formats.json")))
    for case in tab["mx_blocks"]["cases"]:
        block = np.full(32, case["rest"])
        head = case["block_head"]
        block[:len(head)] = head
        codes, scales = mx_quantize(block[None, :])
        assert scales[0, 0] == case["scale_code"]
        assert [int(c) for c in codes[0, :len(head)]] == [int(c, 16) for c in case["codes_head"]]


def test_mx_scale_exact_for_powers_of_two():
    for p in range(-100, 100, 7):
        assert mx_scale_exponent(2.0 ** p) == max(p - 8, -127)
        assert mx_scale_exponent(2.0 ** p * 1.999) == max(p - 8, -127)
    assert mx_scale_exponent(0.0) == -127


def test_mx_blocks_restart_and_partial_block():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((3, 70))
    v[1, 64:] = 0.0
    codes, scales = mx_quantize(v)
    assert codes.shape == (3, 70) and scales.shape == (3, 3)
    for r in range(3):
        for b in range(3):
            blk = v[r, 32 * b: 32 * b + 32]
            c2, s2 = mx_quantize(blk[None, :])
            assert s2[0, 0] == scales[r, b]
            assert np.array_equal(c2[0], codes[r, 32 * b: 32 * b + 32])
    assert scales[1, 2] == 0


def test_mx_small_integers_are_exact():
    """Integers of magnitude <= 16 in a block whose largest is a power of two
    fit E4M3 after scaling, so MX dequantisation returns them exactly and an
    MX product equals the plain integer product."""
    rng = np.random.default_rng(2)
    a = rng.integers(-16, 17, size=(5, 64)).astype(np.float64)
    b = rng.integers(-16, 17, size=(7, 64)).astype(np.float64)
    a[:, ::32] = 16.0
    b[:, ::32] = 16.0
    qa = mx_dequantize(*mx_quantize(a))
    qb = mx_dequantize(*mx_quantize(b))
    assert np.array_equal(qa, a) and np.array_equal(qb, b)
    assert np.array_equal(qa @ qb.T, (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64))


def test_mx_error_bound():
    """Within the non-saturating range each element is within half an E4M3
    quantum (2^-4 relative for normals, 2^(X-10) absolute for subnormals)."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 32)) * np.exp(rng.uniform(-5, 5, size=(64, 1)))
    codes, scales = mx_quantize(v)
    q = mx_dequantize(codes, scales)
    X = scales.astype(np.int64) - 127
    scaled = np.abs(v) * 2.0 ** (-X)
    sat = scaled > 448
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** (X - 10))
    assert np.all(np.abs(q - v)[~sat] <= bound[~sat] * (1 + 1e-12))
