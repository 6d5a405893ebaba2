"""Pins for the oracle's rounding helpers, E2M1 element coding and FP4 groups.

Each check ties the oracle to something other than itself: library
conversions (torch bf16, numpy fp16), the E2M1 bit definition, hand-derived
encodings, a second rounding algorithm (fp32 division + piecewise
round-half-even), lossless grids and invariants.
"""

import numpy as np
import pytest
import torch

from oracle import e2m1
from oracle import formats as F
from oracle.numerics import (bf16_bits, bf16_from_bits, fp16_bits, round_bf16,
                             round_fp16)


def _all_bf16_finite():
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(20000) * 1e38).astype(np.float32)]).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x)
    np.testing.assert_array_equal(got, ref)


def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 10, rng.standard_normal(20000) * 1e-6,
                        np.array([65504.0, 65519.0, 65520.0, 2.0 ** -25, 3 * 2.0 ** -25])])
    ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(round_fp16(x), ref)


def test_e2m1_values_from_bit_definition(golden):
    # sign | e1 e0 | m with bias 1; exponent 0 is subnormal (m * 0.5)
    def from_bits(n):
        s, e, m = (n >> 3) & 1, (n >> 1) & 3, n & 1
        mag = m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
        return -mag if s else mag
    table = {int(n): float(v) for n, v in golden("e2m1_values.txt")}
    for n in range(16):
        want = from_bits(n)
        got = e2m1.decode(np.array([n], np.uint8))[0]
        assert got == want and (np.signbit(got) == np.signbit(want))
        if n < 8:
            assert table[n] == want


def test_e2m1_hand_cases(golden):
    for x, s, nib in golden("e2m1_encode_cases.txt"):
        got = int(e2m1.encode(np.array([float(x)]), float(s))[0])
        assert got == int(nib), (x, s, nib, got)


def _e2m1_by_division(x, s):
    """Second algorithm: q = fl32(|x| / s), then round-half-even on the E2M1 grid piecewise."""
    q = (np.abs(x).astype(np.float32) / np.float32(s)).astype(np.float64)
    v = np.where(q < 2.0, np.rint(q * 2.0) / 2.0,
                 np.where(q < 4.0, np.rint(q), np.rint(q / 2.0) * 2.0))
    v = np.minimum(v, 6.0)
    idx = np.searchsorted(e2m1.MAGNITUDES, v)
    return ((np.signbit(x).astype(np.uint8) << 3) | idx).astype(np.uint8)


@pytest.mark.parametrize("s_bits", [0x3F80, 0x3E4D, 0x3FC0, 0x4120, 0x3B80, 0x0F80, 0x42F7])
def test_e2m1_all_bf16_inputs_vs_division(s_bits):
    s = float(bf16_from_bits(np.array([s_bits], np.uint16))[0])
    x = _all_bf16_finite()
    x = x[np.abs(x) <= 8 * s]
    got = e2m1.encode(x, s)
    want = _e2m1_by_division(x, s)
    np.testing.assert_array_equal(got, want)


def test_e2m1_encode_error_and_monotone():
    s = 0.375
    x = np.linspace(-3, 3, 20001)
    nib = e2m1.encode(x, s)
    rec = e2m1.decode(nib) * s
    # nearest: error at most half the local spacing (0.25 s below 2s, 0.5 s below 4s, 1 s above)
    bound = np.where(np.abs(x) < 2 * s, 0.25 * s, np.where(np.abs(x) < 4 * s, 0.5 * s, 1.0 * s))
    assert np.all(np.abs(rec - np.clip(x, -6 * s, 6 * s)) <= bound + 1e-15)
    assert np.all(np.diff(rec) >= 0)


def test_fp4_group_scale_and_lossless_grid():
    rng = np.random.default_rng(3)
    # lossless: values on s * E2M1 with the group max at 6 s and s bf16
    s = round_bf16(np.abs(rng.standard_normal((64, 8))) + 0.01)
    idx = rng.integers(0, 8, size=(64, 8, 16))
    idx[..., 3] = 7
    sign = rng.integers(0, 2, size=idx.shape)
    x = np.where(sign, -1.0, 1.0) * e2m1.MAGNITUDES[idx] * s[..., None]
    x = x.reshape(64, 128)
    codes, sc = F.fp4_encode(x)
    np.testing.assert_array_equal(bf16_from_bits(sc), s)
    np.testing.assert_array_equal(F.fp4_decode(codes, sc), x)
    # the group's largest magnitude always codes to the top value
    y = round_bf16(rng.standard_normal((500, 128)) * 3)
    c2, s2 = F.fp4_encode(y)
    nib = F.unpack_nibbles(c2).reshape(500, 8, 16)
    am = np.abs(y.reshape(500, 8, 16)).argmax(-1)
    np.testing.assert_array_equal(np.take_along_axis(nib & 7, am[..., None], -1)[..., 0], 7)


def test_fp4_zero_group_and_scale_dtype():
    x = np.zeros((1, 32))
    x[0, 16:] = round_bf16(np.linspace(-1, 1, 16))
    c, s = F.fp4_encode(x)
    assert c[0, :8].tolist() == [0] * 8 and s[0, 0] == 0
    assert bf16_from_bits(s)[0, 1] == round_bf16(1.0 / 6.0)


def test_nibble_bit_order():
    # channel 2j in the low nibble of byte j
    nib = np.array([[1, 2, 15, 0]], np.uint8)
    assert F.pack_nibbles(nib).tolist() == [[0x21, 0x0F]]
    c = np.array([[1, 2, 3, 0, 3, 3, 3, 3]], np.uint8)
    assert F.pack_2bit(c).tolist() == [[0b00111001, 0xFF]]
    b = np.array([[1, 0, 0, 0, 0, 0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0]], np.uint8)
    assert F.pack_bits(b).tolist() == [[0x81, 0x02]]
    rng = np.random.default_rng(4)
    z = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_nibbles(F.pack_nibbles(z)), z)
    z = rng.integers(0, 4, (5, 64)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_2bit(F.pack_2bit(z)), z)
    z = rng.integers(0, 2, (5, 64)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_bits(F.pack_bits(z)), z)


def test_bits_helpers_roundtrip():
    x = round_bf16(np.array([1.5, -2.25, 3e-20, 0.0]))
    np.testing.assert_array_equal(bf16_from_bits(bf16_bits(x)), x)
    assert bf16_bits(np.array([1.0]))[0] == 0x3F80
    assert fp16_bits(np.array([1.0]))[0] == 0x3C00
