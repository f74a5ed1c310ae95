"""Pins of the oracle's number formats and packed layout against library
routines and exact rational arithmetic."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_neighbours(x: float):
    """Exact bf16 grid neighbours of x via integer arithmetic on Fractions."""
    fx = Fraction(x)
    if fx == 0:
        return fx, fx
    m, e = np.frexp(x)
    q = Fraction(2) ** int(max(e - 8, -133))
    lo = (fx / q).__floor__() * q
    return lo, lo + q


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0, -3.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.bf16_rne(x.astype(np.float64)), ref)


def test_bf16_exact_rounding_rational():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(300) * np.exp(rng.uniform(-10, 10, 300)))
    # exact ties: a bf16 value plus half a quantum
    for base in [1.0, 1.0078125, 3.0, -5.03125, 1e-3]:
        b = float(F.bf16_rne(base))
        _, e = np.frexp(b)
        xs.append(b + 2.0 ** (e - 9))
    for x in xs:
        got = Fraction(float(F.bf16_rne(x)))
        lo, hi = _bf16_neighbours(x)
        fx = Fraction(x)
        if fx - lo < hi - fx:
            want = lo
        elif fx - lo > hi - fx:
            want = hi
        else:  # tie: even last mantissa bit
            q = hi - lo
            want = lo if (lo / q) % 2 == 0 else hi
        assert got == want, x


def test_fp16_up_div_is_smallest_cover():
    rng = np.random.default_rng(2)
    xs = np.abs(rng.standard_normal(3000) * np.exp(rng.uniform(-25, 9, 3000)))
    for m in (3.0, 127.0):
        # include exact multiples m*h of fp16 values and zero
        hs = np.abs(rng.standard_normal(200)).astype(np.float16).astype(np.float64)
        x = np.concatenate([xs, m * hs, [0.0]])
        h, sat = F.fp16_up_div(x, m)
        assert not sat.any()
        for xi, hi in zip(x, h):
            h16 = np.float16(hi)
            assert float(h16) == hi                      # an fp16 value
            assert Fraction(m) * Fraction(hi) >= Fraction(xi)
            if hi > 0:
                prev = float(np.nextafter(h16, np.float16(0)))
                assert Fraction(m) * Fraction(prev) < Fraction(xi)


def test_fp16_up_div_saturates():
    h, sat = F.fp16_up_div(np.array([3 * 65504.0, 3 * 65504.0 + 1.0, 1e9]), 3.0)
    assert list(sat) == [False, True, True]
    assert np.all(h == 65504.0)


def test_rne_quotient_matches_fraction_round():
    rng = np.random.default_rng(3)
    b = np.abs(rng.standard_normal(2000)).astype(np.float16).astype(np.float64) + 2.0 ** -14
    n = rng.integers(-130, 130, 2000)
    # exact half-way points, points just off them, and generic values
    a = np.concatenate([(n + 0.5) * b, (n - 0.5) * b, np.nextafter((n + 0.5) * b, np.inf),
                        np.nextafter((n + 0.5) * b, -np.inf), rng.standard_normal(2000) * 50 * b])
    bb = np.concatenate([b, b, b, b, b])
    got = F.rne_quotient(a, bb)
    for ai, bi, gi in zip(a, bb, got):
        assert round(Fraction(ai) / Fraction(bi)) == int(gi)   # Python rounds half to even


def test_pack_codes_layout():
    q = np.zeros((2, 128), np.uint8)
    q[0, :4] = [0, 1, 2, 3]
    q[1, 4:8] = [3, 3, 3, 3]
    b = F.pack_codes(q)
    assert b.shape == (2, 32)
    assert b[0, 0] == 0b11100100 and b[1, 1] == 0xFF and b[1, 0] == 0
    rng = np.random.default_rng(4)
    q = rng.integers(0, 4, (37, 128)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_codes(F.pack_codes(q), 128), q)


def test_pack_zeros_layout():
    z = np.array([[1, 2], [3, 0], [2, 2]], np.uint8)
    b = F.pack_zeros(z)
    # token 0 nibble = 1 | 2<<2 = 9 (low), token 1 nibble = 3 (high), token 2 = 10 (low)
    assert list(b) == [9 | (3 << 4), 10]
    rng = np.random.default_rng(5)
    for T in (1, 2, 63, 64, 101):
        z = rng.integers(0, 4, (T, 2)).astype(np.uint8)
        np.testing.assert_array_equal(F.unpack_zeros(F.pack_zeros(z), T), z)


def test_fp16_bits_roundtrip_and_golden():
    g = json.load(open(os.path.join(GOLD, "qsac_tiny.json")))["cases"][0]
    np.testing.assert_array_equal(F.fp16_bits(np.array(g["qsac_scale"])), g["qsac_scale_bits"])
    np.testing.assert_array_equal(F.fp16_bits(np.array(g["nearest_scale"])), g["nearest_scale_bits"])
