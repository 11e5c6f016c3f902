"""Pins of the fp8 (OCP E4M3) oracle, independent of its implementation:
hand-derived codes, the format's value table built another way, exact round
trips, brute-force nearest-with-ties-to-even, saturation and the scale."""
import math

import numpy as np

from oracle import fp8


def test_hand_derived_codes():
    cases = [(1.0, 0x38), (448.0, 0x7E), (500.0, 0x7E), (-500.0, 0xFE), (2.0 ** -9, 0x01),
             (1.0625, 0x38),          # tie between 0x38 (1.0) and 0x39 (1.125): even code
             (1.1875, 0x3A),          # tie between 0x39 and 0x3A (1.25): even code
             (3.0, 0x44), (-1.0, 0xB8), (0.0, 0x00), (2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01),
             (2.0 ** -6, 0x08), (240.0, 0x77)]
    x = np.array([c[0] for c in cases], np.float32)
    assert [int(b) for b in fp8.quantize(x, 1.0)] == [c[1] for c in cases]


def test_decode_matches_the_format_table():
    """Every code against a value built from sign, exponent and mantissa with math.ldexp."""
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = fp8.decode(np.array([c]))[0]
        if e == 15 and m == 7:
            assert math.isnan(v)
            continue
        ref = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
        assert v == (-ref if s else ref), c


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = fp8.decode(codes).astype(np.float32)
    assert np.array_equal(fp8.quantize(vals, 1.0), codes.astype(np.uint8))


def test_nearest_with_ties_to_even_by_brute_force():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(300) * 10, rng.standard_normal(100) * 0.01,
                        (np.arange(1, 120) / 8.0)]).astype(np.float32)   # many exact ties
    q = fp8.quantize(x, 1.0)
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for xi, qi in zip(x.astype(np.float64), q):
        d = {c: abs(xi - fp8.decode(np.array([c]))[0]) for c in finite}
        best = min(d.values())
        cands = [c for c, v in d.items() if v == best]
        if len(cands) > 1:   # a tie: the even code (one with the same sign as x when the value is 0)
            cands = [c for c in cands if c % 2 == 0 and (c >> 7) == (1 if xi < 0 else 0)]
        assert int(qi) in cands, (xi, qi, cands)


def test_saturation_and_scale():
    x = np.array([1e6, -1e6, 0.3, -7.5], np.float32)
    assert list(fp8.quantize(x, 1.0)[:2]) == [0x7E, 0xFE]
    s = 0.0625                                          # a power of two: scaling is exact
    q = fp8.quantize(x[2:] * np.float32(1 / s) * np.float32(s), s)
    assert np.array_equal(q, fp8.quantize(x[2:] / np.float32(s), 1.0))
    assert np.allclose(fp8.dequantize(q, s), fp8.decode(q) * s)
