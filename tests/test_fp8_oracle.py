"""Pins of the fp8 (OCP E4M3) oracle, independent of its implementation:
hand-derived codes and dequantized values, the format's value table built another way, exact round
trips, brute-force nearest-with-ties-to-even, saturation and the scale."""
import json
import math
import os

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


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_dequant.json")


def _dequant_matches_golden(fn) -> bool:
    """True when ``fn(codes, scale)`` gives every hand-derived value of the
    fixture exactly (sign of zero included; NaN stays NaN)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = float(np.asarray(fn(np.array([c["code"]]), c["scale"])).ravel()[0])
        want = c["expected"]
        if want is None:
            if not math.isnan(got):
                return False
        elif got != want or math.copysign(1.0, got) != math.copysign(1.0, want):
            return False
    return True


def test_dequantize_hand_derived_values():
    """Codes times non-unit scales, each product worked out by hand from the
    code's sign, exponent and mantissa fields (tests/golden/fp8_dequant.json)."""
    assert _dequant_matches_golden(fp8.dequantize)


def test_dequantize_planted_mistakes_are_caught():
    """Plausible mistakes in dequantize each fail the hand-derived values."""
    mutants = {
        "divides by the scale": lambda c, s: fp8.decode(c) / s,
        "scales the raw code": lambda c, s: s * np.asarray(c, np.float64),
        "drops the sign": lambda c, s: s * np.abs(fp8.decode(c)),
        "ignores the scale": lambda c, s: fp8.decode(c),
        "subnormals as normals": lambda c, s: s * np.where((np.asarray(c) & 0x78) == 0,
                                                             (1 + (np.asarray(c) & 7) / 8.0) * 2.0 ** -6
                                                             * np.where(np.asarray(c) >> 7, -1, 1),
                                                             fp8.decode(c)),
    }
    for name, fn in mutants.items():
        assert not _dequant_matches_golden(fn), name
