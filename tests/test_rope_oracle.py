"""Pins for the rotary-embedding oracle (oracle/rope.py), on the CPU.

Hand-worked rotations (tests/golden/rope.json) fix the sign convention, the
pairing of dims and the frequency schedule; the invariants (identity at
position 0, norm of every pair, dependence of q.k on the position difference
only, composition, inverse, the permutation linking the two pairings) hold
for any correct implementation.  The mutation tests plant plausible mistakes
in copies of the oracle and check that some pin catches each.
"""
import json
import os

import numpy as np
import pytest

from oracle import rope as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def pin_golden(rope_fn, freq_fn):
    g = json.load(open(os.path.join(GOLD, "rope.json")))
    for c in g["cases"]:
        x = np.array(c["x"], np.float64)[None, None, :]
        y = rope_fn(x, np.array([c["pos"]]), c["base"], c["style"])[0, 0]
        assert np.max(np.abs(y - np.array(c["expected"]))) <= g["tolerance"], c["name"]
    f = g["frequencies"]
    assert np.max(np.abs(freq_fn(f["d"], f["base"]) - np.array(f["expected"]))) <= 1e-15


def pin_invariants(rope_fn):
    rng = np.random.default_rng(3)
    for d in (2, 8, 64, 128):
        for style in (R.HALF, R.INTERLEAVED):
            x = rng.standard_normal((5, 3, d))
            pos = np.array([0, 1, 17, 4095, 32767])
            y = rope_fn(x, pos, 10000.0, style)
            assert np.array_equal(y[0], x[0])                        # position 0 is the identity
            a, b = R.pair_dims(d, style)
            assert np.allclose(y[..., a] ** 2 + y[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-12)
            # q . k depends on the position difference only
            q, k = rng.standard_normal((1, 2, d)), rng.standard_normal((1, 2, d))
            for m, n in ((7, 3), (100, 96), (2000, 1996)):
                lhs = np.sum(rope_fn(q, [m], 500.0, style) * rope_fn(k, [n], 500.0, style), axis=-1)
                rhs = np.sum(rope_fn(q, [m - n], 500.0, style) * k, axis=-1)
                assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
            # composition and inverse
            z = rope_fn(rope_fn(x, pos, 10000.0, style), np.array([3, 5, 7, 11, 13]), 10000.0, style)
            assert np.allclose(z, rope_fn(x, pos + np.array([3, 5, 7, 11, 13]), 10000.0, style), atol=1e-9)
            assert np.allclose(rope_fn(y, -pos, 10000.0, style), x, atol=1e-9)


def pin_pairings_related(rope_fn):
    """Interleaved pairing = half pairing on dims permuted (2j, 2j+1) -> (j, j + d/2)."""
    rng = np.random.default_rng(4)
    d = 16
    perm = np.empty(d, np.int64)
    perm[np.arange(d // 2)] = 2 * np.arange(d // 2)
    perm[d // 2 + np.arange(d // 2)] = 2 * np.arange(d // 2) + 1
    x = rng.standard_normal((3, 2, d))
    pos = np.array([1, 9, 300])
    y_int = rope_fn(x, pos, 1000.0, R.INTERLEAVED)
    y_half = rope_fn(x[..., perm], pos, 1000.0, R.HALF)
    assert np.allclose(y_int[..., perm], y_half, atol=1e-12)


def test_golden_rotations():
    pin_golden(R.rope, R.frequencies)


def test_invariants():
    pin_invariants(R.rope)


def test_pairings_related():
    pin_pairings_related(R.rope)


# ----------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# ----------------------------------------------------------------------------
def _variant(freq=None, sign=1.0, pairing=None, swap_out=False):
    def fn(x, positions, base, style):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        a, b = (pairing or R.pair_dims)(d, style)
        th = (freq or R.frequencies)(d, base)
        phi = np.asarray(positions, np.float64)[:, None] * th[None, :]
        c, s = np.cos(phi)[:, None, :], sign * np.sin(phi)[:, None, :]
        y = np.empty_like(x)
        ya = x[..., a] * c - x[..., b] * s
        yb = x[..., a] * s + x[..., b] * c
        y[..., a], y[..., b] = (yb, ya) if swap_out else (ya, yb)
        return y
    return fn


MUTANTS = {
    "frequency without the factor 2": dict(freq=lambda d, base: np.float64(base) ** (-np.arange(d // 2) / d)),
    "sine with the wrong sign": dict(sign=-1.0),
    "half pairing taken as (j, j + 1)": dict(pairing=lambda d, st: (np.arange(d // 2), np.arange(d // 2) + 1)
                                           if st == R.HALF else R.pair_dims(d, st)),
    "interleaved pairing taken as half": dict(pairing=lambda d, st: R.pair_dims(d, R.HALF)),
    "outputs of a pair swapped": dict(swap_out=True),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutants_are_caught(name):
    fn = _variant(**MUTANTS[name])
    freq = MUTANTS[name].get("freq", R.frequencies)
    caught = 0
    for pin in (lambda: pin_golden(fn, freq), lambda: pin_invariants(fn), lambda: pin_pairings_related(fn)):
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught >= 1, name
