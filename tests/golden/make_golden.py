"""Writes the hand-derived fixtures in this folder.

Every expected value below is derived by hand in the ``derivation`` text next
to it (closed forms of softmax attention, the pool layout formula stated in
``include/pka.h`` applied by hand, the slot of a position in a block-table
row, and rotary-embedding rotations worked out
for one or two pairs, fp8 codes times a scale; ``math.cos`` / ``math.sin`` only evaluate the angles
named there).  Nothing here calls the HIP library or
the oracle.  Run from the repository root: ``python tests/golden/make_golden.py``.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def closed_forms():
    two_key = {
        "name": "two_key_ln3",
        "derivation": "d=4 so scale=1/2; q=[1,0,0,0], k0=0, k1=[2ln3,0,0,0] give scaled scores 0 and ln3, "
                      "softmax weights 1/4 and 3/4; o = v0/4 + 3 v1/4 = [1,3,4,1]; the first prompt row sees "
                      "only key 0 so o = v0.",
        "q": [[[1.0, 0.0, 0.0, 0.0]], [[1.0, 0.0, 0.0, 0.0]]],
        "k": [[[0.0, 0.0, 0.0, 0.0]], [[2.0 * math.log(3.0), 0.0, 0.0, 0.0]]],
        "v": [[[4.0, 0.0, -8.0, 1.0]], [[0.0, 4.0, 8.0, 1.0]]],
        "expected_prefill": [[[4.0, 0.0, -8.0, 1.0]], [[1.0, 3.0, 4.0, 1.0]]],
        "tolerance": 1e-12,
    }
    three_key = {
        "name": "three_key_scale1",
        "derivation": "scale=1; q=[ln2, ln4]; keys [1,0],[0,1],[0,0] give scores ln2, ln4, 0, exp-weights "
                      "2,4,1 over 7; v rows [7,0],[0,7],[14,14] give o = [14+14, 28+14]/7 = [4,6] for the "
                      "decode row (position 2).",
        "scale": 1.0,
        "q": [[[math.log(2.0), math.log(4.0)]]],
        "k": [[[1.0, 0.0]], [[0.0, 1.0]], [[0.0, 0.0]]],
        "v": [[[7.0, 0.0]], [[0.0, 7.0]], [[14.0, 14.0]]],
        "expected_decode": [[[4.0, 6.0]]],
        "tolerance": 1e-12,
    }
    return {"citation": "Closed forms of softmax attention; no page prints a worked example.",
            "cases": [two_key, three_key]}


def pool_layout():
    # Both pools: element (b, g, t, i) at ((b*Hkv + g)*16 + t)*d + i.
    # bf16, Hkv=2, d=16:
    #   slot 17 -> b=1, t=1; g=1, i=9 -> ((1*2+1)*16+1)*16+9 = 49*16+9 = 793
    #   slot 0, g=0, i=0             -> 0
    #   slot 15 (b=0, t=15), g=0, i=7 -> 15*16+7 = 247;   i=8 -> 248
    #   slot 16 (b=1, t=0), g=0, i=0  -> (2*16+0)*16 = 512 (block 1 starts after 2 heads x 16 rows)
    # fp32, Hkv=1, d=8:
    #   slot 33 -> b=2, t=1; g=0, i=5 -> ((2*1+0)*16+1)*8+5 = 33*8+5 = 269
    return {
        "derivation": "Each entry applies the documented formula by hand: K and V element (b, g, t, i) at "
                      "((b*Hkv+g)*16+t)*d+i, b = slot//16, t = slot%16.",
        "cases": [
            {"elem_bytes": 2, "hkv": 2, "d": 16, "slot": 17, "g": 1, "i": 9, "k": 793, "v": 793},
            {"elem_bytes": 2, "hkv": 2, "d": 16, "slot": 0, "g": 0, "i": 0, "k": 0, "v": 0},
            {"elem_bytes": 2, "hkv": 2, "d": 16, "slot": 15, "g": 0, "i": 7, "k": 247, "v": 247},
            {"elem_bytes": 2, "hkv": 2, "d": 16, "slot": 15, "g": 0, "i": 8, "k": 248, "v": 248},
            {"elem_bytes": 2, "hkv": 2, "d": 16, "slot": 16, "g": 0, "i": 0, "k": 512, "v": 512},
            {"elem_bytes": 4, "hkv": 1, "d": 8, "slot": 33, "g": 0, "i": 5, "k": 269, "v": 269},
        ],
    }


def rope_cases():
    """Rotary embedding worked by hand.  Pair j of a d-dim row rotates by pos * theta_j,
    theta_j = base^(-2j/d); (a, b) -> (a cos - b sin, a sin + b cos)."""
    c1, s1 = math.cos(1.0), math.sin(1.0)
    c3, s3 = math.cos(3.0), math.sin(3.0)
    cases = [
        {"name": "d2_unit_a", "d": 2, "base": 10000.0, "style": 0, "pos": 1, "x": [1.0, 0.0],
         "derivation": "d=2: one pair, theta_0 = base^0 = 1, angle 1: (1,0) -> (cos 1, sin 1)",
         "expected": [c1, s1]},
        {"name": "d2_unit_b", "d": 2, "base": 10000.0, "style": 1, "pos": 1, "x": [0.0, 1.0],
         "derivation": "d=2, angle 1: (0,1) -> (-sin 1, cos 1); both pairings agree at d=2",
         "expected": [-s1, c1]},
        {"name": "d2_pos3", "d": 2, "base": 500.0, "style": 0, "pos": 3, "x": [2.0, 1.0],
         "derivation": "angle 3: (2,1) -> (2 cos 3 - sin 3, 2 sin 3 + cos 3)",
         "expected": [2 * c3 - s3, 2 * s3 + c3]},
        {"name": "d2_negative_pos", "d": 2, "base": 10000.0, "style": 0, "pos": -1, "x": [1.0, 0.0],
         "derivation": "angle -1: (1,0) -> (cos 1, -sin 1)",
         "expected": [c1, -s1]},
        {"name": "d4_half_second_pair", "d": 4, "base": 100.0, "style": 0, "pos": 10, "x": [0.0, 1.0, 0.0, 0.0],
         "derivation": "d=4, base 100: theta = (1, 100^(-1/2) = 0.1); half pairing: pair 1 = dims (1, 3); "
                       "pos 10 gives angle 1 on pair 1: e1 -> cos 1 e1 + sin 1 e3",
         "expected": [0.0, c1, 0.0, s1]},
        {"name": "d4_interleaved_second_pair", "d": 4, "base": 100.0, "style": 1, "pos": 10,
         "x": [0.0, 0.0, 1.0, 0.0],
         "derivation": "interleaved pairing: pair 1 = dims (2, 3), angle 10 * 0.1 = 1: e2 -> cos 1 e2 + sin 1 e3",
         "expected": [0.0, 0.0, c1, s1]},
        {"name": "d4_half_first_pair", "d": 4, "base": 100.0, "style": 0, "pos": 1, "x": [0.0, 0.0, 1.0, 0.0],
         "derivation": "half pairing: pair 0 = dims (0, 2), angle 1 * 1: e2 is its b -> -sin 1 e0 + cos 1 e2",
         "expected": [-s1, 0.0, c1, 0.0]},
    ]
    freqs = {"d": 8, "base": 10000.0, "derivation": "10000^(-2j/8) = 10^(-j)",
             "expected": [1.0, 0.1, 0.01, 0.001]}
    return {"cases": cases, "frequencies": freqs, "tolerance": 1e-13}


def slots():
    # Slot of position p in a sequence whose block-table row is [5, 2, 7, 0]:
    # row[p // 16] * 16 + p % 16.
    #   p = 0, 1, 15  -> block 5: 80, 81, 95
    #   p = 16, 17, 31 -> block 2: 32, 33, 47
    #   p = 32, 47     -> block 7: 112, 127
    #   p = 48, 63     -> block 0: 0, 15
    return {
        "derivation": "slot = row[p // 16] * 16 + p % 16 applied by hand to the row [5, 2, 7, 0] (the slot "
                      "definition stated in include/pka.h; the pages give no worked example).",
        "row": [5, 2, 7, 0],
        "positions": [0, 1, 15, 16, 17, 31, 32, 47, 48, 63],
        "expected": [80, 81, 95, 32, 33, 47, 112, 127, 0, 15],
    }


def fp8_dequant():
    """E4M3 codes times a per-head scale, worked by hand from the code's fields
    (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent
    field 0 is subnormal, m * 2^-9; S.1111.111 is NaN).  Scales are chosen so
    every product is exact in binary64."""
    cases = [
        {"code": 0x38, "scale": 0.5, "expected": 0.5,
         "derivation": "0 0111 000: e=7, m=0 -> 1.0 * 2^(7-7) = 1; times 0.5 = 0.5"},
        {"code": 0x7E, "scale": 3.0, "expected": 1344.0,
         "derivation": "0 1111 110: e=15, m=6 -> 1.75 * 2^8 = 448 (largest finite); times 3 = 1344"},
        {"code": 0x01, "scale": 2.0 ** -4, "expected": 2.0 ** -13,
         "derivation": "0 0000 001: subnormal, 1 * 2^-9; times 2^-4 = 2^-13"},
        {"code": 0xB8, "scale": 0.75, "expected": -0.75,
         "derivation": "1 0111 000: sign set, 1.0; times 0.75 = -0.75"},
        {"code": 0x44, "scale": 0.375, "expected": 1.125,
         "derivation": "0 1000 100: e=8, m=4 -> 1.5 * 2 = 3; times 0.375 = 1.125"},
        {"code": 0x0F, "scale": 4.0, "expected": 0.1171875,
         "derivation": "0 0001 111: e=1, m=7 -> 1.875 * 2^-6 = 0.029296875; times 4 = 0.1171875"},
        {"code": 0xFE, "scale": 2.5, "expected": -1120.0,
         "derivation": "1 1111 110: -448; times 2.5 = -1120"},
        {"code": 0x06, "scale": 8.0, "expected": 0.09375,
         "derivation": "0 0000 110: subnormal, 6 * 2^-9 = 0.01171875; times 8 = 0.09375"},
        {"code": 0x80, "scale": 5.0, "expected": -0.0,
         "derivation": "1 0000 000: negative zero; times 5 = -0"},
        {"code": 0x7F, "scale": 2.0, "expected": None,
         "derivation": "0 1111 111: NaN; any scale keeps it NaN (null here)"},
    ]
    return {"citation": "OCP 8-bit floating point E4M3 format (the fp8 cache reading; the pages name an fp8 "
                        "option without its encoding).", "cases": cases}


if __name__ == "__main__":
    with open(os.path.join(HERE, "slots.json"), "w") as f:
        json.dump(slots(), f, indent=1)
    with open(os.path.join(HERE, "rope.json"), "w") as f:
        json.dump(rope_cases(), f, indent=1)
    with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
        json.dump(closed_forms(), f, indent=1)
    with open(os.path.join(HERE, "pool_layout.json"), "w") as f:
        json.dump(pool_layout(), f, indent=1)
    with open(os.path.join(HERE, "fp8_dequant.json"), "w") as f:
        json.dump(fp8_dequant(), f, indent=1)
