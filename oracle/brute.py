"""Pure-Python scalar brute force of causal attention, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It exists to pin
``oracle.attention`` with code that shares nothing with it: nested loops over
Python floats, ``math.exp`` and ``math.fsum``; no NumPy arithmetic.  Same
definition as ``oracle.attention``: row ``i`` of a sequence with ``kv_len``
keys and ``q_len`` new rows sits at position ``kv_len - q_len + i`` and sees
keys ``0..that position``; query head ``h`` reads KV head ``h // (Hq/Hkv)``.
"""
from __future__ import annotations

import math


def brute_sequence(q, k, v, scale=None):
    """``q``: nested lists [q_len][Hq][d]; ``k, v``: [kv_len][Hkv][d]. Returns [q_len][Hq][d]."""
    q_len = len(q)
    kv_len = len(k)
    hq = len(q[0]) if q_len else 0
    hkv = len(k[0]) if kv_len else 0
    d = len(k[0][0]) if kv_len else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = []
    for i in range(q_len):
        pos = kv_len - q_len + i
        row = []
        for h in range(hq):
            g = (h * hkv) // hq
            scores = []
            for j in range(pos + 1):
                dot = math.fsum(float(q[i][h][x]) * float(k[j][g][x]) for x in range(d))
                scores.append(dot * scale)
            top = max(scores)
            ws = [math.exp(s - top) for s in scores]
            total = math.fsum(ws)
            vec = []
            for x in range(d):
                vec.append(math.fsum(ws[j] * float(v[j][g][x]) for j in range(pos + 1)) / total)
            row.append(vec)
        out.append(row)
    return out
