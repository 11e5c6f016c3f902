"""Pins for the fp64 oracle, on the CPU.

Each pin checks the oracle against something other than itself: an
independent pure-Python brute force, closed forms derived by hand
(``tests/golden``), and invariants of softmax attention.  The mutation tests
at the end plant plausible mistakes in copies of the oracle (dropped scale,
top-left causal alignment, wrong GQA head map, excluded own key, transposed
value read, missing max subtraction) and check that some pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import brute
from paged_kv_attention_append_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Pin functions, parameterised by the attention_seq implementation under test.
# ----------------------------------------------------------------------------
def pin_closed_forms(attn_seq):
    cases = json.load(open(os.path.join(GOLD, "closed_forms.json")))["cases"]
    for c in cases:
        q = np.array(c["q"], np.float64)
        k = np.array(c["k"], np.float64)
        v = np.array(c["v"], np.float64)
        scale = c.get("scale")
        out = attn_seq(q, k, v, scale)
        exp = np.array(c.get("expected_prefill", c.get("expected_decode")), np.float64)
        assert np.max(np.abs(out - exp)) <= c["tolerance"], c["name"]


def pin_onehot_causal(attn_seq):
    """q = 0 gives uniform weights over visible keys; one-hot V rows expose the
    visible set: o[j] = 1/(p+1) for j <= p, else 0 (bottom-right aligned)."""
    for kv_len, q_len in [(7, 7), (9, 3), (6, 1)]:
        d = kv_len
        q = np.zeros((q_len, 1, d))
        k = np.random.default_rng(0).standard_normal((kv_len, 1, d))
        v = np.eye(kv_len)[:, None, :]
        out = attn_seq(q, k, v, None)
        for i in range(q_len):
            p = kv_len - q_len + i
            exp = np.where(np.arange(kv_len) <= p, 1.0 / (p + 1), 0.0)
            assert np.max(np.abs(out[i, 0] - exp)) <= 1e-14


def pin_gqa_constant_values(attn_seq):
    """Every V row of KV head g equal to c_g gives o = c_{h // (Hq/Hkv)} exactly."""
    rng = np.random.default_rng(1)
    hq, hkv, d, kv = 8, 2, 4, 5
    c = np.array([[1.0, 2.0, 3.0, 4.0], [-5.0, 6.0, -7.0, 8.0]])
    v = np.broadcast_to(c[None], (kv, hkv, d)).copy()
    k = rng.standard_normal((kv, hkv, d))
    q = rng.standard_normal((kv, hq, d))
    out = attn_seq(q, k, v, None)
    for h in range(hq):
        assert np.max(np.abs(out[:, h] - c[h // (hq // hkv)])) <= 1e-12


def pin_brute_force(attn_seq):
    rng = np.random.default_rng(2)
    for hq, hkv, d, kv, ql in [(2, 2, 8, 6, 6), (4, 2, 8, 9, 3), (4, 1, 4, 5, 1), (2, 2, 16, 17, 17)]:
        q = rng.standard_normal((ql, hq, d))
        k = rng.standard_normal((kv, hkv, d)) * 2.0
        v = rng.standard_normal((kv, hkv, d))
        got = attn_seq(q, k, v, None)
        ref = np.array(brute.brute_sequence(q.tolist(), k.tolist(), v.tolist()))
        assert np.max(np.abs(got - ref)) <= 1e-12


def pin_large_scores(attn_seq):
    """Scores near 700 overflow exp() unless the row max is subtracted."""
    q = np.array([[[30.0, 0.0]]])
    k = np.array([[[47.0, 0.0]], [[46.0, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    out = attn_seq(q, k, v, 1.0)        # scores 1410, 1380 -> weights 1/(1+e^-30), ...
    w1 = 1.0 / (1.0 + math.exp(-30.0))
    assert np.all(np.isfinite(out))
    assert abs(out[0, 0, 0] - w1) <= 1e-12 and abs(out[0, 0, 1] - (1 - w1)) <= 1e-12


PINS = [pin_closed_forms, pin_onehot_causal, pin_gqa_constant_values, pin_brute_force, pin_large_scores]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    pin(A.attention_seq)


# ----------------------------------------------------------------------------
# Invariants (P2-P8, P13, P14).
# ----------------------------------------------------------------------------
def test_one_key_returns_v_exactly():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 3, 8))
    k = rng.standard_normal((1, 3, 8))
    v = rng.standard_normal((1, 3, 8))
    assert np.array_equal(A.attention_seq(q, k, v), v)


def test_weights_sum_to_one():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((12, 16)) * 3
    v = rng.standard_normal((12, 16))
    _, w = A.attend_rows(q, k, v, np.array([0, 3, 7, 11, 11]), 0.25, return_weights=True)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(w[0, 1:] == 0.0) and np.all(w[1, 4:] == 0.0)


def test_zero_query_gives_mean():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((10, 2, 8))
    v = rng.standard_normal((10, 2, 8))
    out = A.attention_seq(np.zeros((10, 2, 8)), k, v)
    for p in range(10):
        assert np.max(np.abs(out[p] - v[: p + 1].mean(axis=0))) <= 1e-13


def test_equal_values_pass_through():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((9, 1, 8))
    row = rng.standard_normal(8)
    v = np.broadcast_to(row, (9, 1, 8)).copy()
    out = A.attention_seq(rng.standard_normal((9, 1, 8)), k, v)
    assert np.max(np.abs(out - row)) <= 1e-13


def test_key_shift_invariance():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((6, 2, 16))
    k = rng.standard_normal((6, 2, 16))
    v = rng.standard_normal((6, 2, 16))
    u = rng.standard_normal((1, 2, 16))
    a = A.attention_seq(q, k, v)
    b = A.attention_seq(q, k + u, v)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_hard_attention_limit():
    rng = np.random.default_rng(8)
    d = 64
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((20, 1, d))
    v = rng.standard_normal((20, 1, d))
    j = 13
    k[j, 0] = 50.0 * math.sqrt(d) * q[0, 0] / np.linalg.norm(q[0, 0])
    out = A.attention_seq(q, k, v)
    assert np.max(np.abs(out[0, 0] - v[j, 0])) <= 1e-12


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((40, 4, 16))
    k = rng.standard_normal((40, 2, 16))
    v = rng.standard_normal((40, 2, 16))
    full = A.attention_seq(q, k, v)
    dec = A.attention_seq(q[-1:], k, v)
    assert np.max(np.abs(full[-1:] - dec)) <= 1e-13
    chunk = A.attention_seq(q[25:], k, v)           # a chunk on 25 cached tokens
    assert np.max(np.abs(full[25:] - chunk)) <= 1e-13


def test_future_keys_do_not_leak():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((12, 2, 8))
    k = rng.standard_normal((12, 2, 8))
    v = rng.standard_normal((12, 2, 8))
    a = A.attention_seq(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[7:] += 100.0
    v2[7:] = -v2[7:]
    b = A.attention_seq(q, k2, v2)
    assert np.array_equal(a[:7], b[:7])


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((7, 8, 16))
    k = rng.standard_normal((7, 2, 16))
    v = rng.standard_normal((7, 2, 16))
    a = A.attention_seq(q, k, v)
    b = A.attention_seq(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.max(np.abs(a - b)) <= 1e-14


def test_batch_permutation_permutes_outputs():
    step = W.random_step(12, W.F32, 4, 2, 16, [9, 3, 17, 1], [9, 3, 17, 1])
    out = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    perm = [2, 0, 3, 1]
    out_p = A.attention_ragged([step.q[i] for i in perm], [step.k_ctx[i] for i in perm],
                               [step.v_ctx[i] for i in perm])
    cu = step.cu_q_lens
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in perm])
    assert np.array_equal(out[rows], out_p)


def test_prefill_varlen_splits_sequences():
    step = W.random_step(13, W.F32, 2, 2, 8, [4, 6], [4, 6])
    q = step.packed_q()
    k, v = step.new_kv()
    a = A.prefill_varlen(q, k, v, step.cu_q_lens)
    b = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    assert np.array_equal(a, b)
    # Attending across the sequence boundary would change the second prompt's rows.
    c = A.attention_seq(q, k, v)
    assert np.max(np.abs(c[4:] - a[4:])) > 1e-3


def test_tiny_fp32_brute_force():
    """The tiny ragged fp32 workload, prefill then decode, against brute force."""
    pre, dec = W.tiny_fp32(1)
    got = A.attention_ragged(pre.q, pre.k_ctx, pre.v_ctx)
    ref = np.concatenate([np.array(brute.brute_sequence(pre.q[s].tolist(), pre.k_ctx[s].tolist(),
                                                        pre.v_ctx[s].tolist()))
                          for s in range(pre.num_seqs)])
    assert np.max(np.abs(got - ref)) <= 1e-12
    got = A.attention_ragged(dec.q, dec.k_ctx, dec.v_ctx)
    ref = np.concatenate([np.array(brute.brute_sequence(dec.q[s].tolist(), dec.k_ctx[s].tolist(),
                                                        dec.v_ctx[s].tolist()))
                          for s in range(dec.num_seqs)])
    assert np.max(np.abs(got - ref)) <= 1e-12


# ----------------------------------------------------------------------------
# Mutation tests: a planted mistake in a copy of the oracle must fail a pin.
# ----------------------------------------------------------------------------
def _mutant(scale_fn=None, causal_offset=0, head_map=None, transpose_v=False, no_max=False):
    def attend(q, k, v, positions, scale):
        z = (q @ k.T) * scale
        vis = np.arange(k.shape[0])[None, :] <= positions[:, None] + causal_offset
        z = np.where(vis, z, -np.inf)
        e = np.exp(z) if no_max else np.exp(z - z.max(axis=1, keepdims=True))
        w = e / e.sum(axis=1, keepdims=True)
        vv = v[:, ::-1] if transpose_v else v
        return w @ vv

    def attn_seq(q_seq, k_seq, v_seq, scale=None):
        q_len, hq, d = q_seq.shape
        kv_len, hkv, _ = k_seq.shape
        scale = (scale_fn(d) if scale_fn else 1.0 / math.sqrt(d)) if scale is None else scale
        pos = np.arange(kv_len - q_len, kv_len)
        pos = pos if head_map != "top_left" else np.arange(q_len)
        out = np.empty((q_len, hq, d))
        for h in range(hq):
            g = head_map(h, hq, hkv) if callable(head_map) else h // (hq // hkv)
            out[:, h] = attend(q_seq[:, h], k_seq[:, g], v_seq[:, g], pos, scale)
        return out
    return attn_seq


MUTANTS = {
    "dropped_scale": _mutant(scale_fn=lambda d: 1.0),
    "excludes_own_key": _mutant(causal_offset=-1),
    "sees_one_future_key": _mutant(causal_offset=+1),
    "top_left_causal": _mutant(head_map="top_left"),
    "gqa_modulo_map": _mutant(head_map=lambda h, hq, hkv: h % hkv),
    "reversed_value_dims": _mutant(transpose_v=True),
    "no_max_subtraction": _mutant(no_max=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mutant = MUTANTS[name]
    caught = 0
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught += 1
    assert caught >= 1, f"no pin catches mutant {name}"
