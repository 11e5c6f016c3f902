"""CPU tests of the pool-layout oracle (append/gather), bf16 rounding and the
seeded workload generator."""
import json
import os

import numpy as np
import pytest

from oracle import paged_layout as L
from paged_kv_attention_append_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_layout_formula_matches_hand_derived_offsets():
    g = json.load(open(os.path.join(GOLD, "pool_layout.json")))
    for c in g["cases"]:
        b, t = c["slot"] // 16, c["slot"] % 16
        assert L.k_index(b, c["g"], t, c["i"], c["hkv"], c["d"]) == c["k"]
        assert L.v_index(b, c["g"], t, c["i"], c["hkv"], c["d"]) == c["v"]


@pytest.mark.parametrize("elem", [np.uint16, np.uint32])
@pytest.mark.parametrize("hkv,d", [(1, 64), (2, 128), (3, 64)])
def test_layout_is_a_bijection(elem, hkv, d):
    nb = 3
    n = nb * hkv * 16 * d
    b, g, t, i = np.meshgrid(np.arange(nb), np.arange(hkv), np.arange(16), np.arange(d), indexing="ij")
    ki = L.k_index(b, g, t, i, hkv, d).ravel()
    vi = L.v_index(b, g, t, i, hkv, d).ravel()
    assert np.array_equal(np.sort(ki), np.arange(n))
    assert np.array_equal(np.sort(vi), np.arange(n))
    # every (block, head) tile is one contiguous run of 16*d elements
    for kk in (ki, vi):
        tiles = kk.reshape(nb, hkv, -1)
        assert np.all(tiles.max(axis=2) - tiles.min(axis=2) == 16 * d - 1)


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_append_round_trip_and_sentinels(dtype):
    step = W.random_step(21, dtype, 4, 2, 64, [5, 17, 33, 1], [5, 2, 1, 1])
    hkv, d = step.num_kv_heads, step.head_dim
    if dtype == W.BF16:
        to_bits = lambda a: W.bf16_bits(a)
        sentinel, et = np.uint16(0x7FC0), np.uint16
    else:
        to_bits = lambda a: np.ascontiguousarray(a, np.float32).view(np.uint32)
        sentinel, et = np.uint32(0x7FC00000), np.uint32
    n = step.num_blocks * hkv * 16 * d
    kp = np.full(n, sentinel, et)
    vp = np.full(n, sentinel, et)
    kc, vc = step.cached_kv()
    kp, vp = L.append(kp, vp, to_bits(kc), to_bits(vc), step.cached_slot_mapping(), hkv, d)
    kn, vn = step.new_kv()
    kp, vp = L.append(kp, vp, to_bits(kn), to_bits(vn), step.new_slot_mapping(), hkv, d)
    for s in range(step.num_seqs):
        kg, vg = L.gather(kp, vp, step.block_tables[s], int(step.kv_lens[s]), hkv, d)
        assert np.array_equal(kg, to_bits(step.k_ctx[s]))
        assert np.array_equal(vg, to_bits(step.v_ctx[s]))
    slots = np.concatenate([step.cached_slot_mapping(), step.new_slot_mapping()])
    km, vm = L.written_mask(step.num_blocks, slots, hkv, d)
    assert np.all(kp[~km] == sentinel) and np.all(vp[~vm] == sentinel)
    assert km.sum() == vm.sum() == int(step.kv_lens.sum()) * hkv * d


def test_append_skips_negative_slots():
    kp = np.zeros(2 * 16 * 8, np.uint32)
    vp = np.zeros_like(kp)
    new = np.arange(3 * 1 * 8, dtype=np.uint32).reshape(3, 1, 8) + 1
    kp2, vp2 = L.append(kp, vp, new, new, np.array([3, -1, 20]), 1, 8)
    km, _ = L.written_mask(2, np.array([3, 20]), 1, 8)
    assert np.all(kp2[~km] == 0) and km.sum() == 16


def test_bf16_rounding_golden():
    g = json.load(open(os.path.join(GOLD, "bf16_rounding.json")))
    for c in g["cases"]:
        f = np.array([int(c["f32_bits"], 16)], np.uint32).view(np.float32)
        assert int(W.bf16_bits(f)[0]) == int(c["bf16_bits"], 16), c["note"]


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    ours = W.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_generator_is_deterministic():
    a = W.random_step(5, W.BF16, 4, 2, 64, [20, 40], [20, 1])
    b = W.random_step(5, W.BF16, 4, 2, 64, [20, 40], [20, 1])
    assert np.array_equal(a.block_tables, b.block_tables)
    for x, y in zip(a.k_ctx + a.v_ctx + a.q, b.k_ctx + b.v_ctx + b.q):
        assert np.array_equal(x, y)


def _check_tables(step):
    used = []
    for s in range(step.num_seqs):
        nb = (int(step.kv_lens[s]) + 15) // 16
        row = step.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < step.num_blocks)
        assert np.all(row[nb:] == -1)
        used.extend(row[:nb].tolist())
    assert len(used) == len(set(used)), "a block is shared by two sequences"


def test_workload_shapes():
    pre, dec = W.tiny_fp32(1)
    assert list(pre.kv_lens) == [5, 17, 32, 64] and pre.total_q == 118
    assert list(dec.kv_lens) == [6, 18, 33, 65] and dec.total_q == 4
    assert np.array_equal(pre.block_tables, dec.block_tables)
    _check_tables(dec)
    used_prefill = sum((l + 15) // 16 for l in pre.kv_lens)
    assert used_prefill == 9
    # prefill blocks come first from the permutation, decode blocks after them
    pre_blocks = set(dec.block_tables[s][i] for s in range(4) for i in range((int(pre.kv_lens[s]) + 15) // 16))
    assert len(pre_blocks) == 9
    for s in range(4):
        np.testing.assert_array_equal(pre.k_ctx[s], dec.k_ctx[s][:-1])
    p = W.prefill_ragged(3)
    assert p.total_q == 4096 and np.all(p.q_lens == p.kv_lens)
    assert np.all(p.kv_lens[:-1] >= 16) and np.all(p.kv_lens <= 1024)
    _check_tables(p)
    assert p.new_slot_mapping().shape == (4096,)
    assert len(set(p.new_slot_mapping().tolist())) == 4096


def test_mixed_and_decode_workload_structure():
    m = W.mixed_gqa(4)
    assert m.num_seqs == 130 and m.total_q == 128 + 2048
    assert np.all(m.kv_lens[:128] >= 256) and np.all(m.kv_lens[:128] <= 2048)
    assert np.all(m.kv_lens[128:] == 2048) and np.all(m.q_lens[128:] == 1024)
    _check_tables(m)
    d = W.decode_mha_7b(2)
    assert d.num_seqs == 64 and np.all(d.q_lens == 1)
    assert d.num_q_heads == d.num_kv_heads == 32 and abs(d.sigma - 0.5) < 1e-12
    _check_tables(d)


def test_copy_blocks_moves_every_token_of_each_block():
    """Block copy pinned through the (already pinned) gather: for each pair,
    the destination block read through a one-block table equals the source
    block read the same way, token by token; every other destination block
    keeps its sentinel; out-of-range pairs do nothing."""
    hkv, d, nb_src, nb_dst = 3, 8, 6, 5
    rng = np.random.default_rng(9)
    ks = rng.integers(0, 2**16, nb_src * hkv * 16 * d, dtype=np.uint16)
    vs = rng.integers(0, 2**16, nb_src * hkv * 16 * d, dtype=np.uint16)
    kd = np.full(nb_dst * hkv * 16 * d, 0xABCD, np.uint16)
    vd = np.full(nb_dst * hkv * 16 * d, 0x1234, np.uint16)
    pairs = np.array([[4, 0], [1, 3], [7, 1], [2, -1], [5, 2]], np.int32)   # [7, 1], [2, -1] out of range
    k2, v2 = L.copy_blocks(ks, vs, kd, vd, pairs, hkv, d, nb_src, nb_dst)
    for sb, db in [(4, 0), (1, 3), (5, 2)]:
        a = L.gather(ks, vs, np.array([sb]), 16, hkv, d)
        b = L.gather(k2, v2, np.array([db]), 16, hkv, d)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for db in (1, 4):
        b = L.gather(k2, v2, np.array([db]), 16, hkv, d)
        assert (b[0] == 0xABCD).all() and (b[1] == 0x1234).all()
    # the copy touches exactly the three destination blocks' elements
    changed = np.flatnonzero(k2 != kd)
    tile = hkv * 16 * d
    assert set(np.unique(changed // tile)) <= {0, 2, 3}


def test_copy_blocks_within_one_pool_is_copy_on_write():
    """Copying inside one pool: the destinations become the sources' contents,
    the sources are unchanged (a shared prefix block duplicated before a
    sequence writes into it)."""
    hkv, d, nb = 2, 4, 4
    rng = np.random.default_rng(10)
    k = rng.integers(0, 2**32, nb * hkv * 16 * d, dtype=np.uint32)
    v = rng.integers(0, 2**32, nb * hkv * 16 * d, dtype=np.uint32)
    k2, v2 = L.copy_blocks(k, v, k, v, np.array([[0, 3], [1, 2]]), hkv, d, nb, nb)
    tile = hkv * 16 * d
    assert np.array_equal(k2[3 * tile:4 * tile], k[0:tile]) and np.array_equal(v2[2 * tile:3 * tile], v[tile:2 * tile])
    assert np.array_equal(k2[:2 * tile], k[:2 * tile]) and np.array_equal(v2[:2 * tile], v[:2 * tile])


def test_f16_rounding_matches_hand_derived_bits():
    """IEEE binary16 nearest-even: hand-derived patterns, including a tie that
    rounds to even, the largest finite value and the smallest subnormal."""
    cases = [(1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (2.0 ** -24, 0x0001),
             (1.0 + 2.0 ** -11, 0x3C00),            # tie: 1.0 (even) wins over 1 + 2^-10
             (1.0 + 3 * 2.0 ** -11, 0x3C02),        # tie: 1 + 2^-9 (even) wins over 1 + 2^-10
             (1.0 / 3.0, 0x3555), (0.1, 0x2E66)]
    x = np.array([c[0] for c in cases], np.float32)
    assert [int(b) for b in W.f16_bits(x)] == [c[1] for c in cases]
    r = W.round_to_dtype(x, W.F16)
    assert np.array_equal(W.f16_bits(r), W.f16_bits(x))
