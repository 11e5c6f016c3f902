"""Block copy between paged pools (pka_kv_copy_blocks), bit for bit against
the oracle's copy_blocks: copy-on-write inside one device pool, swap out to a
pinned host pool and back, fp32 / d = 64, out-of-range pairs, attention
through copied blocks, and rejection of a pageable host pool on the host."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import paged_layout as L
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, pool_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def random_cache(num_blocks, hkv, d, dtype, seed, pinned_host=False):
    """A cache whose pools hold random raw bits (NaN patterns included: the copy moves bits)."""
    rng = np.random.default_rng(seed)
    n = num_blocks * hkv * 16 * d
    c = pka.KVCache.allocate(num_blocks, hkv, d, dtype, pinned_host=pinned_host)
    if dtype == torch.bfloat16:
        kb = rng.integers(0, 2**16, n, dtype=np.uint16).view(np.int16)
        vb = rng.integers(0, 2**16, n, dtype=np.uint16).view(np.int16)
        c.k_pool.view(torch.int16).copy_(torch.from_numpy(kb))
        c.v_pool.view(torch.int16).copy_(torch.from_numpy(vb))
    else:
        kb = rng.integers(0, 2**32, n, dtype=np.uint32).view(np.int32)
        vb = rng.integers(0, 2**32, n, dtype=np.uint32).view(np.int32)
        c.k_pool.view(torch.int32).copy_(torch.from_numpy(kb))
        c.v_pool.view(torch.int32).copy_(torch.from_numpy(vb))
    torch.cuda.synchronize()
    return c


def run_copy(src, dst, pairs):
    pka.kv_copy_blocks(src, dst, torch.from_numpy(np.asarray(pairs, np.int32)).cuda())
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,hkv,d", [(torch.bfloat16, 8, 128), (torch.float32, 2, 64), (torch.bfloat16, 32, 64)])
def test_copy_within_one_pool_bitwise(dtype, hkv, d):
    say(f"copy within one pool {dtype} hkv={hkv} d={d}")
    nb = 64
    c = random_cache(nb, hkv, d, dtype, 1)
    k0, v0 = pool_bits(c)
    rng = np.random.default_rng(2)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:20], perm[20:40]], 1)           # sources and destinations disjoint
    pairs = np.concatenate([pairs, [[nb, 5], [3, -2], [-1, 7]]])  # out-of-range pairs: skipped
    run_copy(c, c, pairs)
    k1, v1 = pool_bits(c)
    ek, ev = L.copy_blocks(k0, v0, k0, v0, pairs, hkv, d, nb, nb)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev)


def test_swap_out_to_pinned_host_and_back_bitwise():
    say("swap out to pinned host pool and back")
    hkv, d = 8, 128
    dev = random_cache(96, hkv, d, torch.bfloat16, 3)
    host = random_cache(40, hkv, d, torch.bfloat16, 4, pinned_host=True)
    assert host.k_pool.is_pinned() and host.k_pool.device.type == "cpu"
    k0, v0 = pool_bits(dev)
    hk0, hv0 = pool_bits(host)
    hk0, hv0 = hk0.copy(), hv0.copy()
    out_pairs = np.array([[10, 0], [11, 1], [50, 39], [95, 20]])
    run_copy(dev, host, out_pairs)                            # swap out
    hk1, hv1 = pool_bits(host)
    ek, ev = L.copy_blocks(k0, v0, hk0, hv0, out_pairs, hkv, d, 96, 40)
    assert np.array_equal(hk1, ek) and np.array_equal(hv1, ev)
    in_pairs = np.array([[0, 60], [1, 61], [39, 62], [20, 63]])
    run_copy(host, dev, in_pairs)                             # swap in, to other blocks
    k2, v2 = pool_bits(dev)
    ek2, ev2 = L.copy_blocks(hk1, hv1, k0, v0, in_pairs, hkv, d, 40, 96)
    assert np.array_equal(k2, ek2) and np.array_equal(v2, ev2)
    tile = hkv * 16 * d
    for a, b in [(10, 60), (11, 61), (50, 62), (95, 63)]:
        assert np.array_equal(k2[b * tile:(b + 1) * tile], k0[a * tile:(a + 1) * tile])


def test_decode_through_copied_blocks_is_bitwise_identical():
    """A decode whose block table points at copies of the blocks gives the
    same output bits as through the originals."""
    say("decode through copied blocks")
    step = W.random_step(71, W.BF16, 8, 2, 128, [300, 47, 1000], [1, 1, 1])
    ds = DeviceStep(step, fill=0.0)
    ds.fill_cache()
    a = ds.decode()
    nb = step.num_blocks
    big = pka.KVCache.allocate(2 * nb, 2, 128, torch.bfloat16, fill=float("nan"))
    used = sorted({int(b) for s in range(step.num_seqs) for b in step.block_tables[s][: (int(step.kv_lens[s]) + 15) // 16]})
    new_id = {b: nb + i for i, b in enumerate(used)}
    run_copy(ds.cache, big, [[b, new_id[b]] for b in used])
    bt = step.block_tables.copy()
    for s in range(step.num_seqs):
        n = (int(step.kv_lens[s]) + 15) // 16
        bt[s][:n] = [new_id[int(b)] for b in bt[s][:n]]
    q = ds.q.view(step.num_seqs, step.num_q_heads, step.head_dim)
    b = pka.attn_decode_paged(q, big, torch.from_numpy(bt.astype(np.int32)).cuda(), ds.kv_lens, int(step.max_kv_len))
    assert torch.equal(a, b)


def test_pageable_host_pool_is_rejected_before_launch():
    say("pageable host pool rejected")
    dev = random_cache(8, 2, 64, torch.bfloat16, 5)
    pageable = pka.KVCache.allocate(8, 2, 64, torch.bfloat16, device="cpu", fill=0.0)
    assert not pageable.k_pool.is_pinned()
    with pytest.raises(pka.PkaError) as e:
        run_copy(dev, pageable, [[0, 1]])
    assert e.value.status == -1
