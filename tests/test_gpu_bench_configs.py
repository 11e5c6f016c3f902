"""Parity of the configurations the benchmark times beside the five
workloads, at the benchmark's sizes and in its launch configuration: the
headline decode batch in fp16 and without host lengths, the mixed step over
an fp8 cache, and the block copy and swaps of 2048 and 1024 64 KiB blocks.
The copy pools hold random bits here (the benchmark fills them with a
constant), so a misplaced or missed block shows."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from oracle import fp8 as F8
from oracle import paged_layout as L
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, check_whole_pool_append, codes_of, compare, pool_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_decode_mha_f16_full_size():
    say("decode MHA 64 x U{128..2048} fp16, every row, whole-pool append")
    step = W.decode_mha_7b(2, dtype=W.F16)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    compare(ds.decode(), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.F16, "decode_mha fp16")
    check_whole_pool_append(ds, k0, v0, "decode_mha fp16")


def test_decode_mha_without_host_lengths_full_size():
    say("decode MHA 64 x U{128..2048} bf16 without host lengths (index order, automatic splits)")
    step = W.decode_mha_7b(2)
    ds = DeviceStep(step)
    ds.fill_cache()
    compare(ds.decode(host_lens=False), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16,
            "decode_mha without host lengths")


@pytest.mark.timeout(300)
def test_mixed_gqa_fp8_full_size():
    """The mixed step the benchmark times over an fp8 cache (its seeded
    per-kv-head scales): every sequence's codes against the oracle's
    quantizer, every output row against the oracle over the dequantized
    keys and values."""
    say("mixed GQA 32/8 (128 decodes + 2 x 1024 chunks) over an fp8 cache, full size")
    step = W.mixed_gqa(4)
    hkv = step.num_kv_heads
    ks, vs = W.fp8_scales(11, hkv, step.sigma), W.fp8_scales(12, hkv, step.sigma)
    ds = DeviceStep(step, fp8_scales=(ks, vs))
    ds.fill_cache()
    out = ds.mixed()
    k1, v1 = pool_bits(ds.cache)
    kd, vd = [], []
    for s in range(step.num_seqs):
        kc, vc = codes_of(step.k_ctx[s], ks), codes_of(step.v_ctx[s], vs)
        kg, vg = L.gather(k1, v1, step.block_tables[s], int(step.kv_lens[s]), hkv, step.head_dim)
        assert np.array_equal(kg, kc) and np.array_equal(vg, vc), s
        kd.append(np.stack([F8.dequantize(kc[:, g, :], ks[g]) for g in range(hkv)], 1))
        vd.append(np.stack([F8.dequantize(vc[:, g, :], vs[g]) for g in range(hkv)], 1))
    say("mixed fp8: every sequence's codes match the oracle's quantizer")
    compare(out, A.attention_ragged(step.q, kd, vd), W.BF16, "mixed_gqa fp8, every row")


def _random_bits(cache: pka.KVCache, gen: torch.Generator):
    for pool in (cache.k_pool, cache.v_pool):
        bits = torch.randint(-32768, 32768, pool.shape, dtype=torch.int32, generator=gen).to(torch.int16)
        pool.view(torch.int16).copy_(bits)


def test_copy_and_swap_bench_size_bitwise():
    """The benchmark's copy cases (GQA 8 kv heads, d = 128, bf16; seed-7
    block permutation of an 8192-block pool): 2048 copy-on-write pairs inside
    the device pool, 1024 blocks out to a pinned host pool and 1024 back in,
    each compared byte for byte with the oracle's block copy."""
    hkv, d, nb, nh = 8, 128, 8192, 1024
    say(f"block copy {2048} pairs in an {nb}-block pool, swap {nh} out and in, bitwise")
    gen = torch.Generator().manual_seed(70)
    dev = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16)
    host = pka.KVCache.allocate(nh, hkv, d, torch.bfloat16, pinned_host=True)
    _random_bits(dev, gen)
    _random_bits(host, gen)
    torch.cuda.synchronize()
    perm = np.random.default_rng(7).permutation(nb)
    cow = np.stack([perm[:2048], perm[2048:4096]], 1).astype(np.int32)
    out_pairs = np.stack([perm[:nh], np.arange(nh)], 1).astype(np.int32)
    in_pairs = np.stack([np.arange(nh), perm[4096:4096 + nh]], 1).astype(np.int32)

    k0, v0 = pool_bits(dev)
    pka.kv_copy_blocks(dev, dev, torch.from_numpy(cow).cuda())
    torch.cuda.synchronize()
    k1, v1 = pool_bits(dev)
    ek, ev = L.copy_blocks(k0, v0, k0, v0, cow, hkv, d, nb, nb)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev), "copy-on-write"

    hk0, hv0 = (x.copy() for x in pool_bits(host))  # host pools: pool_bits shares their memory
    pka.kv_copy_blocks(dev, host, torch.from_numpy(out_pairs).cuda())
    torch.cuda.synchronize()
    hk1, hv1 = (x.copy() for x in pool_bits(host))
    ek, ev = L.copy_blocks(k1, v1, hk0, hv0, out_pairs, hkv, d, nb, nh)
    assert np.array_equal(hk1, ek) and np.array_equal(hv1, ev), "swap out"

    pka.kv_copy_blocks(host, dev, torch.from_numpy(in_pairs).cuda())
    torch.cuda.synchronize()
    k2, v2 = pool_bits(dev)
    ek, ev = L.copy_blocks(hk1, hv1, k1, v1, in_pairs, hkv, d, nh, nb)
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev), "swap in"
    say("copy-on-write, swap out and swap in: every pool byte as the oracle's copy")
