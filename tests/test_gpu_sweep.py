"""Seeded random sweep of the attention entry points against the oracle
(seeds 101-108).

Each seed draws one configuration -- dtype (bf16 or fp16), kv heads, group
size G in {1, 2, 3, 4, 8}, head dim, batch size and kv lengths, a share of
them at block and tile edges -- and runs it through the prefill, the decode
(a drawn split count, with or without the host lengths), the mixed step
(rows drawn among decode, chunk, whole prompt and idle) and speculative
verify (a drawn row count and split count), and the mixed step again over an
fp8 cache.  Every output is compared with the fp64 oracle at the dtype's
tolerance.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, compare, say

pytestmark = pytest.mark.gpu
SEEDS = list(range(101, 109))
EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(seed):
    rng = np.random.default_rng(seed)
    dtype = W.BF16 if seed % 2 else W.F16
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    if hkv * g > 16:
        hkv = max(1, 16 // g)
    d = int(rng.choice([64, 128]))
    b = int(rng.integers(1, 9))
    kv = [int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(1, 1100)) for _ in range(b)]
    return rng, dtype, hkv * g, hkv, d, kv


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_prefill(seed):
    rng, dtype, hq, hkv, d, kv = draw(seed)
    say(f"sweep {seed} prefill {dtype} {hq}/{hkv} d={d} lens={kv}")
    step = W.random_step(seed, dtype, hq, hkv, d, kv, kv)
    out = DeviceStep(step).prefill()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, f"sweep {seed} prefill")


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_decode(seed):
    rng, dtype, hq, hkv, d, kv = draw(seed)
    splits = int(rng.choice([0, 1, 2, 3, 7]))
    hint = bool(rng.integers(2))
    say(f"sweep {seed} decode {dtype} {hq}/{hkv} d={d} kv={kv} splits={splits} host_lens={hint}")
    step = W.random_step(seed, dtype, hq, hkv, d, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.decode(num_splits=splits, host_lens=hint)
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, f"sweep {seed} decode")


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_mixed(seed):
    rng, dtype, hq, hkv, d, kv = draw(seed)
    ql = []
    for L in kv:
        kind = int(rng.integers(4))          # decode, chunk, whole prompt, idle
        ql.append([1, int(rng.integers(1, L + 1)), L, 0][kind])
    say(f"sweep {seed} mixed {dtype} {hq}/{hkv} d={d} kv={kv} q={ql}")
    step = W.random_step(seed, dtype, hq, hkv, d, kv, ql)
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.mixed()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, f"sweep {seed} mixed")


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_verify(seed):
    rng, dtype, hq, hkv, d, kv = draw(seed)
    nq = int(rng.integers(2, 10))
    kv = [max(L, nq) for L in kv]
    splits = int(rng.choice([0, 1, 2, 5]))
    say(f"sweep {seed} verify {dtype} {hq}/{hkv} d={d} kv={kv} nq={nq} splits={splits}")
    step = W.random_step(seed, dtype, hq, hkv, d, kv, [nq] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    q = ds.q.view(step.num_seqs, nq, hq, d)
    out = pka.attn_verify_paged(q, ds.cache, ds.block_tables, ds.kv_lens, int(step.max_kv_len), num_splits=splits,
                                kv_lens_host=ds.kv_lens_host if seed % 3 else None)
    torch.cuda.synchronize()
    compare(out.view(-1, hq, d), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, f"sweep {seed} verify")


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_fp8_mixed(seed):
    """The mixed-step draw over an fp8 E4M3 cache with drawn per-head scales,
    against the oracle attending over the dequantized keys and values."""
    from test_gpu_fp8 import dequantized_ctx, fp8_step
    rng, dtype, hq, hkv, d, kv = draw(seed)
    ql = [[1, int(rng.integers(1, L + 1)), L, 0][int(rng.integers(4))] for L in kv]
    say(f"sweep {seed} fp8 mixed {dtype} {hq}/{hkv} d={d} kv={kv} q={ql}")
    step, ks, vs, ds = fp8_step(seed, dtype, hq, hkv, d, kv, ql)
    ds.fill_cache()
    out = ds.mixed()
    kd, vd = dequantized_ctx(step, ks, vs)
    compare(out, A.attention_ragged(step.q, kd, vd), dtype, f"sweep {seed} fp8 mixed")
