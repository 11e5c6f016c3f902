"""The decode entry point that allocates nothing (pka_attn_decode_paged_noalloc)
against the workspace decode (pka_attn_decode_paged), through the C ABI: two
calls in a row, the second on a smaller batch, each with split partials in
the library's fixed device scratch; outputs bit-identical to the workspace
call (same kernels, same plan) and within the bf16 bound of the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(ds, splits, hint):
    st = ds.step
    q = ds.q.view(st.num_seqs, st.num_q_heads, st.head_dim)
    hl = ds.kv_lens_host if hint else None
    ref = pka.attn_decode_paged(q, ds.cache, ds.block_tables, ds.kv_lens, st.max_kv_len, num_splits=splits,
                                kv_lens_host=hl)
    got = torch.full_like(q, float("nan"))
    pka.attn_decode_paged_noalloc(q, ds.cache, ds.block_tables, ds.kv_lens, st.max_kv_len, num_splits=splits,
                                  kv_lens_host=hl, out=got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("splits,hint", [(4, True), (0, False), (7, False)])
def test_noalloc_decode_two_calls_match_workspace_decode(splits, hint):
    cases = [("larger", 61, 48, 32, 8, (128, 2048)), ("smaller", 62, 9, 16, 4, (20, 700))]
    for what, seed, B, hq, hkv, (lo, hi) in cases:
        rng = np.random.default_rng(seed)
        kv = rng.integers(lo, hi + 1, size=B)
        step = W.random_step(seed, W.BF16, hq, hkv, 128, kv, np.ones(B, np.int64), sigma=1.0)
        need = pka.decode_workspace_size(B, hq, hkv, 128, step.max_kv_len, splits)
        say(f"noalloc decode {what}: B={B} GQA {hq}/{hkv} kv {lo}..{hi} splits={splits} hint={hint} "
            f"partials {need} B")
        ds = DeviceStep(step)
        ds.fill_cache()
        ref, got = _both(ds, splits, hint)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), what
        compare(got, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, f"noalloc decode {what}")


def test_noalloc_decode_rejects_plans_beyond_the_scratch():
    """A plan whose partials exceed the fixed scratch is refused before any
    launch; the output buffer is left untouched.  (The kernels never run, so
    the pool and tables only need valid shapes.)"""
    B, hq, hkv, max_blocks = 512, 64, 8, 64
    assert pka.decode_workspace_size(B, hq, hkv, 128, 1024, 64) > pka.NOALLOC_SCRATCH_BYTES
    say("noalloc decode: a plan beyond the scratch is rejected on the host")
    cache = pka.KVCache.allocate(16, hkv, 128, torch.bfloat16, fill=0.0)
    q = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, max_blocks), dtype=torch.int32, device="cuda")
    kvl = torch.full((B,), 1024, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(pka.PkaError) as e:
        pka.attn_decode_paged_noalloc(q, cache, bt, kvl, 1024, num_splits=64, out=out)
    assert e.value.status == pka.PKA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
