"""GPU parity at the five workloads' full sizes, in the same launch
configuration the benchmark times (automatic split plan).  Every output row
is compared with the fp64 oracle; every appended pool is checked byte for
byte, whole, against the oracle's append."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from oracle import paged_layout as L
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, check_whole_pool_append, compare, pool_bits, say, value_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_tiny_fp32_prefill_then_decode():
    """4 prompts {5,17,32,64}, fp32, 2/2 heads, d=64, 16-block permuted pool:
    causal prefill with append, then one decode step with append."""
    say("tiny fp32 prefill -> decode")
    pre, dec = W.tiny_fp32(1)
    ds = DeviceStep(dec)             # pools and tables for the whole run
    k0, v0 = pool_bits(ds.cache)
    pre_ds = DeviceStep(pre)
    out = pre_ds.prefill()
    compare(out, A.attention_ragged(pre.q, pre.k_ctx, pre.v_ctx), W.F32, "tiny prefill")
    ds.append_cached()               # the prompts' K/V (slots of positions 0..L-1)
    ds.append_new()                  # the decode tokens
    torch.cuda.synchronize()
    k1, v1 = pool_bits(ds.cache)
    ek, ev = k0, v0
    for kk, vv, sl in [(dec.cached_kv()[0], dec.cached_kv()[1], dec.cached_slot_mapping()),
                       (dec.new_kv()[0], dec.new_kv()[1], dec.new_slot_mapping())]:
        ek, ev = L.append(ek, ev, value_bits(kk, W.F32), value_bits(vv, W.F32), sl, 2, 64)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev)
    out = ds.decode()
    compare(out, A.attention_ragged(dec.q, dec.k_ctx, dec.v_ctx), W.F32, "tiny decode")
    # the mixed entry point on the same decode rows
    out = ds.mixed()
    compare(out, A.attention_ragged(dec.q, dec.k_ctx, dec.v_ctx), W.F32, "tiny decode via mixed")


def test_decode_mha_64x_ctx128_2048():
    say("decode MHA 64 seqs ctx 128..2048 bf16")
    step = W.decode_mha_7b(2)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    out = ds.decode()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "decode_mha")
    check_whole_pool_append(ds, k0, v0, "decode_mha")


def test_prefill_ragged_4096():
    say("prefill ragged 4096 tokens bf16")
    step = W.prefill_ragged(3)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    out = ds.prefill()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "prefill_ragged")
    ds.append_new()
    torch.cuda.synchronize()
    k1, v1 = pool_bits(ds.cache)
    kn, vn = step.new_kv()
    ek, ev = L.append(k0, v0, value_bits(kn, W.BF16), value_bits(vn, W.BF16), step.new_slot_mapping(), 32, 128)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev)


@pytest.mark.timeout(300)
def test_prefill_one_8192_token_prompt():
    """The long-prompt prefill the benchmark times (one 8192-token prompt,
    32/32 heads, seed 10), in its launch configuration: every output row of
    every head against the oracle's causal attention."""
    say("prefill one 8192-token prompt bf16, every row")
    step = W.make_step("prefill_1x8192", W.BF16, 32, 32, 128, [8192], [8192], 10)
    out = DeviceStep(step).prefill()
    compare(out, A.attention_seq(step.q[0], step.k_ctx[0], step.v_ctx[0]), W.BF16, "prefill_1x8192")


def test_mixed_gqa_128_decode_2_chunks():
    say("mixed GQA 32/8: 128 decodes + 2 x 1024 chunks")
    step = W.mixed_gqa(4)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    out = ds.mixed()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "mixed_gqa")
    check_whole_pool_append(ds, k0, v0, "mixed_gqa")


@pytest.mark.timeout(300)
def test_long_decode_gqa_16x32768():
    say("long decode GQA 64/8 16 x 32768 bf16")
    step = W.long_decode_gqa(5)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    out = ds.decode()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "long_decode")
    check_whole_pool_append(ds, k0, v0, "long_decode")


def test_spec_verify_gqa_64x5_rows():
    """Speculative verify (the first next-step row): 64 sequences x 5 new rows
    at the end of U{128..2048}-token contexts, GQA 32/8, through the mixed
    entry point; every row against the oracle, the appended K/V bit-exact."""
    say("spec verify GQA 32/8: 64 seqs x 5 rows")
    step = W.spec_verify_gqa(6)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    out = ds.mixed()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "spec_verify")
    check_whole_pool_append(ds, k0, v0, "spec_verify")


def test_spec_verify_gqa_through_verify_entry_point():
    """The same speculative-verify workload through pka_attn_verify_paged (the
    decode-unit path with the automatic split plan)."""
    say("spec verify GQA 32/8 via verify entry point")
    step = W.spec_verify_gqa(6)
    ds = DeviceStep(step)
    ds.fill_cache()
    q = ds.q.view(step.num_seqs, 5, 32, 128)
    out = pka.attn_verify_paged(q, ds.cache, ds.block_tables, ds.kv_lens, int(step.max_kv_len),
                                kv_lens_host=ds.kv_lens_host)
    torch.cuda.synchronize()
    compare(out.view(-1, 32, 128), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "spec_verify(verify)")
