"""Calls on separate streams at once.  Each entry point keeps no state
between calls beyond its arguments (the caller's workspace), so a decode, a
prefill and a mixed step launched concurrently on three streams give the
same bits as the same calls run one after another."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, compare, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_concurrent_calls_on_three_streams_bitwise():
    say("decode, prefill and mixed step on three streams at once vs one after another")
    rng = np.random.default_rng(91)
    dec = W.random_step(91, W.BF16, 32, 8, 128, rng.integers(64, 2049, 48), [1] * 48)
    pre_lens = [1024, 700, 300]
    pre = W.random_step(92, W.BF16, 16, 16, 128, pre_lens, pre_lens)
    mkv = np.concatenate([rng.integers(64, 1500, 24), [1536]])
    mql = np.concatenate([np.ones(24, np.int64), [512]])
    mix = W.random_step(93, W.BF16, 32, 8, 128, mkv, mql)
    dd, dp, dm = DeviceStep(dec), DeviceStep(pre), DeviceStep(mix)
    dd.fill_cache()
    dm.fill_cache()
    kn, vn = pre.new_kv()
    kn, vn = dev(kn, dp.dt), dev(vn, dp.dt)
    qd = dd.q.view(dec.num_seqs, 32, 128)
    wsd = torch.empty(max(256, pka.decode_workspace_size(dec.num_seqs, 32, 8, 128, dec.max_kv_len, 4,
                                                          dd.cache.dtype_code)), dtype=torch.uint8, device="cuda")
    wsm = torch.empty(max(256, pka.mixed_workspace_size(mix.num_seqs, 32, 8, 128, int(mkv[:24].max()))),
                      dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(qd), torch.empty_like(dp.q), torch.empty_like(dm.q)]
    cu_p, cu_m, kv_m = (torch.from_numpy(x) for x in (dp.cu_q_host, dm.cu_q_host, dm.kv_lens_host))
    calls = [
        lambda: pka.attn_decode_paged(qd, dd.cache, dd.block_tables, dd.kv_lens, dec.max_kv_len, num_splits=4,
                                      workspace=wsd, out=outs[0]),
        lambda: pka.attn_prefill_varlen(dp.q, kn, vn, dp.cu_q, cu_p, out=outs[1]),
        lambda: pka.attn_mixed_step(dm.q, dm.cache, dm.cu_q, cu_m, dm.kv_lens, kv_m, dm.block_tables,
                                    workspace=wsm, out=outs[2]),
    ]
    refs = []
    for c, o in zip(calls, outs):
        c()
        torch.cuda.synchronize()
        refs.append(o.clone())
    compare(refs[0], A.attention_ragged(dec.q, dec.k_ctx, dec.v_ctx), W.BF16, "decode (sequential)")
    compare(refs[1], A.attention_ragged(pre.q, pre.k_ctx, pre.v_ctx), W.BF16, "prefill (sequential)")
    compare(refs[2], A.attention_ragged(mix.q, mix.k_ctx, mix.v_ctx), W.BF16, "mixed (sequential)")
    streams = [torch.cuda.Stream() for _ in calls]
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        order = [0, 1, 2] if rep % 2 == 0 else [2, 1, 0]
        for i in order:
            with torch.cuda.stream(streams[i]):
                calls[i]()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i], refs[i]), (rep, i)
    say("three streams at once: every output bit-equal to the sequential calls, 4 rounds")
