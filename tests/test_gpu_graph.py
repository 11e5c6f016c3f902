"""The library's calls captured into a HIP graph (torch.cuda.graph) and
replayed, for launch-bound serving loops.

Nothing the entry points launch is a memset or an allocation, so a captured
step (append + attention) replays as recorded.  Each test captures one step,
replays it several times with the program's own eager work and
synchronisations between the replays, and checks every replay bit for bit
against the eager run of the same step (and the eager run against the
oracle).
"""
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


def eager_noise(n):
    """Unrelated eager work between replays."""
    x = torch.randn(1 << 20, device="cuda")
    for _ in range(n):
        x = x * 1.0001 + 1.0
    torch.cuda.synchronize()
    return x


def capture_and_replay(step_fn, replays=4):
    ref = step_fn().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm the allocator outside capture
        step_fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step_fn()
    for i in range(replays):
        eager_noise(3 + i)
        out.fill_(float("nan"))                     # the replay must write every output element
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager step"
    return ref


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_graph_decode_step(dtype):
    say(f"graph: append + decode step, {dtype}")
    kv = [300, 17, 1000, 64, 129, 5]
    step = W.random_step(81, dtype, 8, 2, 128 if dtype == W.BF16 else 64, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.append_cached()
    kn, vn = step.new_kv()
    kn, vn = dev(kn, ds.dt), dev(vn, ds.dt)
    slots = dev(step.new_slot_mapping().astype(np.int32))
    q = ds.q.view(step.num_seqs, 8, step.head_dim)
    ws = torch.zeros(max(256, pka.decode_workspace_size(step.num_seqs, 8, 2, step.head_dim, step.max_kv_len, 0,
                                                         ds.cache.dtype_code)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step_fn():
        pka.kv_append(ds.cache, kn, vn, slots)
        return pka.attn_decode_paged(q, ds.cache, ds.block_tables, ds.kv_lens, step.max_kv_len, workspace=ws,
                                     out=out, kv_lens_host=torch.from_numpy(ds.kv_lens_host))

    ref = capture_and_replay(step_fn)
    compare(ref, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, "graph decode (eager)")


def test_graph_mixed_step():
    say("graph: append + mixed step (decodes + a chunk)")
    kv, ql = [300, 700, 64, 500], [1, 96, 1, 1]
    step = W.random_step(82, W.BF16, 8, 2, 128, kv, ql)
    ds = DeviceStep(step)
    ds.append_cached()
    kn, vn = step.new_kv()
    kn, vn = dev(kn, ds.dt), dev(vn, ds.dt)
    slots = dev(step.new_slot_mapping().astype(np.int32))
    ws = torch.zeros(max(256, pka.mixed_workspace_size(step.num_seqs, 8, 2, 128,
                                                        int(step.kv_lens[step.q_lens == 1].max()))),
                     dtype=torch.uint8, device="cuda")
    cu_host, kv_host = torch.from_numpy(ds.cu_q_host), torch.from_numpy(ds.kv_lens_host)
    out = torch.empty_like(ds.q)

    def step_fn():
        pka.kv_append(ds.cache, kn, vn, slots)
        return pka.attn_mixed_step(ds.q, ds.cache, ds.cu_q, cu_host, ds.kv_lens, kv_host, ds.block_tables,
                                   workspace=ws, out=out)

    ref = capture_and_replay(step_fn)
    compare(ref, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "graph mixed (eager)")


def test_graph_prefill_step():
    """Append of a ragged batch's keys/values plus its varlen prefill (prompts
    over several work units, ragged tails), captured and replayed."""
    say("graph: append + prefill step")
    lens = [700, 33, 1, 300]
    step = W.random_step(83, W.BF16, 8, 2, 128, lens, lens)
    ds = DeviceStep(step)
    kn, vn = step.new_kv()
    kn, vn = dev(kn, ds.dt), dev(vn, ds.dt)
    slots = dev(step.new_slot_mapping().astype(np.int32))
    cu_host = torch.from_numpy(ds.cu_q_host)
    out = torch.empty_like(ds.q)

    def step_fn():
        pka.kv_append(ds.cache, kn, vn, slots)
        return pka.attn_prefill_varlen(ds.q, kn, vn, ds.cu_q, cu_host, out=out)

    ref = capture_and_replay(step_fn)
    compare(ref, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "graph prefill (eager)")


def test_graph_noalloc_decode_step():
    """The decode entry point that allocates nothing, with split partials in
    its fixed device scratch (forced splits), captured with the append."""
    say("graph: append + decode through the no-allocation entry point, 3 splits")
    kv = [1500, 17, 900, 64, 2048]
    step = W.random_step(84, W.BF16, 16, 2, 128, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.append_cached()
    kn, vn = step.new_kv()
    kn, vn = dev(kn, ds.dt), dev(vn, ds.dt)
    slots = dev(step.new_slot_mapping().astype(np.int32))
    q = ds.q.view(step.num_seqs, 16, 128)
    out = torch.empty_like(q)
    hint = torch.from_numpy(ds.kv_lens_host)

    def step_fn():
        pka.kv_append(ds.cache, kn, vn, slots)
        return pka.attn_decode_paged_noalloc(q, ds.cache, ds.block_tables, ds.kv_lens, step.max_kv_len,
                                             num_splits=3, out=out, kv_lens_host=hint)

    ref = capture_and_replay(step_fn)
    compare(ref, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "graph noalloc decode (eager)")
