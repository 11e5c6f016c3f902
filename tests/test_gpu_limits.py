"""GPU parity beyond the benchmark sizes, in the default launch configuration:
one 65536-token prompt (its K/V also appended into the pool), decode over
262144 keys (a block-table row used to its full width, automatic and fixed
split plans), and a mixed step whose chunk has 16384 rows on 16384 cached
tokens beside 64 decode rows.  Long rows are checked on samples (work-unit and
key-tile edges, the first and last rows, random rows) against the oracle's
causal attention of those rows; decode rows and the appended pools in full."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, check_whole_pool_append, compare, pool_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sampled_rows(n: int, seed: int) -> np.ndarray:
    """Rows at 16-, 32-, 48- and 192-row boundaries, the middle, the ends and
    16 random rows of an n-row sequence."""
    edges = [0, 1, 15, 16, 31, 32, 47, 48, 191, 192, 193, n // 2 - 1, n // 2, n - 49, n - 48, n - 33, n - 32,
             n - 2, n - 1]
    rnd = np.random.default_rng(seed).integers(0, n, 16)
    return np.unique(np.clip(np.concatenate([edges, rnd]), 0, n - 1))


def rows_ref(q_seq, k_seq, v_seq, rows, positions):
    """Oracle rows ``rows`` of one sequence (query row r at absolute position
    positions[i]), every query head: ``[len(rows)][Hq][d]``.  The G query heads
    of a kv head go through the oracle together as G rows at the same
    positions, so each kv head's keys are converted once."""
    _, hq, d = q_seq.shape
    hkv = k_seq.shape[1]
    G = hq // hkv
    scale = A.default_scale(d)
    out = np.empty((len(rows), hq, d))
    for g in range(hkv):
        qg = q_seq[rows, g * G:(g + 1) * G, :].reshape(len(rows) * G, d)
        pg = np.repeat(np.asarray(positions, np.int64), G)
        out[:, g * G:(g + 1) * G, :] = A.attend_rows(qg, k_seq[:, g], v_seq[:, g], pg, scale).reshape(
            len(rows), G, d)
    return out


@pytest.mark.timeout(300)
def test_prefill_one_65536_token_prompt_sampled_rows():
    n = 65536
    say(f"prefill one {n}-token prompt, GQA 8/1, d=128, bf16: whole-pool append, sampled rows")
    step = W.make_step("prefill_1x65536", W.BF16, 8, 1, 128, [n], [n], 20)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    check_whole_pool_append(ds, k0, v0, "prefill_1x65536")
    out = ds.prefill().view(n, 8, 128)
    rows = sampled_rows(n, 1)
    ref = rows_ref(step.q[0], step.k_ctx[0], step.v_ctx[0], rows, rows)
    compare(out[torch.from_numpy(rows).cuda()], ref, W.BF16, "prefill_1x65536 sampled rows")


@pytest.mark.timeout(300)
def test_decode_262144_keys_full_table_row():
    kv = [262144, 262143, 17, 100000]
    say(f"decode over up to {kv[0]} keys (table row of {kv[0] // 16} blocks), GQA 8/1, d=128, bf16")
    step = W.make_step("decode_262144", W.BF16, 8, 1, 128, kv, [1] * len(kv), 21)
    assert step.max_blocks_per_seq == kv[0] // 16
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    check_whole_pool_append(ds, k0, v0, "decode_262144")
    ref = np.concatenate([rows_ref(step.q[s], step.k_ctx[s], step.v_ctx[s], [0], [kv[s] - 1])
                          for s in range(len(kv))])
    for splits in (0, 1, 64):
        compare(ds.decode(num_splits=splits), ref, W.BF16, f"decode_262144 splits={splits}")


@pytest.mark.timeout(300)
def test_mixed_16384_row_chunk_on_16384_cached_tokens():
    rng = np.random.default_rng(22)
    n_dec, chunk, cached = 64, 16384, 16384
    kv = np.concatenate([rng.integers(1, 4097, size=n_dec), [cached + chunk]])
    ql = np.concatenate([np.ones(n_dec, np.int64), [chunk]])
    say(f"mixed: {n_dec} decode rows + one {chunk}-row chunk on {cached} cached tokens, GQA 8/1, d=128, bf16")
    step = W.make_step("mixed_16384_chunk", W.BF16, 8, 1, 128, kv, ql, 22)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    check_whole_pool_append(ds, k0, v0, "mixed_16384_chunk")
    out = ds.mixed()
    compare(out[:n_dec], A.attention_ragged(step.q[:n_dec], step.k_ctx[:n_dec], step.v_ctx[:n_dec]), W.BF16,
            "mixed_16384_chunk decode rows")
    rows = sampled_rows(chunk, 2)
    ref = rows_ref(step.q[n_dec], step.k_ctx[n_dec], step.v_ctx[n_dec], rows, cached + rows)
    compare(out[torch.from_numpy(n_dec + rows).cuda()], ref, W.BF16, "mixed_16384_chunk sampled chunk rows")
