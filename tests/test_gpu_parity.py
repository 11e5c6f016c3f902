"""GPU parity of the HIP path against the fp64 oracle on small seeded cases
that still span several tiles, ragged tails, GQA groupings and both head
dims; plus the bit-exact append and the invariance pins (block permutation,
NaN-poisoned free slots, batch permutation, causality, split counts)."""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from oracle import paged_layout as L
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import DeviceStep, compare, pool_bits, say, to_f64, value_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------------------
# Append (bit-exact)
# ---------------------------------------------------------------------------
APPEND_CASES = [
    (W.F32, 2, 64, [5, 17, 32, 64], [5, 17, 32, 64]),
    (W.F32, 1, 128, [3, 40], [1, 40]),
    (W.BF16, 2, 128, [1, 16, 17, 100], [1, 3, 17, 50]),
    (W.BF16, 8, 64, [33, 9], [2, 9]),
    (W.BF16, 3, 128, [47], [47]),
    (W.F16, 4, 128, [1, 16, 17, 100], [1, 3, 17, 50]),
]


@pytest.mark.parametrize("dtype,hkv,d,kv,ql", APPEND_CASES)
def test_append_bit_exact(dtype, hkv, d, kv, ql):
    say(f"append {dtype} hkv={hkv} d={d} kv={kv} q={ql}")
    step = W.random_step(31, dtype, hkv, hkv, d, kv, ql)
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    ds.fill_cache()
    k1, v1 = pool_bits(ds.cache)
    kc, vc = step.cached_kv()
    kn, vn = step.new_kv()
    ek, ev = L.append(k0, v0, value_bits(kc, dtype), value_bits(vc, dtype), step.cached_slot_mapping(), hkv, d)
    ek, ev = L.append(ek, ev, value_bits(kn, dtype), value_bits(vn, dtype), step.new_slot_mapping(), hkv, d)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev)


def test_append_skips_negative_and_out_of_range_slots():
    say("append with skipped slots")
    step = W.random_step(32, W.BF16, 2, 2, 128, [40], [40])
    ds = DeviceStep(step)
    k0, v0 = pool_bits(ds.cache)
    slots = step.new_slot_mapping().copy()
    slots[3] = -1
    slots[10] = -7
    slots[20] = step.num_blocks * 16 + 5     # beyond the pool: skipped
    ds.append_new(slots)
    torch.cuda.synchronize()
    k1, v1 = pool_bits(ds.cache)
    kn, vn = step.new_kv()
    ref_slots = slots.copy()
    ref_slots[20] = -1
    ek, ev = L.append(k0, v0, value_bits(kn, W.BF16), value_bits(vn, W.BF16), ref_slots, 2, 128)
    assert np.array_equal(k1, ek) and np.array_equal(v1, ev)


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    (W.BF16, 4, 4, 128, [1, 7, 64, 65, 130, 300]),   # G=1: prompts shorter than one key tile and than the ring's three tiles, ragged tails
    (W.BF16, 8, 2, 64, [33, 100, 5, 2]),             # G=4: 4 heads share a K/V tile
    (W.BF16, 6, 2, 128, [70, 1, 129]),               # G=3
    (W.BF16, 4, 2, 128, [200, 63]),                  # G=2
    (W.BF16, 32, 2, 128, [90]),                      # G=16
    (W.F32, 2, 2, 64, [5, 17, 32, 64]),
    (W.F32, 4, 1, 128, [20, 3]),
    (W.F32, 4, 2, 64, [200, 131, 64]),               # fp32: several keys per lane of the row's wave
    (W.F16, 4, 4, 128, [1, 7, 64, 65, 130, 300]),   # fp16: same shapes through the F16 kernels
    (W.F16, 8, 2, 64, [33, 100, 5, 2]),
    (W.BF16, 2, 2, 128, [513, 256, 257, 31, 1]),     # G=1: several 192-row work units, unit and key-tile edges
    (W.BF16, 8, 2, 128, [150, 64, 65, 129]),         # G=4: 48-position units of 4 heads
    (W.F16, 4, 2, 64, [300, 97, 128]),               # G=2: 96-position units, fp16, d=64
]


# The prefill unit comes in two shapes (32 or 48 query rows per wave); the
# library picks one per launch by its amount of work, and these small cases
# would all take the 32-row one, so each runs under both shapes, forced
# through PKA_PREFILL_UNIT_ROWS.
UNIT_ROWS = ["auto", "32", "48"]


@pytest.mark.parametrize("rows", UNIT_ROWS)
@pytest.mark.parametrize("dtype,hq,hkv,d,lens", PREFILL_CASES)
def test_prefill_matches_oracle(dtype, hq, hkv, d, lens, rows, monkeypatch):
    if rows != "auto":
        monkeypatch.setenv("PKA_PREFILL_UNIT_ROWS", rows)
    say(f"prefill {dtype} {hq}/{hkv} d={d} lens={lens} unit rows {rows}")
    step = W.random_step(41, dtype, hq, hkv, d, lens, lens)
    ds = DeviceStep(step)
    out = ds.prefill()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(out, ref, dtype, "prefill")


@pytest.mark.parametrize("dtype,hq,hkv,d,lens", [c for c in PREFILL_CASES if c[0] != W.F32])
def test_prefill_unit_shapes_bit_identical(dtype, hq, hkv, d, lens, monkeypatch):
    """Each query row is computed the same way by both unit shapes (the same
    key tiles in the same order, the same softmax and rounding), so the two
    shapes' outputs agree bit for bit."""
    say(f"prefill shapes {dtype} {hq}/{hkv} d={d} lens={lens}")
    step = W.random_step(42, dtype, hq, hkv, d, lens, lens)
    ds = DeviceStep(step)
    outs = []
    for rows in ("32", "48"):
        monkeypatch.setenv("PKA_PREFILL_UNIT_ROWS", rows)
        outs.append(ds.prefill().clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("rows", ["32", "48"])
@pytest.mark.parametrize("hq,hkv,dtype", [(2, 2, W.BF16), (4, 2, W.BF16), (8, 2, W.F16)])
def test_prefill_dominant_late_key(hq, hkv, dtype, rows, monkeypatch):
    """A key far inside the prompt whose score exceeds every earlier one by
    hundreds (log2 units): the rows that see it must switch their running
    maximum mid-prompt (the lazy rescale, taken when a lane's weight sum
    passes its limit).  Rows before it are unaffected; rows after it put
    almost all weight on its value row."""
    monkeypatch.setenv("PKA_PREFILL_UNIT_ROWS", rows)
    say(f"prefill dominant late key {hq}/{hkv} {dtype} unit rows {rows}")
    lens = [300, 90]
    step = W.random_step(45, dtype, hq, hkv, 128, lens, lens)
    q0, k0 = step.q[0], step.k_ctx[0]
    q0[:] = W.round_to_dtype(q0 + 3.0, dtype)       # every query row shares a component along ones
    k0[200] = 20.0                                  # key 200: score ~ 20 * 3 * 128 / sqrt(128) = 679
    step.k_ctx[0] = k0
    out = DeviceStep(step).prefill()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(out, ref, dtype, "prefill dominant late key")


def test_prefill_explicit_scale_and_empty_prompts():
    say("prefill explicit scale, empty prompts")
    step = W.random_step(42, W.BF16, 4, 4, 64, [0, 50, 0, 20], [0, 50, 0, 20])
    ds = DeviceStep(step)
    out = ds.prefill(scale=0.05)
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx, scale=0.05)
    compare(out, ref, W.BF16, "prefill scale=0.05")


def test_prefill_many_prompts_level_grid():
    """More prompts than the launch's work-map table holds (256): the launch
    falls back to the plain level grid.  Same results as the oracle, and the
    first 200 prompts' rows equal a mapped launch over those prompts alone."""
    rng = np.random.default_rng(44)
    lens = rng.integers(0, 40, size=600)
    lens[7] = 200
    say(f"prefill {len(lens)} prompts (level-grid fallback), total {int(lens.sum())} rows")
    # Values N(0, 0.5^2): rows with one or two keys return a V row, and with
    # 3M N(0,1) draws some |o| exceed 4, where half a bf16 ulp (1.6e-2) is
    # already above the 1e-2 bound.
    step = W.random_step(44, W.BF16, 4, 2, 64, lens, lens, sigma=0.5)
    out = DeviceStep(step).prefill()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(out, ref, W.BF16, "prefill 600 prompts")
    head = W.Step(step.name, step.dtype, 4, 2, 64, step.kv_lens[:200], step.q_lens[:200], step.k_ctx[:200],
                  step.v_ctx[:200], step.q[:200], step.block_tables[:200], step.num_blocks)
    out200 = DeviceStep(head).prefill()
    assert torch.equal(out[: int(lens[:200].sum())], out200)


def test_prefill_causality_bitwise():
    say("prefill causality")
    step = W.random_step(43, W.BF16, 4, 4, 128, [200], [200])
    a = DeviceStep(step).prefill()
    k2 = step.k_ctx[0].copy()
    v2 = step.v_ctx[0].copy()
    k2[150:] = W.round_to_dtype(k2[150:] * -3.0 + 1.0, W.BF16)
    v2[150:] = W.round_to_dtype(v2[150:] * 2.0 - 1.0, W.BF16)
    step.k_ctx[0], step.v_ctx[0] = k2, v2
    b = DeviceStep(step).prefill()
    assert torch.equal(a[:150], b[:150])
    assert not torch.equal(a[150:], b[150:])


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
DECODE_CASES = [
    (W.BF16, 4, 4, 128, [1, 2, 15, 16, 17, 33, 300, 1000]),  # G=1
    (W.BF16, 8, 2, 128, [500, 64, 7]),                        # G=4
    (W.BF16, 16, 2, 64, [129, 1]),                            # G=8, d=64
    (W.BF16, 6, 2, 128, [77, 250]),                           # G=3
    (W.BF16, 32, 1, 128, [260]),                              # G=32: two row groups
    (W.F32, 2, 2, 64, [6, 18, 33, 65]),
    (W.F32, 8, 2, 128, [40, 3]),
    (W.F32, 4, 2, 64, [300, 129, 1000, 1]),          # fp32: up to 16 keys per lane
    (W.F16, 4, 4, 128, [1, 2, 15, 16, 17, 33, 300, 1000]),
    (W.F16, 16, 2, 64, [129, 1]),
]


@pytest.mark.parametrize("dtype,hq,hkv,d,kv", DECODE_CASES)
def test_decode_matches_oracle(dtype, hq, hkv, d, kv):
    say(f"decode {dtype} {hq}/{hkv} d={d} kv={kv}")
    step = W.random_step(51, dtype, hq, hkv, d, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(ds.decode(), ref, dtype, "decode")
    compare(ds.decode(host_lens=False), ref, dtype, "decode, device lengths only")


def test_decode_host_lengths_are_a_hint_only():
    """The host lengths only choose the dispatch order: at a fixed split count
    the outputs with the hint, without it, and with a stale (shuffled) hint
    are bit-identical; the automatic plan with and without it is within
    tolerance of the oracle."""
    say("decode: host lengths as a scheduling hint")
    kv = [1500, 33, 700, 2048, 1, 260, 999, 64]
    step = W.random_step(56, W.BF16, 8, 2, 128, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    stale = np.random.default_rng(1).permutation(ds.kv_lens_host).astype(np.int32)
    for splits in (1, 3):
        outs = [ds.decode(num_splits=splits, host_lens=h).view(torch.int16) for h in (True, False, stale)]
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), splits
    for h in (True, False):
        compare(ds.decode(host_lens=h), ref, W.BF16, f"decode auto plan, host lengths {h}")


def test_decode_rows_without_keys_are_zero():
    """A decode row whose kv_len is 0 (or negative) sees no key: its output is
    zero (the defined device-side behaviour), with and without host lengths,
    split or not; the other rows match the oracle."""
    say("decode: rows with no keys")
    kv = [40, 300, 7, 1000]
    step = W.random_step(59, W.BF16, 8, 2, 128, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    lens = np.array([0, 300, -3, 1000], np.int32)    # rows 0 and 2 see no key
    ds.kv_lens = torch.from_numpy(lens).cuda()
    ds.kv_lens_host = lens
    keep = [1, 3]
    ref = A.attention_ragged([step.q[i] for i in keep], [step.k_ctx[i] for i in keep], [step.v_ctx[i] for i in keep])
    for splits in (0, 3):
        for host in (True, False):
            out = ds.decode(num_splits=splits, host_lens=host)
            assert torch.count_nonzero(out[[0, 2]]) == 0, (splits, host)
            compare(out[keep], ref, W.BF16, f"decode rows with keys (splits {splits}, host lengths {host})")


def test_decode_more_sequences_than_the_order_holds():
    """1100 sequences with host lengths: beyond the 1024 the longest-first
    order holds, the call keeps index order and the unsorted plan."""
    say("decode: 1100 sequences with host lengths")
    kv = np.random.default_rng(57).integers(1, 200, 1100)
    step = W.random_step(58, W.BF16, 4, 2, 64, kv, [1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(ds.decode(), ref, W.BF16, "decode 1100 seqs, host lengths")
    assert torch.equal(ds.decode(num_splits=2).view(torch.int16), ds.decode(num_splits=2, host_lens=False).view(torch.int16))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 0, 10 ** 6])
def test_decode_split_counts(splits):
    say(f"decode splits={splits}")
    step = W.random_step(52, W.BF16, 16, 4, 128, [1000, 17, 640, 1, 999], [1] * 5)
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.decode(num_splits=splits)
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(out, ref, W.BF16, f"decode splits={splits}")


def test_decode_one_key_returns_v_bitwise():
    say("decode one key")
    step = W.random_step(53, W.BF16, 8, 2, 128, [1, 1, 1], [1, 1, 1])
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.decode().cpu()
    for s in range(3):
        for h in range(8):
            v = torch.from_numpy(step.v_ctx[s][0, h // 4]).to(torch.bfloat16)
            assert torch.equal(out[s, h], v)


def _permuted_tables(step, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(step.num_blocks).astype(np.int32)
    bt = step.block_tables.copy()
    mask = bt >= 0
    bt[mask] = perm[bt[mask]]
    return bt


def test_decode_block_permutation_and_poison_bitwise():
    say("decode block permutation / NaN poison")
    step = W.random_step(54, W.BF16, 8, 8, 128, [700, 33, 1, 250], [1] * 4)
    a_ds = DeviceStep(step, fill=float("nan"))
    a_ds.fill_cache()
    a = a_ds.decode()
    bt = _permuted_tables(step, 5)
    b_ds = DeviceStep(step, fill=0.0, block_tables=bt)
    slots_c = np.concatenate([(bt[s][np.arange(c) // 16].astype(np.int64) * 16 + np.arange(c) % 16)
                              for s, c in enumerate(step.cached_lens)]).astype(np.int32)
    slots_n = np.array([bt[s][(c) // 16] * 16 + c % 16 for s, c in enumerate(step.cached_lens)], np.int32)
    b_ds.append_cached(slots_c)
    b_ds.append_new(slots_n)
    torch.cuda.synchronize()
    b = b_ds.decode()
    assert torch.equal(a, b)


def test_decode_batch_permutation_bitwise():
    say("decode batch permutation")
    kv = [300, 5, 1200, 64]
    step = W.random_step(55, W.BF16, 8, 2, 128, kv, [1] * 4)
    ds = DeviceStep(step)
    ds.fill_cache()
    a = ds.decode().cpu()
    perm = [2, 0, 3, 1]
    p = W.Step(step.name, step.dtype, 8, 2, 128, step.kv_lens[perm], step.q_lens[perm],
               [step.k_ctx[i] for i in perm], [step.v_ctx[i] for i in perm], [step.q[i] for i in perm],
               step.block_tables[perm], step.num_blocks)
    pds = DeviceStep(p)
    pds.fill_cache()
    b = pds.decode().cpu()
    assert torch.equal(a[perm], b)


# ---------------------------------------------------------------------------
# Mixed chunked-prefill + decode
# ---------------------------------------------------------------------------
MIXED_CASES = [
    (W.BF16, 8, 2, 128, [300, 1, 64, 500, 40, 2], [1, 1, 37, 130, 0, 2]),
    (W.BF16, 4, 4, 64, [129, 1000, 16], [129, 1, 16]),
    (W.BF16, 6, 2, 128, [77, 180], [1, 100]),
    (W.F32, 2, 2, 64, [20, 65, 6], [1, 30, 6]),
    (W.BF16, 8, 2, 128, [40, 700, 100, 300, 90], [1, 1, 64, 1, 90]),  # decode rows not contiguous
    (W.F16, 8, 2, 128, [300, 1, 64, 500, 40, 2], [1, 1, 37, 130, 0, 2]),
    # Few-row sequences (q_len * G <= 32) run on decode units, longer ones on
    # tiles: both sides of that bound, beside decode rows and a long chunk.
    (W.BF16, 8, 2, 128, [900, 70, 8, 33, 9, 300, 2000], [7, 8, 8, 9, 1, 200, 2]),  # G=4: 8 rows short, 9 tiles
    (W.BF16, 4, 4, 128, [513, 40, 600, 33, 80, 1], [2, 17, 32, 33, 1, 1]),          # MHA: up to 32 rows short
    (W.BF16, 32, 2, 64, [300, 301, 302, 5], [2, 3, 1, 5]),                           # G=16: only 2 rows short
    (W.F16, 64, 2, 128, [300, 40, 90], [2, 1, 40]),                                  # G=32: no short rows
]


@pytest.mark.parametrize("dtype,hq,hkv,d,kv,ql", MIXED_CASES)
def test_mixed_matches_oracle(dtype, hq, hkv, d, kv, ql):
    say(f"mixed {dtype} {hq}/{hkv} d={d} kv={kv} q={ql}")
    step = W.random_step(61, dtype, hq, hkv, d, kv, ql)
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.mixed()
    ref = A.attention_ragged(step.q, step.k_ctx, step.v_ctx)
    compare(out, ref, dtype, "mixed")


SPEC_CASES = [
    (8, 2, 128, [300, 5, 1000, 64, 17], 4),   # G=4, k=4 drafts; a 5-token context is all new rows
    (4, 4, 64, [129, 40, 700], 2),            # MHA, d=64, k=2
    (16, 2, 128, [90, 2048], 7),              # G=8, k=7
]


@pytest.mark.parametrize("hq,hkv,d,kv,k", SPEC_CASES)
def test_spec_verify_rows_match_oracle(hq, hkv, d, kv, k):
    """Multi-token decode rows (speculative verify: q_len = k + 1 per sequence)
    through the mixed entry point: row i of a sequence sees keys
    0 .. kv_len - k - 1 + i (bottom-right causal), against the oracle."""
    say(f"spec verify {hq}/{hkv} d={d} kv={kv} k={k}")
    step = W.random_step(66, W.BF16, hq, hkv, d, kv, [k + 1] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    out = ds.mixed()
    compare(out, A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "spec verify")


def test_spec_verify_last_row_equals_decode():
    """The last of the k + 1 verify rows and a one-row decode of the same
    token over the same keys agree within the bf16 tolerance (the verify rows
    are extra matrix-core columns of the decode unit)."""
    say("spec verify last row vs decode")
    kv, k = [700, 64, 1500], 4
    spec = W.random_step(67, W.BF16, 8, 2, 128, kv, [k + 1] * 3)
    sds = DeviceStep(spec)
    sds.fill_cache()
    rows = to_f64(sds.mixed())
    last = rows[np.cumsum([k + 1] * 3) - 1]
    dec = W.Step("d", W.BF16, 8, 2, 128, spec.kv_lens.copy(), np.ones(3, np.int64), spec.k_ctx, spec.v_ctx,
                 [q[-1:] for q in spec.q], spec.block_tables, spec.num_blocks)
    dds = DeviceStep(dec)
    dds.fill_cache()
    d_out = to_f64(dds.decode())
    err = np.abs(last - d_out)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


VERIFY_CASES = [
    (W.BF16, 8, 2, 128, [300, 5, 1000, 64, 17], 5, 0),   # G=4: 20 columns, 2 row groups
    (W.BF16, 32, 8, 128, [700, 2048, 129], 5, 3),        # 3 splits
    (W.BF16, 4, 4, 64, [129, 40, 700], 3, 1),            # MHA, d=64, whole-sequence units
    (W.BF16, 16, 2, 128, [90, 2048], 8, 0),              # G=8 x 8 rows: 64 columns, 4 row groups
    (W.BF16, 8, 8, 128, [33, 1500], 2, 0),               # G=1
    (W.F16, 8, 2, 128, [300, 77, 1000], 5, 0),
    (W.BF16, 4, 1, 64, [64, 200, 1000], 64, 0),          # the ABI's maximum of 64 rows: 256 columns, 8 row groups
    (W.BF16, 2, 2, 128, [70, 64], 64, 2),                # 64 rows, kv_len == nq for one sequence (all rows new)
]


@pytest.mark.parametrize("dtype,hq,hkv,d,kv,nq,splits", VERIFY_CASES)
def test_verify_paged_matches_oracle(dtype, hq, hkv, d, kv, nq, splits):
    """pka_attn_verify_paged: nq rows per sequence on the decode unit (rows x
    heads as matrix-core columns, each with its own causal limit)."""
    say(f"verify {dtype} {hq}/{hkv} d={d} kv={kv} nq={nq} splits={splits}")
    step = W.random_step(68, dtype, hq, hkv, d, kv, [nq] * len(kv))
    ds = DeviceStep(step)
    ds.fill_cache()
    q = ds.q.view(step.num_seqs, nq, hq, d)
    out = pka.attn_verify_paged(q, ds.cache, ds.block_tables, ds.kv_lens, int(step.max_kv_len),
                                num_splits=splits,
                                kv_lens_host=ds.kv_lens_host if nq % 2 else None)
    torch.cuda.synchronize()
    compare(out.view(-1, hq, d), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), dtype, "verify")


def test_verify_last_row_bitwise_equals_decode():
    """With whole-sequence units (num_splits = 1) the last verify row's matrix
    column sees exactly the decode row's blocks, keys and order: bit-equal."""
    say("verify last row vs decode, bitwise")
    kv, nq = [700, 64, 1500, 33], 5
    spec = W.random_step(69, W.BF16, 8, 2, 128, kv, [nq] * 4)
    sds = DeviceStep(spec)
    sds.fill_cache()
    q = sds.q.view(4, nq, 8, 128)
    rows = pka.attn_verify_paged(q, sds.cache, sds.block_tables, sds.kv_lens, int(spec.max_kv_len), num_splits=1)
    d_out = pka.attn_decode_paged(q[:, nq - 1].contiguous(), sds.cache, sds.block_tables, sds.kv_lens,
                                  int(spec.max_kv_len), num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(rows[:, nq - 1], d_out)


def test_mixed_many_decode_rows_without_order():
    """More decode rows than the host-built longest-first order holds (1024):
    the kernel falls back to locating the k-th decode row itself."""
    say("mixed: 1100 decode rows + 2 chunks (no dispatch order)")
    rng = np.random.default_rng(62)
    kv = np.concatenate([rng.integers(1, 60, 1100), [90, 200]])
    ql = np.concatenate([np.ones(1100, np.int64), [37, 130]])
    perm = rng.permutation(len(kv))        # chunks and decode rows interleaved
    step = W.random_step(63, W.BF16, 8, 2, 64, kv[perm], ql[perm])
    ds = DeviceStep(step)
    ds.fill_cache()
    compare(ds.mixed(), A.attention_ragged(step.q, step.k_ctx, step.v_ctx), W.BF16, "mixed, 1100 decode rows")


def test_mixed_equals_separate_decode_and_chunks():
    """Mixed-step rows match the oracle of the decode rows and the chunk rows
    computed as separate batches (the mixed step is their union)."""
    say("mixed = decode rows + chunk rows")
    step = W.random_step(62, W.BF16, 8, 2, 128, [900, 400, 1], [1, 257, 1])
    ds = DeviceStep(step)
    ds.fill_cache()
    out = to_f64(ds.mixed())
    cu = step.cu_q_lens
    for s in range(step.num_seqs):
        ref = A.attention_seq(step.q[s], step.k_ctx[s], step.v_ctx[s])
        err = np.abs(out[cu[s]:cu[s + 1]] - ref)
        assert err.max() <= 1e-2 and err.mean() <= 1e-3


def test_mixed_block_permutation_and_poison_bitwise():
    say("mixed block permutation / NaN poison")
    step = W.random_step(63, W.BF16, 8, 2, 128, [300, 1, 200, 77], [1, 1, 150, 1])
    a_ds = DeviceStep(step, fill=float("nan"))
    a_ds.fill_cache()
    a = a_ds.mixed()
    bt = _permuted_tables(step, 9)
    b_ds = DeviceStep(step, fill=0.0, block_tables=bt)
    allslots = []
    for s in range(step.num_seqs):
        p = np.arange(int(step.kv_lens[s]))
        allslots.append(bt[s][p // 16].astype(np.int64) * 16 + p % 16)
    cached = np.concatenate([allslots[s][: int(step.cached_lens[s])] for s in range(step.num_seqs)])
    new = np.concatenate([allslots[s][int(step.cached_lens[s]):] for s in range(step.num_seqs)])
    b_ds.append_cached(cached.astype(np.int32))
    b_ds.append_new(new.astype(np.int32))
    torch.cuda.synchronize()
    b = b_ds.mixed()
    assert torch.equal(a, b)


def test_decode_equals_last_prefill_row():
    """A decode row over kv_len keys matches the last row of a causal prefill
    of the same kv_len tokens (both against the oracle, and to each other
    within tolerance)."""
    say("decode vs last prefill row")
    lens = [90, 300]
    pre = W.random_step(64, W.BF16, 4, 4, 128, lens, lens)
    p_out = to_f64(DeviceStep(pre).prefill())
    dec = W.Step("d", W.BF16, 4, 4, 128, pre.kv_lens.copy(), np.ones(2, np.int64), pre.k_ctx, pre.v_ctx,
                 [q[-1:] for q in pre.q], pre.block_tables, pre.num_blocks)
    ds = DeviceStep(dec)
    ds.fill_cache()
    d_out = to_f64(ds.decode())
    last = p_out[np.cumsum(lens) - 1]
    assert np.abs(last - d_out).max() <= 1e-2
