"""Append fused with the rotary position embedding (pka_kv_append_rope) on the
GPU, against the oracle (oracle/rope.py, oracle/paged_layout.py, oracle/fp8.py).

The kernel evaluates each angle in fp64 and rotates in fp32, so every result
is within delta = 2^-22 (|a| + |b|) of the exact rotation y of its pair (a, b)
before the final rounding (derivation: cos and sin rounded to fp32, one
rounded product and one fused multiply-add, each at most 2^-24 relative, sum
at most 3 * 2^-24 (|a| + |b|)).  The checks:
* fp32 outputs: |out - y| <= delta;
* bf16, fp16 and fp8 outputs: out lies between the type's roundings of
  y - delta' and y + delta' (delta' adds 2^-24 |y| for forming the bounds in
  fp32), i.e. it is a correct rounding of some value within delta of y;
* V rows and every slot not written: bit for bit, as the plain append;
* skipped slots (negative, past the pool) write nothing; q rows are rotated
  whatever the slot.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import fp8 as F8
from oracle import paged_layout as L
from oracle import rope as R
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import FP8_POISON, DeviceStep, compare, dev, pool_bits, say, to_f64, value_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


TORCH = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}


def pair_magnitude(x: np.ndarray, style: int) -> np.ndarray:
    """|a| + |b| of the rotation pair each element belongs to."""
    a, b = R.pair_dims(x.shape[-1], style)
    m = np.empty(x.shape, np.float64)
    s = np.abs(x[..., a]).astype(np.float64) + np.abs(x[..., b])
    m[..., a] = s
    m[..., b] = s
    return m


def bracket(y, mag):
    """fp32 bounds lo <= y - delta, hi >= y + delta."""
    dp = 2.0 ** -22 * mag + 2.0 ** -24 * np.abs(y)
    return (y - dp).astype(np.float32), (y + dp).astype(np.float32)


def round_to(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == W.F16:
        return x32.astype(np.float16).astype(np.float64)
    if dtype == W.BF16:
        return W.round_to_dtype(x32, W.BF16).astype(np.float64)
    return x32.astype(np.float64)


def check_rotated(out: np.ndarray, y: np.ndarray, mag: np.ndarray, dtype: str, what: str, scale=None):
    """out: values as stored (fp8: decoded codes times scale)."""
    if dtype == W.F32 and scale is None:
        err = np.abs(out - y) - 2.0 ** -22 * mag
        assert err.max() <= 0, (what, float(err.max()))
        return
    lo, hi = bracket(y, mag)
    if scale is None:
        rlo, rhi = round_to(lo, dtype), round_to(hi, dtype)
    else:  # fp8 codes of value / scale, per head (last-but-one axis)
        rlo = np.empty(y.shape)
        rhi = np.empty(y.shape)
        for g in range(y.shape[-2]):
            rlo[..., g, :] = F8.dequantize(F8.quantize(lo[..., g, :], scale[g]), scale[g])
            rhi[..., g, :] = F8.dequantize(F8.quantize(hi[..., g, :], scale[g]), scale[g])
    # Rounding is monotone: a rounding of any value in [y - delta, y + delta] lies in [rlo, rhi]
    # (one value, or two adjacent ones, except where cancellation makes |y| << |a| + |b|).
    ok = (out >= rlo) & (out <= rhi)
    say(f"{what}: {np.sum(~ok)} of {out.size} outside the bound; {np.mean(rlo == rhi):.6f} of bounds pin one value")
    assert ok.all(), what


def make_case(seed, dtype, hkv, hq, d, T, num_blocks, max_pos=32767):
    rng = np.random.default_rng(seed)
    slots = rng.permutation(num_blocks * 16)[:T].astype(np.int32)
    slots[::7] = -1                                   # padding tokens
    if T > 3:
        slots[3] = num_blocks * 16 + 5                # past the pool: skipped
    pos = rng.integers(0, max_pos + 1, T).astype(np.int32)
    pos[:2] = [0, 1]
    k = W.round_to_dtype(rng.standard_normal((T, hkv, d)).astype(np.float32), dtype)
    v = W.round_to_dtype(rng.standard_normal((T, hkv, d)).astype(np.float32), dtype)
    q = W.round_to_dtype(rng.standard_normal((T, hq, d)).astype(np.float32) * 2, dtype)
    return slots, pos, k, v, q


def placed(rows: np.ndarray, slots: np.ndarray, num_blocks: int, hkv: int, d: int):
    """Pool-shaped fp64 array holding rows at their slots (NaN elsewhere), via the layout oracle."""
    n = num_blocks * hkv * 16 * d
    empty = np.full(n, np.nan)
    p, _ = L.append(empty, empty, rows.astype(np.float64), rows.astype(np.float64),
                    np.where(slots < num_blocks * 16, slots, -1), hkv, d)
    return p


CASES = [
    (W.BF16, 8, 32, 128, R.HALF, 10000.0),
    (W.BF16, 4, 4, 64, R.INTERLEAVED, 10000.0),
    (W.F16, 8, 16, 128, R.INTERLEAVED, 1e6),
    (W.F16, 2, 8, 64, R.HALF, 500000.0),
    (W.F32, 2, 4, 128, R.HALF, 10000.0),
    (W.F32, 4, 4, 64, R.INTERLEAVED, 100.0),
]


@pytest.mark.parametrize("dtype,hkv,hq,d,style,base", CASES)
def test_append_rope_matches_oracle(dtype, hkv, hq, d, style, base):
    say(f"append rope {dtype} hkv={hkv} hq={hq} d={d} style={style} base={base}")
    nb, T = 24, 150
    slots, pos, k, v, q = make_case(81, dtype, hkv, hq, d, T, nb)
    fill = 0.0 if dtype == W.F32 else float("nan")
    cache = pka.KVCache.allocate(nb, hkv, d, TORCH[dtype], fill=fill)
    k0, v0 = pool_bits(cache)
    q_dev = dev(q, TORCH[dtype])
    q_out = torch.empty_like(q_dev)
    pka.kv_append_rope(cache, dev(k, TORCH[dtype]), dev(v, TORCH[dtype]), dev(slots), dev(pos), q=q_dev,
                       q_out=q_out, rope_base=base, rope_style=style)
    torch.cuda.synchronize()
    k1, v1 = pool_bits(cache)
    valid = np.where(slots < nb * 16, slots, -1)
    # V and untouched K slots: bit for bit
    _, ev = L.append(k0, v0, value_bits(k, dtype), value_bits(v, dtype), valid, hkv, d)
    assert np.array_equal(v1, ev)
    km, _ = L.written_mask(nb, valid, hkv, d)
    assert np.array_equal(k1[~km], k0[~km])
    # rotated K in the pool
    yk = R.rope(k, pos, base, style)
    y_pool, m_pool = placed(yk, slots, nb, hkv, d), placed(pair_magnitude(k, style), slots, nb, hkv, d)
    k_vals = to_f64(cache.k_pool)
    check_rotated(k_vals[km], y_pool[km], m_pool[km], dtype, "rotated K")
    # rotated q, every token
    check_rotated(to_f64(q_out).reshape(q.shape), R.rope(q, pos, base, style), pair_magnitude(q, style), dtype,
                  "rotated q")
    assert torch.equal(q_dev.cpu(), torch.from_numpy(q).to(TORCH[dtype]))   # input untouched


def test_append_rope_in_place_q_and_no_q():
    say("append rope: q in place, and K only")
    dtype, hkv, hq, d, nb, T = W.BF16, 4, 8, 128, 16, 60
    slots, pos, k, v, q = make_case(82, dtype, hkv, hq, d, T, nb)
    c1 = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=0.0)
    c2 = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=0.0)
    qa = dev(q, torch.bfloat16)
    qb = dev(q, torch.bfloat16)
    q_sep = torch.empty_like(qa)
    args = (dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(slots), dev(pos))
    pka.kv_append_rope(c1, *args, q=qa, q_out=q_sep)
    pka.kv_append_rope(c2, *args, q=qb)             # in place
    torch.cuda.synchronize()
    assert torch.equal(q_sep.view(torch.int16), qb.view(torch.int16))
    c3 = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=0.0)
    pka.kv_append_rope(c3, *args)                   # no q rows
    torch.cuda.synchronize()
    for a, b in ((c1, c2), (c1, c3)):
        assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
        assert torch.equal(a.v_pool.view(torch.int16), b.v_pool.view(torch.int16))


def test_append_rope_position_zero_is_plain_append():
    """At position 0 every rotation is the identity: the pools equal the plain
    append's bit for bit and q is unchanged."""
    say("append rope at position 0")
    dtype, hkv, hq, d, nb, T = W.BF16, 8, 8, 128, 16, 100
    slots, _, k, v, q = make_case(83, dtype, hkv, hq, d, T, nb)
    pos = np.zeros(T, np.int32)
    c1 = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=float("nan"))
    c2 = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=float("nan"))
    qd = dev(q, torch.bfloat16)
    pka.kv_append_rope(c1, dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(slots), dev(pos), q=qd,
                       rope_style=R.INTERLEAVED)
    pka.kv_append(c2, dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(slots))
    torch.cuda.synchronize()
    assert torch.equal(c1.k_pool.view(torch.int16), c2.k_pool.view(torch.int16))
    assert torch.equal(c1.v_pool.view(torch.int16), c2.v_pool.view(torch.int16))
    assert torch.equal(qd.cpu(), torch.from_numpy(q).to(torch.bfloat16))


@pytest.mark.parametrize("act,style", [(W.BF16, R.HALF), (W.F16, R.INTERLEAVED)])
def test_append_rope_fp8_pools(act, style):
    say(f"append rope fp8 pools act={act} style={style}")
    hkv, hq, d, nb, T = 8, 32, 128, 24, 150
    slots, pos, k, v, q = make_case(84, act, hkv, hq, d, T, nb)
    ks, vs = W.fp8_scales(85, hkv), W.fp8_scales(86, hkv)
    cache = pka.KVCache.allocate(nb, hkv, d, torch.uint8, fill=FP8_POISON, act_dtype=TORCH[act],
                                 k_scale=dev(ks), v_scale=dev(vs))
    k0, v0 = pool_bits(cache)
    q_dev = dev(q, TORCH[act])
    pka.kv_append_rope(cache, dev(k, TORCH[act]), dev(v, TORCH[act]), dev(slots), dev(pos), q=q_dev,
                       rope_style=style)
    torch.cuda.synchronize()
    k1, v1 = pool_bits(cache)
    valid = np.where(slots < nb * 16, slots, -1)
    v_codes = np.empty(v.shape, np.uint8)
    for g in range(hkv):
        v_codes[:, g, :] = F8.quantize(v[:, g, :], vs[g])
    _, ev = L.append(k0, v0, np.zeros(v.shape, np.uint8), v_codes, valid, hkv, d)
    assert np.array_equal(v1, ev)
    km, _ = L.written_mask(nb, valid, hkv, d)
    assert np.array_equal(k1[~km], k0[~km])
    # decoded K codes, placed per head: compare head by head through the pool layout
    yk = R.rope(k, pos, base=10000.0, style=style)
    mk = pair_magnitude(k, style)
    rows = []
    for t in np.nonzero(valid >= 0)[0]:
        b, o = valid[t] // 16, valid[t] % 16
        idx = np.stack([L.k_index(b, g, o, np.arange(d), hkv, d) for g in range(hkv)])
        rows.append(np.stack([F8.dequantize(k1[idx[g]], ks[g]) for g in range(hkv)]))
    got = np.stack(rows)
    sel = valid >= 0
    check_rotated(got, yk[sel], mk[sel], act, "rotated K, fp8 codes", scale=ks)
    check_rotated(to_f64(q_dev).reshape(q.shape), R.rope(q, pos, 10000.0, style), pair_magnitude(q, style), act,
                  "rotated q (fp8 cache)")


def test_rope_then_decode_matches_oracle():
    """End to end: the step's keys appended with RoPE at their positions, the
    new token's q rotated in the same call, then paged decode, against the
    oracle attending with rotated q and K."""
    from oracle import attention as A
    say("rope append + decode vs oracle")
    step = W.random_step(87, W.BF16, 8, 2, 128, [300, 17, 1000], [1, 1, 1])
    ds = DeviceStep(step, fill=0.0)
    kc, vc = step.cached_kv()
    kn, vn = step.new_kv()
    cpos = np.concatenate([np.arange(int(c)) for c in step.cached_lens]).astype(np.int32)
    npos = (step.kv_lens - 1).astype(np.int32)
    pka.kv_append_rope(ds.cache, dev(kc, torch.bfloat16), dev(vc, torch.bfloat16),
                       dev(step.cached_slot_mapping()), dev(cpos))
    q_rot = torch.empty_like(ds.q)
    pka.kv_append_rope(ds.cache, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), dev(step.new_slot_mapping()),
                       dev(npos), q=ds.q, q_out=q_rot)
    torch.cuda.synchronize()
    ds.q = q_rot
    out = ds.decode()
    # The cache holds the rotated keys rounded to bf16 and attention takes the rotated q in bf16:
    # the oracle attends over the exact rotations rounded to bf16 (nearest-even).
    def rot16(x, p):
        return W.round_to_dtype(R.rope(x, p, 10000.0, R.HALF).astype(np.float32), W.BF16)
    k_rot = [rot16(k, np.arange(k.shape[0])) for k in step.k_ctx]
    q_ref = [rot16(qq, npos[s:s + 1]) for s, qq in enumerate(step.q)]
    compare(out, A.attention_ragged(q_ref, k_rot, step.v_ctx), W.BF16, "rope + decode")


def test_append_rope_prefill_ragged_4096():
    """The benchmark's RoPE append at full size: the 4096 tokens of the ragged
    prefill batch (32/32 heads, d = 128, bf16) at positions 0..L-1 of each
    prompt, q rotated in place; every K row gathered through the block tables
    and every q row against the oracle's rotation, V bit for bit."""
    say("append rope, ragged prefill 4096 tokens")
    step = W.prefill_ragged(3)
    ds = DeviceStep(step, fill=0.0)
    kn, vn = step.new_kv()
    pos = np.concatenate([np.arange(int(l)) for l in step.q_lens]).astype(np.int32)
    pka.kv_append_rope(ds.cache, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), dev(step.new_slot_mapping()),
                       dev(pos), q=ds.q)
    torch.cuda.synchronize()
    k1, v1 = pool_bits(ds.cache)
    got_k, want_k, mag_k = [], [], []
    for s in range(step.num_seqs):
        kg, vg = L.gather(k1, v1, step.block_tables[s], int(step.kv_lens[s]), 32, 128)
        assert np.array_equal(vg, value_bits(step.v_ctx[s], W.BF16))
        got_k.append(W.bf16_bits_to_f32(kg).astype(np.float64))
        want_k.append(R.rope(step.k_ctx[s], np.arange(int(step.kv_lens[s])), 10000.0, R.HALF))
        mag_k.append(pair_magnitude(step.k_ctx[s], R.HALF))
    check_rotated(np.concatenate(got_k), np.concatenate(want_k), np.concatenate(mag_k), W.BF16, "rotated K (4096)")
    q = step.packed_q()
    check_rotated(to_f64(ds.q).reshape(q.shape), R.rope(q, pos, 10000.0, R.HALF), pair_magnitude(q, R.HALF),
                  W.BF16, "rotated q (4096)")
