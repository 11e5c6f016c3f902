"""Seeded synthetic ragged batches for paged-KV attention.

This module only *draws inputs*: sequence lengths, a block allocation, slot
numbers and Q/K/V values.  It contains none of the attention arithmetic, so
both the fp64 oracle (under ``oracle/``) and the HIP path can be fed from it
without sharing any compute code.

Shapes follow the serving defaults the pages print: a prefill token budget
of 4096 (``max_batch_prefill_tokens``), a total-token cap of 2048 per request
(``max_total_tokens``), 128 concurrent requests (``max_concurrent_requests``)
-- TGI architecture page (data-sketchers wiki), router options -- and head
dimension 128 (BlitzScale documentation, "Build": the attention kernels are
generated for head dim 128).  The block allocator that hands out fixed-size
KV blocks lives in the router (TGI architecture page, "The Router": a queue,
a scheduler and a block allocator); here it is a seeded random permutation of
the pool, so block tables are fragmented.

Conventions (readings where the pages are silent):
  * ``kv_len`` counts every key a sequence attends in this step, including
    the tokens appended in this step; ``q_len`` is the number of new tokens.
    The first ``kv_len - q_len`` tokens are already cached.
  * A query row ``i`` of a sequence sits at absolute position
    ``kv_len - q_len + i``.
  * Block size is 16 tokens; token ``p`` of a sequence lives in block
    ``block_table[p // 16]`` at offset ``p % 16``; its slot number is
    ``block * 16 + offset``.
  * bf16 values are produced by rounding float32 draws to nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) -- input preparation only.
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the uint16 bits.

    Inputs must be finite.  The rounding adds 0x7FFF plus the lowest kept bit
    to the float32 bit pattern and truncates the low 16 bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's conversion: nearest-even)
    and return the uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values exactly representable in ``dtype``."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(bf16_bits(x))
    if dtype == F16:
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# One attention step over a ragged batch.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Step:
    """One forward step of one attention layer over a ragged batch.

    Arrays hold float32 values that are exact in ``dtype``.
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_lens: np.ndarray          # int64 [B]   keys attended (cached + new)
    q_lens: np.ndarray           # int64 [B]   new tokens this step
    k_ctx: List[np.ndarray]      # per sequence float32 [kv_len][Hkv][d]
    v_ctx: List[np.ndarray]      # per sequence float32 [kv_len][Hkv][d]
    q: List[np.ndarray]          # per sequence float32 [q_len][Hq][d]
    block_tables: np.ndarray     # int32 [B][max_blocks]  (-1 = unused entry)
    num_blocks: int              # pool size in blocks
    sigma: float = 1.0

    # ---- derived integer structure (no attention arithmetic) -------------
    @property
    def num_seqs(self) -> int:
        return int(len(self.kv_lens))

    @property
    def cached_lens(self) -> np.ndarray:
        return self.kv_lens - self.q_lens

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.q_lens)
        return cu

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def slots(self, seq: int, start: int, stop: int) -> np.ndarray:
        """Slot numbers of positions ``start..stop-1`` of sequence ``seq``."""
        p = np.arange(start, stop, dtype=np.int64)
        blk = self.block_tables[seq][p // BLOCK_SIZE].astype(np.int64)
        return (blk * BLOCK_SIZE + p % BLOCK_SIZE).astype(np.int32)

    def cached_slot_mapping(self) -> np.ndarray:
        """Slots of every cached (pre-existing) token, sequences in order."""
        parts = [self.slots(s, 0, int(self.cached_lens[s])) for s in range(self.num_seqs)]
        return np.concatenate(parts) if parts else np.zeros(0, np.int32)

    def new_slot_mapping(self) -> np.ndarray:
        """Slots of this step's new tokens, packed like ``cu_q_lens``."""
        parts = [self.slots(s, int(self.cached_lens[s]), int(self.kv_lens[s]))
                 for s in range(self.num_seqs)]
        return np.concatenate(parts) if parts else np.zeros(0, np.int32)

    def cached_kv(self):
        """Packed K and V of cached tokens, [N][Hkv][d] each."""
        d, h = self.head_dim, self.num_kv_heads
        ks = [self.k_ctx[s][: int(self.cached_lens[s])] for s in range(self.num_seqs)]
        vs = [self.v_ctx[s][: int(self.cached_lens[s])] for s in range(self.num_seqs)]
        if not ks:
            z = np.zeros((0, h, d), np.float32)
            return z, z
        return np.concatenate(ks), np.concatenate(vs)

    def new_kv(self):
        """Packed K and V of this step's new tokens, [total_q][Hkv][d] each."""
        d, h = self.head_dim, self.num_kv_heads
        ks = [self.k_ctx[s][int(self.cached_lens[s]):] for s in range(self.num_seqs)]
        vs = [self.v_ctx[s][int(self.cached_lens[s]):] for s in range(self.num_seqs)]
        if not ks:
            z = np.zeros((0, h, d), np.float32)
            return z, z
        return np.concatenate(ks), np.concatenate(vs)

    def packed_q(self) -> np.ndarray:
        if not self.q:
            return np.zeros((0, self.num_q_heads, self.head_dim), np.float32)
        return np.concatenate(self.q)

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max()) if self.num_seqs else 0


def _alloc_blocks(rng: np.random.Generator, kv_lens: np.ndarray, num_blocks: int,
                  order: Optional[List[np.ndarray]] = None):
    """Hand out blocks from a seeded permutation of the pool, in sequence order.

    ``order`` optionally gives, per allocation round, the number of tokens each
    sequence needs to cover in that round (used for prefill-then-decode, where
    the decode step takes its extra blocks after every prefill allocation).
    """
    perm = rng.permutation(num_blocks).astype(np.int32)
    nblk = (kv_lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    max_blocks = int(max(1, nblk.max())) if len(kv_lens) else 1
    tables = np.full((len(kv_lens), max_blocks), -1, dtype=np.int32)
    cursor = 0
    have = np.zeros(len(kv_lens), dtype=np.int64)
    rounds = order if order is not None else [kv_lens]
    for need_tokens in rounds:
        need = (np.asarray(need_tokens) + BLOCK_SIZE - 1) // BLOCK_SIZE
        for s in range(len(kv_lens)):
            extra = int(need[s] - have[s])
            if extra > 0:
                tables[s, have[s]: have[s] + extra] = perm[cursor: cursor + extra]
                cursor += extra
                have[s] += extra
    if cursor > num_blocks:
        raise ValueError("pool too small")
    return tables


def _pool_size(kv_lens: np.ndarray, spare: float = 0.125) -> int:
    used = int(((kv_lens + BLOCK_SIZE - 1) // BLOCK_SIZE).sum())
    return max(1, used + int(np.ceil(used * spare)))


def _draw_values(rng, kv_lens, q_lens, hq, hkv, d, sigma, dtype):
    k_ctx, v_ctx, q = [], [], []
    for s in range(len(kv_lens)):
        kl, ql = int(kv_lens[s]), int(q_lens[s])
        k = rng.standard_normal((kl, hkv, d), dtype=np.float32) * np.float32(sigma)
        v = rng.standard_normal((kl, hkv, d), dtype=np.float32) * np.float32(sigma)
        qq = rng.standard_normal((ql, hq, d), dtype=np.float32) * np.float32(sigma)
        k_ctx.append(round_to_dtype(k, dtype))
        v_ctx.append(round_to_dtype(v, dtype))
        q.append(round_to_dtype(qq, dtype))
    return k_ctx, v_ctx, q


def make_step(name, dtype, hq, hkv, d, kv_lens, q_lens, seed, sigma=1.0,
              num_blocks=None, alloc_rounds=None, rng=None) -> Step:
    """Build a step from explicit lengths; draws blocks then values from ``seed``.

    Draw order: block permutation, then for each sequence K, V, Q.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if np.any(q_lens > kv_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= kv_len")
    nb = num_blocks if num_blocks is not None else _pool_size(kv_lens)
    tables = _alloc_blocks(rng, kv_lens, nb, alloc_rounds)
    k_ctx, v_ctx, q = _draw_values(rng, kv_lens, q_lens, hq, hkv, d, sigma, dtype)
    return Step(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                kv_lens=kv_lens, q_lens=q_lens, k_ctx=k_ctx, v_ctx=v_ctx, q=q,
                block_tables=tables, num_blocks=nb, sigma=sigma)


def fp8_scales(seed: int, hkv: int, sigma: float = 1.0, lo: float = 2.5, hi: float = 8.0) -> np.ndarray:
    """Seeded per-kv-head fp32 scales for an fp8 (E4M3, largest finite 448)
    cache: scale[g] = sigma * u / 448 with u uniform in [lo, hi), so a head
    stores values up to about u standard deviations without saturating (the
    smaller u, the more of the normal tail saturates).  Input drawing only."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(lo, hi, size=hkv)
    return (np.float32(sigma) * u.astype(np.float32) / np.float32(448.0)).astype(np.float32)


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------
def tiny_fp32(seed: int = 1):
    """Tiny ragged fp32 batch: prompts {5,17,32,64}, 2/2 heads, d=64, 16-block pool.

    Returns ``(prefill, decode)``: one causal prefill over the four prompts,
    then one decode step per sequence (kv_len = prompt + 1).  Both steps share
    the block tables (decode blocks are taken after all prefill blocks) and
    the K/V/Q values (the decode row is the prompt's next position).
    """
    rng = np.random.default_rng(seed)
    prompts = np.array([5, 17, 32, 64], dtype=np.int64)
    full = prompts + 1
    tables = _alloc_blocks(rng, full, 16, order=[prompts, full])
    hq = hkv = 2
    d = 64
    k_ctx, v_ctx, q_all = _draw_values(rng, full, full, hq, hkv, d, 1.0, F32)
    pre = Step("tiny_fp32_prefill", F32, hq, hkv, d, prompts.copy(), prompts.copy(),
               [k[:-1] for k in k_ctx], [v[:-1] for v in v_ctx], [qq[:-1] for qq in q_all],
               tables, 16, 1.0)
    dec = Step("tiny_fp32_decode", F32, hq, hkv, d, full.copy(), np.ones(4, np.int64),
               k_ctx, v_ctx, [qq[-1:] for qq in q_all], tables, 16, 1.0)
    return pre, dec


def decode_mha_7b(seed: int = 2, batch: int = 64, lo: int = 128, hi: int = 2048, dtype: str = BF16) -> Step:
    """Decode-only continuous batch, bf16 (or ``dtype``): 64 sequences, kv_len ~
    U{128..2048}, 32/32 heads, d=128, values N(0, 0.5^2), one new token per
    sequence."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    name = "decode_mha_b64_ctx128-2048" + ("" if dtype == BF16 else "_" + dtype)
    return make_step(name, dtype, 32, 32, 128, kv, np.ones(batch, np.int64), seed, sigma=0.5, rng=rng)


def prefill_lengths(rng: np.random.Generator, budget: int = 4096, lo: int = 16, hi: int = 1024):
    """Prompt lengths ~ U{lo..hi} drawn until the total reaches ``budget``; the
    last draw is clipped so the total is exactly ``budget``."""
    lens = []
    total = 0
    while total < budget:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, budget - total)
        lens.append(L)
        total += L
    return np.array(lens, dtype=np.int64)


def prefill_ragged(seed: int = 3, budget: int = 4096) -> Step:
    """Ragged prefill batch, bf16: prompts ~ U{16..1024} packed to 4096 tokens,
    32/32 heads, d=128, causal, values N(0,1); K/V also appended into blocks."""
    rng = np.random.default_rng(seed)
    lens = prefill_lengths(rng, budget)
    return make_step("prefill_ragged_4096", BF16, 32, 32, 128, lens, lens.copy(), seed, rng=rng)


def mixed_gqa(seed: int = 4, n_decode: int = 128, lo: int = 256, hi: int = 2048,
              n_chunks: int = 2, chunk: int = 1024, cached: int = 1024) -> Step:
    """Mixed chunked-prefill + decode step, bf16 GQA 32/8, d=128: 128 decode
    rows (kv_len ~ U{256..2048}) then 2 chunks of 1024 rows on 1024 cached
    tokens; values N(0,1)."""
    rng = np.random.default_rng(seed)
    kv_dec = rng.integers(lo, hi + 1, size=n_decode).astype(np.int64)
    kv = np.concatenate([kv_dec, np.full(n_chunks, cached + chunk, np.int64)])
    ql = np.concatenate([np.ones(n_decode, np.int64), np.full(n_chunks, chunk, np.int64)])
    return make_step("mixed_gqa_128dec_2x1024chunk", BF16, 32, 8, 128, kv, ql, seed, rng=rng)


def long_decode_gqa(seed: int = 5, batch: int = 16, ctx: int = 32768) -> Step:
    """Long-context decode, bf16 GQA 64/8, d=128: 16 sequences at kv_len 32768,
    fully shuffled pool, values N(0,1)."""
    rng = np.random.default_rng(seed)
    kv = np.full(batch, ctx, np.int64)
    return make_step("long_decode_gqa_b16_ctx32768", BF16, 64, 8, 128, kv, np.ones(batch, np.int64),
                     seed, rng=rng)


def spec_verify_gqa(seed: int = 6, batch: int = 64, draft: int = 4, lo: int = 128, hi: int = 2048) -> Step:
    """Speculative-verify step, bf16 GQA 32/8, d=128: 64 sequences, each with
    draft + 1 = 5 new query rows (the last accepted token and 4 draft tokens)
    at the end of a context of kv_len ~ U{128..2048} tokens (new ones
    included); values N(0,1)."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    ql = np.full(batch, draft + 1, np.int64)
    return make_step("spec_verify_gqa_b64_k4", BF16, 32, 8, 128, kv, ql, seed, rng=rng)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "decode_mha": decode_mha_7b,
    "prefill_ragged": prefill_ragged,
    "mixed_gqa": mixed_gqa,
    "long_decode_gqa": long_decode_gqa,
    "spec_verify_gqa": spec_verify_gqa,
}


def random_step(seed: int, dtype: str, hq: int, hkv: int, d: int, kv_lens, q_lens,
                sigma: float = 1.0, spare: float = 0.125) -> Step:
    """Small step with explicit lengths for tests (pool gets ``spare`` extra)."""
    kv_lens = np.asarray(kv_lens, np.int64)
    return make_step(f"random_{seed}", dtype, hq, hkv, d, kv_lens, q_lens, seed, sigma=sigma,
                     num_blocks=_pool_size(kv_lens, spare))
