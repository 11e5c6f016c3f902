"""KV-pool layout formula: the oracle for the slot-mapped append and the
block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring): not for the product path.

The pages say only that the model server reserves a GPU region for the KV
cache (BlitzScale documentation, server components: CacheManager) and that
fixed-size blocks are handed out by the router's block allocator (TGI
architecture page, "The Router").  The layout is therefore this library's own
definition, stated in its public header; the oracle writes it out plainly:

  block size 16; a token with slot ``s`` lives in block ``b = s // 16`` at
  offset ``t = s % 16``; the token at position ``p`` of a sequence whose
  block-table row is ``row`` has slot ``row[p // 16] * 16 + p % 16``.  K and V pools share one layout,
  ``[num_blocks][Hkv][16][d]``: element (b, head g, offset t, dim i) is at
      ((b * Hkv + g) * 16 + t) * d + i

Pools are handled as flat arrays of raw element bits (uint16 for bf16,
uint32 for fp32), so appends are checked byte for byte.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def slot_of(block_row, position):
    """Slot of the token at ``position`` (int or int array) of a sequence whose
    block-table row is ``block_row``: the block holding that position, times
    16, plus the offset inside it."""
    p = np.asarray(position, np.int64)
    return np.asarray(block_row, np.int64)[p // BLOCK] * BLOCK + p % BLOCK


def k_index(b, g, t, i, hkv: int, d: int):
    """Flat K-pool element index (works on ints or int64 arrays); the layout is
    the same for every element size."""
    return ((b * hkv + g) * BLOCK + t) * d + i


def v_index(b, g, t, i, hkv: int, d: int):
    """Flat V-pool element index (same layout as K)."""
    return ((b * hkv + g) * BLOCK + t) * d + i


def append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
           slot_mapping: np.ndarray, hkv: int, d: int):
    """Return copies of the pools with each new token written at its slot.

    ``k_new, v_new``: ``[T][Hkv][d]`` raw element bits, same dtype as the pools.
    A negative slot means "skip this token".  Element (token, g, i) goes to
    the pool index of (slot // 16, g, slot % 16, i); the tokens are taken a
    few thousand at a time so that large pools stay quick to build.
    """
    kp = k_pool.copy()
    vp = v_pool.copy()
    slots = np.asarray(slot_mapping, np.int64)
    g = np.arange(hkv, dtype=np.int64)[None, :, None]
    dims = np.arange(d, dtype=np.int64)[None, None, :]
    step = 4096
    for t0 in range(0, len(slots), step):
        tok = t0 + np.nonzero(slots[t0:t0 + step] >= 0)[0]
        b = (slots[tok] // BLOCK)[:, None, None]
        t = (slots[tok] % BLOCK)[:, None, None]
        kp[k_index(b, g, t, dims, hkv, d)] = k_new[tok]
        vp[v_index(b, g, t, dims, hkv, d)] = v_new[tok]
    return kp, vp


def gather(k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray, kv_len: int,
           hkv: int, d: int):
    """Read one sequence's K and V, ``[kv_len][Hkv][d]`` each, through its block table."""
    dims = np.arange(d, dtype=np.int64)
    k = np.empty((kv_len, hkv, d), dtype=k_pool.dtype)
    v = np.empty((kv_len, hkv, d), dtype=v_pool.dtype)
    for p in range(kv_len):
        b = int(block_table[p // BLOCK])
        t = p % BLOCK
        for g in range(hkv):
            k[p, g] = k_pool[k_index(b, g, t, dims, hkv, d)]
            v[p, g] = v_pool[v_index(b, g, t, dims, hkv, d)]
    return k, v


def written_mask(num_blocks: int, slot_mapping: np.ndarray, hkv: int, d: int):
    """Boolean masks over the flat pools: True where some slot was written."""
    n = num_blocks * hkv * BLOCK * d
    km = np.zeros(n, bool)
    vm = np.zeros(n, bool)
    dims = np.arange(d, dtype=np.int64)
    for slot in np.asarray(slot_mapping, np.int64):
        if slot < 0:
            continue
        b, t = slot // BLOCK, slot % BLOCK
        for g in range(hkv):
            km[k_index(b, g, t, dims, hkv, d)] = True
            vm[v_index(b, g, t, dims, hkv, d)] = True
    return km, vm


def copy_blocks(k_src: np.ndarray, v_src: np.ndarray, k_dst: np.ndarray, v_dst: np.ndarray,
                pairs: np.ndarray, hkv: int, d: int, src_blocks: int, dst_blocks: int):
    """Return copies of the destination pools after copying whole blocks.

    For each (source block, destination block) pair, every element of the
    source block -- all heads ``g``, offsets ``t`` and dims ``i`` -- is written
    to the same (g, t, i) of the destination block.  Pairs with an id outside
    ``[0, src_blocks)`` / ``[0, dst_blocks)`` are skipped.  The pairs are
    applied in order (the library requires distinct destinations that are not
    also sources, where the order cannot matter).
    """
    kd = k_dst.copy()
    vd = v_dst.copy()
    g, t, i = np.meshgrid(np.arange(hkv), np.arange(BLOCK), np.arange(d), indexing="ij")
    g, t, i = g.ravel().astype(np.int64), t.ravel().astype(np.int64), i.ravel().astype(np.int64)
    for sb, db in np.asarray(pairs, np.int64).reshape(-1, 2):
        if not (0 <= sb < src_blocks and 0 <= db < dst_blocks):
            continue
        kd[k_index(db, g, t, i, hkv, d)] = k_src[k_index(sb, g, t, i, hkv, d)]
        vd[v_index(db, g, t, i, hkv, d)] = v_src[v_index(sb, g, t, i, hkv, d)]
    return kd, vd
