"""fp64 definition of causal attention over ragged sequences.

TEST INFRASTRUCTURE ONLY (see the package docstring): not for the product path.

Definition followed (the pages name the kernels -- flash-attention and Paged
Attention, TGI overview note (dongnian.icu), feature list -- but print no
formula; this is the plain definition of scaled dot-product attention with a
causal mask, which those kernels compute exactly up to rounding order):

  For a sequence with ``kv_len`` keys of which ``q_len`` are new this step,
  query row ``i`` sits at absolute position ``p = kv_len - q_len + i`` and
  attends keys ``j = 0..p`` (its own key included: the new key/value is
  written to the cache before attention).  For query head ``h`` the keys and
  values come from KV head ``h // (Hq // Hkv)``.

      z_j = scale * <q, k_j>,   w_j = exp(z_j - max z) / sum_k exp(z_k - max z),
      o   = sum_j w_j v_j,      scale = 1/sqrt(d) unless given.

  Prefill is the case ``q_len == kv_len`` (the whole prompt, TGI router
  deep-dive (xxmr.cn), section "Prefill, Decode and past key values"); decode
  is ``q_len == 1`` over the cached past keys/values; a prefill chunk is
  ``0 < q_len < kv_len`` and runs in the same forward as the decodes (same
  article, the prefill-chunking paragraph of the scheduling-loop section).
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np


def default_scale(head_dim: int) -> float:
    """1/sqrt(d)."""
    return 1.0 / math.sqrt(head_dim)


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
                scale: float, return_weights: bool = False):
    """Attention of query rows ``q [n][d]`` over ``k, v [kv_len][d]``.

    Row ``r`` sees keys ``0..positions[r]`` (inclusive).  fp64 throughout.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    positions = np.asarray(positions, np.int64)
    n, kv = q.shape[0], k.shape[0]
    if n == 0:
        out = np.zeros((0, v.shape[1]))
        return (out, np.zeros((0, kv))) if return_weights else out
    if np.any(positions < 0) or np.any(positions >= kv):
        raise ValueError("query position outside the key range")
    z = (q @ k.T) * scale                                   # [n][kv]
    visible = np.arange(kv)[None, :] <= positions[:, None]  # causal: j <= p
    z = np.where(visible, z, -np.inf)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)                                    # exp(-inf) = 0 for hidden keys
    w = e / e.sum(axis=1, keepdims=True)
    out = w @ v
    return (out, w) if return_weights else out


def attention_seq(q_seq: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                  scale: float | None = None) -> np.ndarray:
    """One sequence: ``q_seq [q_len][Hq][d]`` over ``k_seq, v_seq [kv_len][Hkv][d]``.

    Returns ``[q_len][Hq][d]`` in fp64.  Rows are the last ``q_len`` positions.
    """
    q_len, hq, d = q_seq.shape
    kv_len, hkv, _ = k_seq.shape
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if q_len > kv_len:
        raise ValueError("q_len > kv_len")
    scale = default_scale(d) if scale is None else scale
    group = hq // hkv
    pos = np.arange(kv_len - q_len, kv_len)
    out = np.empty((q_len, hq, d))
    for h in range(hq):
        g = h // group
        out[:, h, :] = attend_rows(q_seq[:, h, :], k_seq[:, g, :], v_seq[:, g, :], pos, scale)
    return out


def attention_ragged(q_list: Sequence[np.ndarray], k_list: Sequence[np.ndarray],
                     v_list: Sequence[np.ndarray], scale: float | None = None) -> np.ndarray:
    """Ragged batch: per-sequence Q (new rows) and contiguous K/V (all keys).

    Returns the rows of all sequences packed in sequence order,
    ``[sum q_len][Hq][d]``.  Covers prefill (q_len == kv_len), decode
    (q_len == 1) and the mixed chunked-prefill + decode step.
    """
    outs = [attention_seq(q, k, v, scale) for q, k, v in zip(q_list, k_list, v_list)]
    if not outs:
        return np.zeros((0, 0, 0))
    return np.concatenate(outs, axis=0)


def prefill_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                   scale: float | None = None) -> np.ndarray:
    """Causal prefill over prompts packed by ``cu_seqlens`` (q/k/v ``[T][H][d]``).

    Each prompt attends only its own tokens.
    """
    cu = [int(c) for c in cu_seqlens]
    outs = []
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        outs.append(attention_seq(q[a:b], k[a:b], v[a:b], scale))
    if not outs:
        return np.zeros((0,) + tuple(q.shape[1:]))
    return np.concatenate(outs, axis=0)

