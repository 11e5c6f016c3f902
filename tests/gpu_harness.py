"""Helpers for the GPU parity tests: move a generated step onto the device,
run it through the C ABI (via the ctypes binding), and compare with the
fp64 oracle.  Tolerances: bf16 inputs with fp32 accumulation, max |err|
<= 1e-2 and mean |err| <= 1e-3 over all output elements; fp32, max <= 1e-5.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_attention_append_amd as pka
from paged_kv_attention_append_amd import workloads as W

BF16_MAX, BF16_MEAN, F32_MAX = 1e-2, 1e-3, 1e-5
# fp16 (derived, not given): half an fp16 ulp is 9.8e-4 for |o| in [2, 4); the
# weights rounded to fp16 (relative 2^-11, renormalised by their own sum) add
# at most about as much again.  Mean: ten times below the max, as for bf16.
F16_MAX, F16_MEAN = 2.5e-3, 2.5e-4


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(step):
    return {W.BF16: torch.bfloat16, W.F16: torch.float16}.get(step.dtype, torch.float32)


def dev(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def nan_value(step):
    return float("nan")


FP8_POISON = 0x7F  # an E4M3 NaN code: fills the free slots of fp8 pools


class DeviceStep:
    """A generated step on the GPU: pools, block tables, lengths, Q and K/V.

    With ``fp8_scales = (k_scale, v_scale)`` (numpy fp32 [Hkv]) the pools are
    fp8 E4M3 codes and the step's dtype is the activation dtype."""

    def __init__(self, step: W.Step, fill=float("nan"), block_tables=None, fp8_scales=None):
        self.step = step
        dt = torch_dtype(step)
        self.dt = dt
        if fp8_scales is None:
            self.cache = pka.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, dt, fill=fill)
        else:
            ks, vs = (dev(np.asarray(x, np.float32)) for x in fp8_scales)
            self.cache = pka.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, torch.uint8,
                                              fill=FP8_POISON, act_dtype=dt, k_scale=ks, v_scale=vs)
        bt = step.block_tables if block_tables is None else block_tables
        self.block_tables = dev(bt.astype(np.int32))
        self.kv_lens = dev(step.kv_lens.astype(np.int32))
        self.kv_lens_host = step.kv_lens.astype(np.int32)
        self.cu_q = dev(step.cu_q_lens.astype(np.int32))
        self.cu_q_host = step.cu_q_lens.astype(np.int32)
        self.q = dev(step.packed_q(), dt)

    def append_cached(self, slots=None):
        s = self.step
        kc, vc = s.cached_kv()
        if kc.shape[0] == 0:
            return
        slots = s.cached_slot_mapping() if slots is None else slots
        pka.kv_append(self.cache, dev(kc, self.dt), dev(vc, self.dt), dev(slots.astype(np.int32)))

    def append_new(self, slots=None):
        s = self.step
        kn, vn = s.new_kv()
        if kn.shape[0] == 0:
            return
        slots = s.new_slot_mapping() if slots is None else slots
        pka.kv_append(self.cache, dev(kn, self.dt), dev(vn, self.dt), dev(slots.astype(np.int32)))

    def fill_cache(self):
        self.append_cached()
        self.append_new()
        torch.cuda.synchronize()

    def decode(self, num_splits=0, scale=0.0, host_lens=True):
        """Decode through the C ABI; with ``host_lens`` the host lengths go along
        as the scheduling hint (the benchmark's configuration)."""
        assert np.all(self.step.q_lens == 1)
        q = self.q.view(self.step.num_seqs, self.step.num_q_heads, self.step.head_dim)
        hint = self.kv_lens_host if host_lens is True else (host_lens if host_lens is not False else None)
        out = pka.attn_decode_paged(q, self.cache, self.block_tables, self.kv_lens, self.step.max_kv_len,
                                    scale=scale, num_splits=num_splits, kv_lens_host=hint)
        torch.cuda.synchronize()
        return out

    def mixed(self, scale=0.0):
        out = pka.attn_mixed_step(self.q, self.cache, self.cu_q, torch.from_numpy(self.cu_q_host),
                                  self.kv_lens, torch.from_numpy(self.kv_lens_host), self.block_tables,
                                  scale=scale)
        torch.cuda.synchronize()
        return out

    def prefill(self, scale=0.0):
        s = self.step
        assert np.all(s.q_lens == s.kv_lens)
        kn, vn = s.new_kv()
        out = pka.attn_prefill_varlen(self.q, dev(kn, self.dt), dev(vn, self.dt), self.cu_q,
                                      torch.from_numpy(self.cu_q_host), scale=scale)
        torch.cuda.synchronize()
        return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def compare(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    g = to_f64(gpu).reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"{what}: max|err| {mx:.3e} mean|err| {mean:.3e} over {err.size} elements")
    if dtype == W.BF16:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (what, mx, mean)
    elif dtype == W.F16:
        assert mx <= F16_MAX and mean <= F16_MEAN, (what, mx, mean)
    else:
        assert mx <= F32_MAX, (what, mx)
    return mx, mean


def pool_bits(cache: pka.KVCache):
    k = cache.k_pool.cpu()
    v = cache.v_pool.cpu()
    if k.dtype == torch.uint8:
        return k.numpy(), v.numpy()
    if k.dtype in (torch.bfloat16, torch.float16):
        return k.view(torch.int16).numpy().view(np.uint16), v.view(torch.int16).numpy().view(np.uint16)
    return k.view(torch.int32).numpy().view(np.uint32), v.view(torch.int32).numpy().view(np.uint32)


def value_bits(a: np.ndarray, dtype: str):
    if dtype == W.BF16:
        return W.bf16_bits(a)
    if dtype == W.F16:
        return W.f16_bits(a)
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def check_whole_pool_append(ds: DeviceStep, k0: np.ndarray, v0: np.ndarray, what: str = ""):
    """Both pools, every byte, after ``ds.fill_cache()``, against the oracle's
    append of the step's cached tokens and then its new tokens into the
    pre-append pool bits ``k0, v0``: the written slots hold the inputs' bits
    and every other slot keeps its poison."""
    from oracle import paged_layout as L

    s = ds.step
    k1, v1 = pool_bits(ds.cache)
    kc, vc = s.cached_kv()
    kn, vn = s.new_kv()
    ek, ev = L.append(k0, v0, value_bits(kc, s.dtype), value_bits(vc, s.dtype), s.cached_slot_mapping(),
                      s.num_kv_heads, s.head_dim)
    ek, ev = L.append(ek, ev, value_bits(kn, s.dtype), value_bits(vn, s.dtype), s.new_slot_mapping(),
                      s.num_kv_heads, s.head_dim)
    nk, nv = int(np.count_nonzero(k1 != ek)), int(np.count_nonzero(v1 != ev))
    say(f"{what}: whole-pool append, {k1.size} elements per pool, {nk} K and {nv} V mismatches")
    assert nk == 0 and nv == 0, (what, nk, nv)


def codes_of(x: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[T][Hkv][d] values -> E4M3 codes, head g with scales[g] (the oracle's
    quantizer)."""
    from oracle import fp8 as F8

    out = np.empty(x.shape, np.uint8)
    for g in range(x.shape[1]):
        out[:, g, :] = F8.quantize(x[:, g, :], float(scales[g]))
    return out
