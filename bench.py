"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one continuous-batching forward of one attention layer over one
seeded synthetic batch, inputs resident in HBM: the slot-mapped append of the
step's new K/V, then attention.  The headline workload is the decode-only
batch (64 sequences, kv_len ~ U{128..2048}, 32/32 heads, d=128, bf16): a step
is kv_append of 64 tokens + paged decode (split partials + merge), and the
value is the step's algorithmic HBM bytes over its time (GB/s).  The ragged
4096-token prefill (TFLOP/s) and one 8192-token prompt, the mixed chunked-prefill + decode step, the
speculative-verify rows, the block copy, the append fused with the rotary
embedding, the headline batch in fp16 and over an fp8 KV cache, and the
long-context GQA decode are reported alongside under "secondary".

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --profile decode|prefill|prefill8k|mixed|long|copy|decode_fp8|rope|kvcopy|append --steps K
                                                                      (for rocprofv3)

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
METRIC = "paged decode HBM GB/s (% peak); varlen prefill TFLOP/s (% MFMA peak)"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_attention_append_amd", "csrc")
# The sources each counter-pass entry depends on: the file of its kernels, the
# shared internal header and the entry points that plan its launches.
APPEND_SOURCES = ("pka_append.hip", "pka_internal.h", "pka_api.hip")
ATTN_SOURCES = ("pka_attn_mfma.hip", "pka_internal.h", "pka_api.hip")
APPEND_KEYS = ("append_rope", "kv_copy_blocks", "kv_append_prefill_4096")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(key: str = "") -> str:
    """Hash of the sources the kernels of counter-pass entry ``key`` are built
    from (the append / copy kernels, or the attention kernels)."""
    h = hashlib.sha256()
    for name in (APPEND_SOURCES if key in APPEND_KEYS else ATTN_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# Algorithmic work (bytes that must cross HBM once; flops of unmasked pairs)
# ----------------------------------------------------------------------------
def decode_bytes(step, kv_fp8: bool = False) -> int:
    """K/V of every key once (1 byte per element for an fp8 cache, plus its
    per-head scales), q and out once, the block-table entries and kv_lens."""
    es = 4 if step.dtype == "f32" else 2
    kes = 1 if kv_fp8 else es
    kv = int(step.kv_lens.sum())
    d, hkv, hq, B = step.head_dim, step.num_kv_heads, step.num_q_heads, step.num_seqs
    blocks = int(((step.kv_lens + 15) // 16).sum())
    return kv * hkv * d * 2 * kes + 2 * B * hq * d * es + blocks * 4 + B * 4 + (2 * hkv * 4 if kv_fp8 else 0)


def append_bytes(step, kv_fp8: bool = False) -> int:
    es = 4 if step.dtype == "f32" else 2
    kes = 1 if kv_fp8 else es
    T = step.total_q
    return T * step.num_kv_heads * step.head_dim * 2 * (es + kes) + T * 4


def prefill_work(step):
    es = 2
    T, hq, hkv, d = step.total_q, step.num_q_heads, step.num_kv_heads, step.head_dim
    L = step.kv_lens.astype(np.int64)
    flops = int((4 * d * hq * (L * (L + 1) // 2)).sum())
    byts = T * hq * d * es * 2 + T * hkv * d * es * 2
    return flops, byts


def mixed_work(step, kv_fp8: bool = False):
    es = 2
    kes = 1 if kv_fp8 else es
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    byts = 0
    flops = 0
    for s in range(step.num_seqs):
        kv, ql = int(step.kv_lens[s]), int(step.q_lens[s])
        if ql == 0:
            continue
        byts += kv * hkv * d * 2 * kes + 2 * ql * hq * d * es + ((kv + 15) // 16) * 4
        c = kv - ql
        flops += 4 * d * hq * (ql * c + ql * (ql + 1) // 2)   # row i sees c + i + 1 keys
    return flops, byts


def bench_rope(steps: int, warmup: int) -> dict:
    """Append fused with the rotary embedding on the ragged 4096-token prefill
    batch (32/32 heads, d = 128, bf16): K rotated into the pool, V copied, q
    rotated in place, against the plain append of the same tokens.  Bytes =
    K and V read + written + q read + written + slots + positions."""
    import torch
    rope, plain_append, byts, T, dev = rope_setup()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    us = timed(rope)
    plain = timed(plain_append)
    del dev
    return {"tokens": T, "rope_append_us": round(us, 3), "gbs": round(byts / us / 1e3, 1),
            "frac_hbm_peak": round(byts / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": byts,
            "plain_append_us": round(plain, 3), "style": "half", "base": 10000.0,
            "traffic": traffic_for("append_rope")}


def rope_setup():
    """The RoPE append of the ragged 4096-token prefill batch: (rope call,
    plain append call, algorithmic bytes, tokens, device state)."""
    import paged_kv_attention_append_amd as pka
    from paged_kv_attention_append_amd import workloads as W
    st = W.prefill_ragged(3)
    dev = Dev(st)
    s = dev.sets[0]
    pos = dev.up(np.concatenate([np.arange(int(l)) for l in st.q_lens]).astype(np.int32))
    T, hq, hkv, d = st.total_q, st.num_q_heads, st.num_kv_heads, st.head_dim
    byts = T * hkv * d * 2 * 4 + T * hq * d * 2 * 2 + 8 * T
    return (lambda: pka.kv_append_rope(dev.cache, s["k"], s["v"], dev.slots, pos, q=s["q"]),
            lambda: pka.kv_append(dev.cache, s["k"], s["v"], dev.slots), byts, T, dev)


def bench_copy(steps: int, warmup: int) -> dict:
    """pka_kv_copy_blocks: 2048 random distinct block pairs inside one device
    pool (copy-on-write), and 1024 blocks out to / back from a pinned host
    pool (swap).  Bytes = blocks x (K + V) x Hkv x 16 x d x 2; a device copy
    moves them twice (read + write), a swap once across the host link."""
    import torch
    import paged_kv_attention_append_amd as pka
    res = {}
    for name, src, dst, pairs, moved in copy_cases():
        for _ in range(max(3, warmup // 4)):
            pka.kv_copy_blocks(src, dst, pairs)
        torch.cuda.synchronize()
        n = max(10, steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            pka.kv_copy_blocks(src, dst, pairs)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        res[name] = {"blocks": int(pairs.shape[0]), "us": round(us, 2), "bytes": moved,
                     "gbs": round(moved / us / 1e3, 1)}
    res["device_copy"]["frac_hbm_peak"] = round(res["device_copy"]["gbs"] / HBM_PEAK_GBS, 4)
    res["device_copy"]["traffic"] = traffic_for("kv_copy_blocks")
    return res


def copy_cases():
    """(name, src cache, dst cache, pairs, bytes moved) of the block-copy bench:
    GQA 8 kv heads, d = 128, bf16 (64 KiB per block with K and V)."""
    import torch
    import paged_kv_attention_append_amd as pka
    hkv, d, nb = 8, 128, 8192
    blk = 2 * hkv * 16 * d * 2
    rng = np.random.default_rng(7)
    dev = pka.KVCache.allocate(nb, hkv, d, torch.bfloat16, fill=1.0)
    host = pka.KVCache.allocate(1024, hkv, d, torch.bfloat16, fill=0.0, pinned_host=True)
    perm = rng.permutation(nb)
    cow = torch.from_numpy(np.stack([perm[:2048], perm[2048:4096]], 1).astype(np.int32)).cuda()
    out_pairs = torch.from_numpy(np.stack([perm[:1024], np.arange(1024)], 1).astype(np.int32)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(1024), perm[4096:5120]], 1).astype(np.int32)).cuda()
    return [("device_copy", dev, dev, cow, 2 * 2048 * blk),
            ("swap_out_to_pinned_host", dev, host, out_pairs, 1024 * blk),
            ("swap_in_from_pinned_host", host, dev, in_pairs, 1024 * blk)]


# ----------------------------------------------------------------------------
# Device setup
# ----------------------------------------------------------------------------
class Dev:
    def __init__(self, step, copies: int = 1, kv_fp8: bool = False, host_lens: bool = True):
        import torch
        import paged_kv_attention_append_amd as pka
        self.torch, self.pka, self.step = torch, pka, step
        dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(step.dtype, torch.float32)
        self.dt = dt
        up = lambda a, t=None: (torch.from_numpy(np.ascontiguousarray(a)).to(t) if t is not None
                                else torch.from_numpy(np.ascontiguousarray(a))).cuda()
        self.up = up
        if kv_fp8:  # E4M3 pools with seeded per-kv-head scales; q, new K/V and outputs stay in dt
            from paged_kv_attention_append_amd.workloads import fp8_scales
            ks = up(fp8_scales(11, step.num_kv_heads, step.sigma))
            vs = up(fp8_scales(12, step.num_kv_heads, step.sigma))
            self.cache = pka.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, torch.uint8,
                                              fill=0, act_dtype=dt, k_scale=ks, v_scale=vs)
        else:
            self.cache = pka.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, dt, fill=0.0)
        self.bt = up(step.block_tables.astype(np.int32))
        self.kvl = up(step.kv_lens.astype(np.int32))
        self.kvl_host = torch.from_numpy(step.kv_lens.astype(np.int32))
        self.hint = self.kvl_host if host_lens else None   # decode/verify scheduling hint
        self.cu = up(step.cu_q_lens.astype(np.int32))
        self.cu_host = torch.from_numpy(step.cu_q_lens.astype(np.int32))
        kc, vc = step.cached_kv()
        if kc.shape[0]:
            pka.kv_append(self.cache, up(kc, dt), up(vc, dt), up(step.cached_slot_mapping().astype(np.int32)))
        kn, vn = step.new_kv()
        self.sets = []
        for _ in range(copies):   # distinct buffer sets, cycled to defeat the 256 MB last-level cache
            self.sets.append(dict(q=up(step.packed_q(), dt), k=up(kn, dt), v=up(vn, dt),
                                  out=torch.empty((step.total_q, step.num_q_heads, step.head_dim), dtype=dt,
                                                  device="cuda")))
        self.slots = up(step.new_slot_mapping().astype(np.int32))
        self.ws = None
        torch.cuda.synchronize()

    def append(self, i=0):
        s = self.sets[i % len(self.sets)]
        self.pka.kv_append(self.cache, s["k"], s["v"], self.slots)

    def decode(self, i=0):
        st = self.step
        s = self.sets[i % len(self.sets)]
        q = s["q"].view(st.num_seqs, st.num_q_heads, st.head_dim)
        if self.ws is None:
            n = self.pka.decode_workspace_size(st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim,
                                               st.max_kv_len, 0, self.cache.dtype_code)
            self.ws = self.torch.empty(max(n, 256), dtype=self.torch.uint8, device="cuda")
        self.pka.attn_decode_paged(q, self.cache, self.bt, self.kvl, st.max_kv_len, workspace=self.ws,
                                   out=s["out"].view_as(q), kv_lens_host=self.hint)

    def prefill(self, i=0):
        s = self.sets[i % len(self.sets)]
        self.pka.attn_prefill_varlen(s["q"], s["k"], s["v"], self.cu, self.cu_host, out=s["out"])

    def mixed(self, i=0):
        st = self.step
        s = self.sets[i % len(self.sets)]
        if self.ws is None:
            dec = st.q_lens == 1
            mx = int(st.kv_lens[dec].max()) if dec.any() else 1
            n = self.pka.mixed_workspace_size(st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, mx)
            self.ws = self.torch.empty(max(n, 256), dtype=self.torch.uint8, device="cuda")
        self.pka.attn_mixed_step(s["q"], self.cache, self.cu, self.cu_host, self.kvl, self.kvl_host, self.bt,
                                 workspace=self.ws, out=s["out"])

    def verify(self, i=0):
        """Uniform q_len rows per sequence through attn_verify_paged."""
        st = self.step
        s = self.sets[i % len(self.sets)]
        nq = int(st.q_lens[0])
        q = s["q"].view(st.num_seqs, nq, st.num_q_heads, st.head_dim)
        if getattr(self, "vws", None) is None:
            n = self.pka.verify_workspace_size(st.num_seqs, nq, st.num_q_heads, st.num_kv_heads, st.head_dim,
                                               st.max_kv_len)
            self.vws = self.torch.empty(max(n, 256), dtype=self.torch.uint8, device="cuda")
        self.pka.attn_verify_paged(q, self.cache, self.bt, self.kvl, st.max_kv_len, workspace=self.vws,
                                   out=s["out"].view_as(q), kv_lens_host=self.hint)


def time_calls(torch, fn, n, warmup):
    """Mean duration (ms) of `n` back-to-back calls of fn on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def graph_of(torch, fn):
    """fn's launches captured into a HIP graph (after one warm call on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_step(dev, attn, steps, warmup):
    """Times `steps` steps (append + attn), bracketed by device synchronisation.

    Pass 1: one event pair around the whole loop (step time).  Pass 2: events
    around each call, on the same (current) stream the library launches on,
    for per-call durations of the append and of the attention call."""
    torch = dev.torch
    for i in range(warmup):
        dev.append(i)
        attn(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        dev.append(i)
        attn(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        dev.append(i)
        ev[i][1].record()
        attn(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    app = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    att = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    return step_ms, app, att, wall


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ----------------------------------------------------------------------------
def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(decode_step, prefill_step, decode_budget_s=12.0, prefill_budget_s=10.0):
    """The fp64 oracle as it stands, timed on the host's cores with the BLAS
    thread pool set to the affinity core count: all decode rows of the
    headline batch (GB/s on the same algorithmic bytes as the GPU line), and
    the ragged 4096-token prefill (TFLOP/s on the same flop count)."""
    from oracle import attention as A
    cores = host_cores()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        limiter, blas = None, None

    def timed(fn, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                return reps, time.perf_counter() - t0

    try:
        reps, el = timed(lambda: A.attention_ragged(decode_step.q, decode_step.k_ctx, decode_step.v_ctx),
                         decode_budget_s)
        preps, pel = timed(lambda: A.attention_ragged(prefill_step.q, prefill_step.k_ctx, prefill_step.v_ctx),
                           prefill_budget_s)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    gbs = decode_bytes(decode_step) * reps / el / 1e9
    fl, _ = prefill_work(prefill_step)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": f"fp64 NumPy oracle over all {decode_step.num_seqs} decode rows of the headline batch "
                      f"(attention only), {reps} passes in {el:.1f} s; cores = the process's CPU affinity set, "
                      f"BLAS threads limited to it",
            "prefill": {"value": round(fl * preps / pel / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
                        "blas_threads": blas, "kind": "oracle",
                        "sample": f"fp64 NumPy oracle over the ragged 4096-token prefill batch "
                                  f"({prefill_step.num_seqs} prompts, 32/32 heads), {preps} passes in {pel:.1f} s, "
                                  f"on the GPU line's flop count (unmasked pairs)"}}


def traffic_for(kernel_key: str, launches_per_call: int = 1):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(kernel_key)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return ent.get("bytes_per_call")


def run_decode(step, steps, warmup, key, kv_fp8=False, host_lens=True):
    dev = Dev(step, kv_fp8=kv_fp8, host_lens=host_lens)
    step_ms, app_ms, att_ms, wall = time_step(dev, dev.decode, steps, warmup)
    db, ab = decode_bytes(step, kv_fp8), append_bytes(step, kv_fp8)
    return dev, {
        "workload": step.name, "ms_per_step": step_ms, "append_ms": app_ms, "attn_ms": att_ms,
        "step_gbs": (db + ab) / (step_ms * 1e-3) / 1e9,
        "attn_bytes": db, "append_bytes": ab,
        "attn_gbs": db / (att_ms * 1e-3) / 1e9, "wall_s": wall,
        "traffic": traffic_for(key),
    }


def summarize_traffic(pmc_dir: str):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (directories named
    <workload>_fetch, <workload>_write, copy_fetch, copy_write under pmc_dir)
    into profiles/hbm_traffic.json: HBM bytes per attention call, each counter
    scaled by what it reads for a 1 GiB device copy (bytes moved / counter)."""
    import csv
    import glob

    def per_kernel(name, counter):
        out = {}
        for f in glob.glob(os.path.join(pmc_dir, name, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                out.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
        return {k: sum(v) / len(v) for k, v in out.items()}

    copy_f, copy_w = per_kernel("copy_fetch", "FETCH_SIZE"), per_kernel("copy_write", "WRITE_SIZE")
    ck = [k for k in copy_f if "copy" in k.lower()][0]
    f_scale, w_scale = (1 << 30) / copy_f[ck], (1 << 30) / copy_w[ck]
    old = {}
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if os.path.exists(path):  # entries of workloads without a run here are kept as they were
        with open(path) as f:
            old = json.load(f)
    result = {k: v for k, v in old.items() if isinstance(v, dict) and "bytes_per_call" in v}
    result.update({"fetch_scale": f_scale, "write_scale": w_scale,
                   "calibration": "1 GiB device-to-device copy: bytes moved / counter value"})
    for wl, key, kernels in [("decode", "decode_mha", ["decode_kernel", "decode_reduce_kernel"]),
                             ("prefill", "prefill_ragged", ["prefill16_kernel"]),
                             ("prefill8k", "prefill_1x8192", ["prefill16_kernel"]),
                             ("mixed", "mixed_gqa", ["mixed_kernel", "decode_reduce_kernel"]),
                             ("long", "long_decode", ["decode_kernel", "decode_reduce_kernel"]),
                             ("decode_fp8", "decode_mha_fp8", ["decode_kernel", "decode_reduce_kernel"]),
                             ("rope", "append_rope", ["append_rope_kernel"]),
                             ("append", "kv_append_prefill_4096", ["append_kernel"]),
                             ("kvcopy", "kv_copy_blocks", ["copy_kernel"])]:
        if not glob.glob(os.path.join(pmc_dir, f"{wl}_fetch", "*counter_collection.csv")):
            continue
        fe, wr = per_kernel(f"{wl}_fetch", "FETCH_SIZE"), per_kernel(f"{wl}_write", "WRITE_SIZE")
        tot, parts = 0.0, {}
        for kname in kernels:
            kf = [k for k in fe if k.endswith(kname) or (kname + "<") in k]
            kw = [k for k in wr if k.endswith(kname) or (kname + "<") in k]
            if not kf or not kw:
                continue
            b = fe[kf[0]] * f_scale + wr[kw[0]] * w_scale
            parts[kname] = {"fetch_bytes": fe[kf[0]] * f_scale, "write_bytes": wr[kw[0]] * w_scale}
            tot += b
        result[key] = {"source_hash": kernel_source_hash(key), "bytes_per_call": tot, "kernels": parts}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "hbm_traffic.json"), "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill", "prefill8k", "mixed", "long", "copy", "decode_fp8",
                                          "rope", "kvcopy", "append"])
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR",
                    help="write profiles/hbm_traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE runs")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the attention hot path has no "
                                   "cross-GPU step; run with --gpus 1"}))
        sys.exit(2)

    import torch
    import paged_kv_attention_append_amd as pka
    from paged_kv_attention_append_amd import workloads as W
    pka.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    if args.profile:
        if args.profile == "copy":
            n = 1 << 30
            a = torch.empty(n, dtype=torch.uint8, device="cuda")
            b = torch.empty_like(a)
            for _ in range(args.steps):
                b.copy_(a)
            torch.cuda.synchronize()
            print(json.dumps({"profile": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n}))
            return
        if args.profile in ("rope", "kvcopy", "append"):
            if args.profile == "rope":
                fn = rope_setup()[0]
            elif args.profile == "append":
                # The 4096-token append of the ragged prefill batch over 4
                # rotating input sets, as the benchmark times it (cold).
                adev = Dev(W.prefill_ragged(3), copies=4)
                calls = iter(range(1 << 30))
                fn = lambda: adev.append(next(calls))
            else:
                _, src, dst, pairs, _ = copy_cases()[0]
                fn = lambda: pka.kv_copy_blocks(src, dst, pairs)
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            print(json.dumps({"profile": args.profile, "steps": args.steps}))
            return
        mk = {"decode": W.decode_mha_7b, "prefill": W.prefill_ragged, "mixed": W.mixed_gqa,
              "long": W.long_decode_gqa, "decode_fp8": W.decode_mha_7b,
              "prefill8k": lambda: W.make_step("prefill_1x8192", W.BF16, 32, 32, 128, [8192], [8192], 10)}[args.profile]
        step = mk()
        dev = Dev(step, kv_fp8=args.profile == "decode_fp8")
        attn = {"decode": dev.decode, "prefill": dev.prefill, "mixed": dev.mixed, "long": dev.decode,
                "decode_fp8": dev.decode, "prefill8k": dev.prefill}[args.profile]
        for i in range(args.steps):
            dev.append(i)
            attn(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "steps": args.steps}))
        return

    # ---- headline: decode-only continuous batch --------------------------
    log("headline: decode MHA 64 x U{128..2048}, 32/32 heads, d=128, bf16")
    step = W.decode_mha_7b(2)
    _, head = run_decode(step, args.steps, args.warmup, "decode_mha")
    achieved = head["attn_gbs"]
    result = {
        "metric": METRIC,
        "value": round(head["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_mha_b64_ctx128-2048", "batch": 64, "kv_len": "U{128..2048}",
                   "q_heads": 32, "kv_heads": 32, "head_dim": 128, "block_size": 16, "seed": 2,
                   "step": "kv_append(64 tokens) + attn_decode_paged (host lengths given: longest sequence first, "
                           "automatic split plan)"},
        "roofline": {"bound": "hbm", "kernel": "attn_decode_paged call (decode kernel; merge kernel only when keys are split)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": head["traffic"],
                     "algorithmic_bytes_per_launch": head["attn_bytes"],
                     "avg_launch_us": round(head["attn_ms"] * 1e3, 3)},
        "append": {"us": round(head["append_ms"] * 1e3, 3), "bytes": head["append_bytes"]},
    }
    log(f"decode step {head['ms_per_step']*1e3:.1f} us, attn {head['attn_ms']*1e3:.1f} us "
        f"({achieved:.0f} GB/s), append {head['append_ms']*1e3:.1f} us")

    # ---- secondary workloads -------------------------------------------------
    if not args.no_secondary:
        sec = {}
        log("secondary: tiny fp32 batch (launch-bound decode step: append + decode), eager and as a HIP graph")
        _, dec = W.tiny_fp32(1)
        dev = Dev(dec)

        def tiny_step():
            dev.append(0)
            dev.decode(0)
        eager_ms = time_calls(dev.torch, tiny_step, args.steps, args.warmup)
        g = graph_of(dev.torch, tiny_step)
        graph_ms = time_calls(dev.torch, g.replay, args.steps, args.warmup)
        # Device time of one replay (events around a single replay, the host
        # idle in between): what the step costs once its launches are queued.
        torch_ = dev.torch
        durs = []
        for _ in range(50):
            e0, e1 = torch_.cuda.Event(enable_timing=True), torch_.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch_.cuda.synchronize()
            durs.append(e0.elapsed_time(e1))
        sec["tiny_fp32_decode_step"] = {"eager_us": round(eager_ms * 1e3, 3), "graph_replay_us": round(graph_ms * 1e3, 3),
                                        "graph_device_us": round(float(np.median(durs)) * 1e3, 3),
                                        "sequences": int(dec.num_seqs), "kv_lens": [int(x) for x in dec.kv_lens]}
        del g, dev
        log("secondary: ragged prefill 4096 tokens, 32/32 heads (cold: 4 rotating buffer sets)")
        st = W.prefill_ragged(3)
        dev = Dev(st, copies=4)
        sms, ams, pms, _ = time_step(dev, dev.prefill, args.steps, args.warmup)
        # Warm: the same buffer set every call (inputs resident in the 256 MB MALL).
        wms = time_calls(dev.torch, lambda: dev.prefill(0), args.steps, args.warmup)
        fl, by = prefill_work(st)
        # The attainable roofline: the larger of the matrix-core and the HBM time.
        roof_ms = max(fl / (MFMA_BF16_PEAK_TFLOPS * 1e12), by / (HBM_PEAK_GBS * 1e9)) * 1e3
        sec["prefill_ragged_4096"] = {
            "ms_per_step": round(sms, 5), "prefill_us": round(pms * 1e3, 3), "append_us": round(ams * 1e3, 3),
            "tflops": round(fl / (pms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(fl / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "frac_attainable_roofline": round(roof_ms / pms, 4),
            "prefill_us_warm": round(wms * 1e3, 3), "tflops_warm": round(fl / (wms * 1e-3) / 1e12, 2),
            "prefill_gbs": round(by / (pms * 1e-3) / 1e9, 1),
            "append_gbs": round(append_bytes(st) / (ams * 1e-3) / 1e9, 1),
            "append_frac_hbm_peak": round(append_bytes(st) / (ams * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "append_bytes": append_bytes(st), "append_traffic": traffic_for("kv_append_prefill_4096"),
            "flops": fl, "bytes": by, "traffic": traffic_for("prefill_ragged")}
        del dev
        log("secondary: one 8192-token prompt, 32/32 heads (the prefill kernel with ample work per head)")
        st = W.make_step("prefill_1x8192", W.BF16, 32, 32, 128, [8192], [8192], 10)
        dev = Dev(st)
        n = max(10, args.steps // 10)
        sms, ams, pms, _ = time_step(dev, dev.prefill, n, max(3, args.warmup // 4))
        fl, by = prefill_work(st)
        sec["prefill_1x8192"] = {
            "prefill_us": round(pms * 1e3, 3), "tflops": round(fl / (pms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(fl / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl, "bytes": by,
            "steps": n, "traffic": traffic_for("prefill_1x8192")}
        del dev
        log("secondary: mixed GQA 32/8, 128 decodes + 2 x 1024-token chunks")
        st = W.mixed_gqa(4)
        dev = Dev(st)
        sms, ams, mms, _ = time_step(dev, dev.mixed, args.steps, args.warmup)
        fl, by = mixed_work(st)
        sec["mixed_gqa"] = {
            "ms_per_step": round(sms, 5), "mixed_us": round(mms * 1e3, 3), "append_us": round(ams * 1e3, 3),
            "gbs": round(by / (mms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(by / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / (mms * 1e-3) / 1e12, 2), "flops": fl, "bytes": by,
            "traffic": traffic_for("mixed_gqa")}
        del dev
        log("secondary: the mixed step over an fp8 (E4M3) KV cache, bf16 activations")
        st = W.mixed_gqa(4)
        dev = Dev(st, kv_fp8=True)
        sms, ams, mms, _ = time_step(dev, dev.mixed, max(20, args.steps // 4), max(5, args.warmup // 4))
        fl, by = mixed_work(st, kv_fp8=True)
        sec["mixed_gqa_fp8kv"] = {
            "ms_per_step": round(sms, 5), "mixed_us": round(mms * 1e3, 3), "append_us": round(ams * 1e3, 3),
            "gbs": round(by / (mms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(by / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / (mms * 1e-3) / 1e12, 2), "flops": fl, "bytes": by}
        del dev
        log("secondary: speculative verify GQA 32/8, 64 sequences x 5 rows (mixed entry point)")
        st = W.spec_verify_gqa(6)
        dev = Dev(st)
        sms, ams, mms, _ = time_step(dev, dev.mixed, args.steps, args.warmup)
        fl, by = mixed_work(st)
        sec["spec_verify_gqa_mixed_entry"] = {
            "ms_per_step": round(sms, 5), "verify_us": round(mms * 1e3, 3), "append_us": round(ams * 1e3, 3),
            "gbs": round(by / (mms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(by / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / (mms * 1e-3) / 1e12, 2), "flops": fl, "bytes": by}
        sms, ams, vms, _ = time_step(dev, dev.verify, args.steps, args.warmup)
        sec["spec_verify_gqa"] = {
            "ms_per_step": round(sms, 5), "verify_us": round(vms * 1e3, 3), "append_us": round(ams * 1e3, 3),
            "gbs": round(by / (vms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(by / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "entry_point": "attn_verify_paged", "bytes": by}
        del dev
        log("secondary: KV block copy (GQA 8 kv heads, d=128, bf16; 64 KiB per block with K and V)")
        sec["kv_copy_blocks"] = bench_copy(args.steps, args.warmup)
        log("secondary: append fused with RoPE (K and q rotated), ragged prefill 4096 tokens")
        sec["append_rope_prefill_4096"] = bench_rope(args.steps, args.warmup)
        log("secondary: the headline decode batch without host lengths (index order, unsorted split plan)")
        _, r = run_decode(W.decode_mha_7b(2), max(20, args.steps // 4), max(5, args.warmup // 4),
                          "decode_mha_no_hint", host_lens=False)
        sec["decode_mha_no_host_lengths"] = {"attn_us": round(r["attn_ms"] * 1e3, 3), "gbs": round(r["attn_gbs"], 1),
                                             "frac_hbm_peak": round(r["attn_gbs"] / HBM_PEAK_GBS, 4),
                                             "bytes": r["attn_bytes"]}
        log("secondary: the headline decode batch in fp16")
        _, r = run_decode(W.decode_mha_7b(2, dtype=W.F16), max(20, args.steps // 4), max(5, args.warmup // 4),
                          "decode_mha_f16")
        sec["decode_mha_f16"] = {"attn_us": round(r["attn_ms"] * 1e3, 3), "gbs": round(r["attn_gbs"], 1),
                                 "frac_hbm_peak": round(r["attn_gbs"] / HBM_PEAK_GBS, 4), "bytes": r["attn_bytes"]}
        log("secondary: the headline decode batch over an fp8 (E4M3) KV cache, bf16 activations")
        _, r = run_decode(W.decode_mha_7b(2), max(20, args.steps // 4), max(5, args.warmup // 4),
                          "decode_mha_fp8", kv_fp8=True)
        sec["decode_mha_fp8kv"] = {
            "ms_per_step": round(r["ms_per_step"], 5), "attn_us": round(r["attn_ms"] * 1e3, 3),
            "append_us": round(r["append_ms"] * 1e3, 3), "gbs": round(r["attn_gbs"], 1),
            "frac_hbm_peak": round(r["attn_gbs"] / HBM_PEAK_GBS, 4), "bytes": r["attn_bytes"],
            "step_gbs": round(r["step_gbs"], 1), "append_bytes": r["append_bytes"],
            "traffic": r["traffic"]}
        log("secondary: long decode GQA 64/8, 16 x 32768")
        st = W.long_decode_gqa(5)
        _, r = run_decode(st, max(20, args.steps // 4), max(5, args.warmup // 4), "long_decode")
        sec["long_decode_gqa"] = {
            "ms_per_step": round(r["ms_per_step"], 5), "attn_us": round(r["attn_ms"] * 1e3, 3),
            "gbs": round(r["attn_gbs"], 1), "frac_hbm_peak": round(r["attn_gbs"] / HBM_PEAK_GBS, 4),
            "bytes": r["attn_bytes"], "traffic": r["traffic"]}
        del st
        result["secondary"] = sec

    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on the headline decode batch and the ragged 4096-token prefill")
        result["cpu_baseline"] = cpu_baseline(W.decode_mha_7b(2), W.prefill_ragged(3))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
