"""bench.py on the CPU: the algorithmic bytes and flops the roofline divides
by, against hand-computed values, and the one-GPU contract of --gpus."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_attention_append_amd import workloads as W  # noqa: E402


def test_decode_bytes_by_hand():
    # kv_len 20 and 33, 4/2 heads, d = 64, bf16:
    # K and V: 53 keys x 2 heads x 64 x 2 (K, V) x 2 B = 27136; q and out: 2 x 2 seqs x 4 x 64 x 2 B = 2048;
    # block-table entries: ceil(20/16) + ceil(33/16) = 5 -> 20 B; kv_lens 8 B.
    st = W.random_step(1, W.BF16, 4, 2, 64, [20, 33], [1, 1])
    assert bench.decode_bytes(st) == 27136 + 2048 + 20 + 8
    # fp8 pools: one byte per K/V element, plus the two per-head fp32 scale arrays (2 x 2 x 4 B).
    assert bench.decode_bytes(st, kv_fp8=True) == 13568 + 2048 + 20 + 8 + 16


def test_append_bytes_by_hand():
    # 2 new tokens, 2 kv heads, d = 64, bf16: read and written K and V, 2 x 2 x 64 x 2 x (2 + 2) B, + 2 slots.
    st = W.random_step(1, W.BF16, 4, 2, 64, [20, 33], [1, 1])
    assert bench.append_bytes(st) == 2 * 2 * 64 * 2 * 4 + 8
    assert bench.append_bytes(st, kv_fp8=True) == 2 * 2 * 64 * 2 * 3 + 8


def test_prefill_work_by_hand():
    # prompts 3 and 5, 2/1 heads, d = 64: flops 4 d Hq (3*4/2 + 5*6/2) = 4*64*2*21;
    # bytes: q and out 8 x 2 x 64 x 2 B x 2, k and v 8 x 1 x 64 x 2 B x 2.
    st = W.random_step(1, W.BF16, 2, 1, 64, [3, 5], [3, 5])
    assert bench.prefill_work(st) == (10752, 4096 + 2048)


def test_mixed_work_by_hand():
    # a 3-row chunk on 7 cached keys (kv_len 10) and a decode row on 4 cached (kv_len 5), 2/1 heads, d = 64:
    # chunk: K/V 10 x 64 x 2 x 2 = 2560, q/out 2 x 3 x 2 x 64 x 2 = 1536, 1 table entry; flops 4*64*2*(3*7 + 6)
    # decode: K/V 5 x 256 = 1280, q/out 512, 1 table entry;                         flops 4*64*2*(1*4 + 1)
    st = W.random_step(1, W.BF16, 2, 1, 64, [10, 5], [3, 1])
    assert bench.mixed_work(st) == (512 * 27 + 512 * 5, 2560 + 1536 + 4 + 1280 + 512 + 4)


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in json.loads(res.stdout.strip().splitlines()[-1])["error"]
