"""CPU tests of the C ABI: the library loads, exports every function that
include/pka.h declares, and rejects bad arguments on the host (no GPU call
is reached by any case here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_attention_append_amd as pka

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pka.h")

lib_missing = not os.path.exists(pka.LIB_PATH)
pytestmark = pytest.mark.skipif(lib_missing, reason="libpka.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # aligned, never dereferenced: every case returns before a launch


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(pka_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert set(declared_functions()) == set(pka.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = pka.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = pka.load_library()
    assert lib.pka_version() == 4
    for code, text in pka.STATUS.items():
        assert lib.pka_status_string(code).decode() == text
    assert lib.pka_status_string(99).decode() == "unknown status"


def cache(num_blocks=8, block_size=16, hkv=2, d=128, dtype=pka.PKA_BF16, k=FAKE, v=FAKE, act=0, ks=None,
          vs=None):
    return pka.KVCacheDesc(k, v, num_blocks, block_size, hkv, d, dtype, act, ks, vs)


def append(c, k=FAKE, v=FAKE, slots=FAKE, n=4):
    lib = pka.load_library()
    return lib.pka_kv_append(ctypes.byref(c) if c is not None else None, k, v, slots, n, None)


def test_append_validation():
    assert append(None) == -1
    assert append(cache(block_size=32)) == -2
    assert append(cache(d=96)) == -2
    assert append(cache(dtype=7)) == -2
    assert append(cache(hkv=0)) == -1
    assert append(cache(num_blocks=0)) == -1
    assert append(cache(k=0)) == -1
    assert append(cache(v=FAKE + 4)) == -1           # misaligned pool
    assert append(cache(num_blocks=2 ** 28)) == -1   # slots would overflow int32
    assert append(cache(), n=-1) == -1
    assert append(cache(), n=0) == 0                 # no-op, nothing launched
    assert append(cache(), k=0) == -1
    assert append(cache(), slots=0) == -1
    assert append(cache(), v=FAKE + 2) == -1


def append_rope(c, k=FAKE, v=FAKE, slots=FAKE, pos=FAKE, n=4, q=None, qo=None, hq=0, base=10000.0, style=0):
    lib = pka.load_library()
    return lib.pka_kv_append_rope(ctypes.byref(c) if c is not None else None, k, v, slots, pos, n, q, qo, hq,
                                  base, style, None)


def test_append_rope_validation():
    assert append_rope(None) == -1
    assert append_rope(cache(d=96)) == -2
    assert append_rope(cache(block_size=8)) == -2
    assert append_rope(cache(), n=-1) == -1
    assert append_rope(cache(), n=0) == 0                       # nothing to do
    assert append_rope(cache(), pos=0) == -1                    # positions required
    assert append_rope(cache(), slots=0) == -1
    assert append_rope(cache(), k=FAKE + 2) == -1               # misaligned
    assert append_rope(cache(), base=0.0) == -1
    assert append_rope(cache(), base=-1.0) == -1
    assert append_rope(cache(), base=float("inf")) == -1
    assert append_rope(cache(), base=float("nan")) == -1
    assert append_rope(cache(), style=2) == -1
    assert append_rope(cache(), q=FAKE, qo=None, hq=4) == -1    # q without q_out
    assert append_rope(cache(), q=None, qo=FAKE, hq=4) == -1
    assert append_rope(cache(), q=FAKE, qo=FAKE, hq=0) == -1
    assert append_rope(cache(), q=FAKE, qo=FAKE + 8, hq=4) == -1
    assert append_rope(cache(), q=FAKE, qo=FAKE, hq=4, n=0) == 0
    assert append_rope(cache(dtype=pka.PKA_FP8_E4M3, act=pka.PKA_BF16, ks=FAKE), n=0) == -1  # no v_scale


def test_fp8_cache_validation():
    fp8 = dict(dtype=pka.PKA_FP8_E4M3, ks=FAKE, vs=FAKE)
    assert append(cache(act=pka.PKA_BF16, **fp8), n=0) == 0      # valid description, nothing to do
    assert append(cache(act=pka.PKA_F16, **fp8), n=0) == 0
    assert append(cache(act=0, **fp8)) == -2                     # activation dtype missing
    assert append(cache(act=pka.PKA_F32, **fp8)) == -2           # fp8 pools serve 16-bit activations only
    assert append(cache(act=pka.PKA_BF16, dtype=pka.PKA_FP8_E4M3, vs=FAKE)) == -1   # no k_scale
    assert append(cache(act=pka.PKA_BF16, dtype=pka.PKA_FP8_E4M3, ks=FAKE)) == -1   # no v_scale
    assert append(cache(act=pka.PKA_BF16, d=96, **fp8)) == -2
    assert append(cache(act=pka.PKA_F16), n=0) == -1             # act_dtype must match a 16/32-bit pool
    assert append(cache(act=pka.PKA_BF16), n=0) == 0
    assert append(cache(act=pka.PKA_BF16, **fp8), k=FAKE + 8) == -1   # new keys must be 16-byte aligned
    assert decode(cache(act=pka.PKA_BF16, **fp8), B=0) == 0
    assert decode(cache(act=pka.PKA_BF16, **fp8), hq=3) == -1
    lib = pka.load_library()
    a, b = cache(act=pka.PKA_BF16, **fp8), cache()
    assert lib.pka_kv_copy_blocks(ctypes.byref(a), ctypes.byref(b), FAKE, 1, None) == -1  # pool dtypes differ
    assert lib.pka_kv_copy_blocks(ctypes.byref(a), ctypes.byref(a), FAKE, 0, None) == 0
    # the partials are fp32 whatever the pool holds
    assert (pka.decode_workspace_size(4, 8, 2, 128, 4096, 0, pka.PKA_FP8_E4M3)
            == pka.decode_workspace_size(4, 8, 2, 128, 4096, 0, pka.PKA_BF16) > 0)


def prefill(cu_host, hq=4, hkv=2, d=128, dtype=pka.PKA_BF16, q=FAKE, cu=FAKE):
    lib = pka.load_library()
    arr = np.ascontiguousarray(cu_host, np.int32)
    return lib.pka_attn_prefill_varlen(q, FAKE, FAKE, FAKE, cu, arr.ctypes.data, len(arr) - 1, hq, hkv, d,
                                       dtype, 0.0, None)


def test_prefill_validation():
    assert prefill([1, 4]) == -1              # cu[0] != 0
    assert prefill([0, 5, 3]) == -1           # decreasing
    assert prefill([0, 4], hq=3, hkv=2) == -1
    assert prefill([0, 4], hq=0) == -1
    assert prefill([0, 4], d=80) == -2
    assert prefill([0, 4], dtype=5) == -2
    assert prefill([0, 4], q=0) == -1
    assert prefill([0, 4], q=FAKE + 8) == -1
    assert prefill([0, 4], cu=0) == -1
    assert prefill([0]) == 0                  # no sequences
    assert prefill([0, 0, 0]) == 0            # only empty prompts
    lib = pka.load_library()
    assert lib.pka_attn_prefill_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 2, 128, 1, 0.0, None) == -1


def decode(c, B=4, max_blocks=8, max_kv=100, hq=4, splits=0, ws=0, wsb=0, q=FAKE):
    lib = pka.load_library()
    return lib.pka_attn_decode_paged(q, FAKE, ctypes.byref(c), FAKE, max_blocks, FAKE, None, B, max_kv, hq, 0.0,
                                     splits, ws, wsb, None)


def test_decode_validation():
    assert decode(cache(), hq=3) == -1
    assert decode(cache(), max_kv=129) == -1            # exceeds max_blocks * 16
    assert decode(cache(), max_kv=0) == -1
    assert decode(cache(), max_blocks=0) == -1
    assert decode(cache(), splits=-1) == -1
    assert decode(cache(), B=-2) == -1
    assert decode(cache(), B=0) == 0
    assert decode(cache(), q=0) == -1
    assert decode(cache(d=64, block_size=8)) == -2
    # a forced split needs a workspace
    assert decode(cache(), max_kv=128, splits=4) == -3
    need = pka.decode_workspace_size(4, 4, 2, 128, 128, 4)
    assert need > 0
    assert decode(cache(), max_kv=128, splits=4, ws=FAKE, wsb=need - 1) == -3
    assert decode(cache(), max_kv=128, splits=4, ws=FAKE + 4, wsb=need) == -3


def decode_noalloc(c, B=4, max_blocks=8, max_kv=100, hq=4, splits=0, q=FAKE):
    lib = pka.load_library()
    return lib.pka_attn_decode_paged_noalloc(q, FAKE, ctypes.byref(c), FAKE, max_blocks, FAKE, None, B, max_kv, hq,
                                             0.0, splits, None)


def test_decode_noalloc_validation():
    """The no-allocation decode checks its arguments as the workspace decode
    does, and rejects plans whose partials exceed the fixed scratch, before
    any GPU call."""
    assert decode_noalloc(cache(), hq=3) == -1
    assert decode_noalloc(cache(), max_kv=129) == -1
    assert decode_noalloc(cache(), B=-2) == -1
    assert decode_noalloc(cache(), B=0) == 0
    assert decode_noalloc(cache(), q=0) == -1
    assert decode_noalloc(cache(d=64, block_size=8)) == -2
    # 512 sequences x 64 heads x 64 forced splits of 1024+ keys: 512*64*64*(128*4 + 8) B = 1.09 GB of partials
    assert pka.decode_workspace_size(512, 64, 8, 128, 1024, 64) > pka.NOALLOC_SCRATCH_BYTES
    assert decode_noalloc(cache(hkv=8), B=512, hq=64, max_blocks=64, max_kv=1024, splits=64) == pka.PKA_ERR_SCRATCH_LIMIT
    assert pka.load_library().pka_status_string(-6).decode() == pka.STATUS[-6]


def mixed(c, cu_host, kv_host, max_blocks=8, hq=4):
    lib = pka.load_library()
    cu = np.ascontiguousarray(cu_host, np.int32)
    kv = np.ascontiguousarray(kv_host, np.int32)
    return lib.pka_attn_mixed_step(FAKE, FAKE, ctypes.byref(c), FAKE, cu.ctypes.data, FAKE, kv.ctypes.data,
                                   FAKE, max_blocks, len(cu) - 1, hq, 0.0, 0, 0, None)


def test_mixed_validation():
    assert mixed(cache(), [0, 5, 6], [4, 10]) == -1      # kv_len < q_len
    assert mixed(cache(), [0, 1, 2], [129, 3]) == -1     # kv_len beyond the block table
    assert mixed(cache(), [0, 1, 2], [5, -1]) == -1
    assert mixed(cache(), [1, 2], [5]) == -1
    assert mixed(cache(), [0, 1, 3], [40, 40], hq=5) == -1
    assert mixed(cache(), [0, 0, 0], [7, 9]) == 0         # rows: none
    # decode rows with long keys need the split workspace
    assert mixed(cache(), [0, 1, 2], [128, 128]) == -3


def test_workspace_sizes():
    # fp32 and single-split plans need no workspace
    assert pka.decode_workspace_size(4, 8, 8, 128, 4096, 0, pka.PKA_F32) == 0
    assert pka.decode_workspace_size(4, 8, 8, 128, 4096, 1) == 0
    # forced 3 splits: [B][Hq][S][D] fp32 + [B][Hq][S] (m, l), each rounded up to 256 bytes
    B, hq, d, S = 5, 6, 64, 3
    n = B * hq * S
    r = lambda x: (x + 255) // 256 * 256
    assert pka.decode_workspace_size(B, hq, 2, d, 3 * 16, S) == r(n * d * 4) + r(n * 8)
    # the automatic plan is monotone in max_kv_len, so a workspace sized for a
    # larger bound is always large enough
    for B, hq, hkv in [(1, 8, 1), (16, 64, 8), (64, 32, 32), (130, 32, 8)]:
        sizes = [pka.decode_workspace_size(B, hq, hkv, 128, L, 0) for L in range(1, 40000, 97)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:]))
        msizes = [pka.mixed_workspace_size(B, hq, hkv, 128, L) for L in range(1, 40000, 97)]
        assert msizes == sizes


def copy(src, dst, pairs=FAKE, n=4):
    lib = pka.load_library()
    return lib.pka_kv_copy_blocks(ctypes.byref(src) if src is not None else None,
                                  ctypes.byref(dst) if dst is not None else None, pairs, n, None)


def test_copy_blocks_validation():
    assert copy(None, cache()) == -1
    assert copy(cache(), None) == -1
    assert copy(cache(block_size=8), cache()) == -2
    assert copy(cache(), cache(d=96)) == -2
    assert copy(cache(hkv=2), cache(hkv=4)) == -1      # mismatched caches
    assert copy(cache(d=64), cache(d=128)) == -1
    assert copy(cache(dtype=pka.PKA_F32), cache()) == -1
    assert copy(cache(), cache(), n=-1) == -1
    assert copy(cache(), cache(), pairs=None) == -1
    assert copy(cache(), cache(), pairs=None, n=0) == 0   # no-op
    assert copy(cache(num_blocks=3), cache(num_blocks=100), n=0) == 0  # pool sizes may differ


def verify(c, nq=5, max_kv=100, n=4, dtype_ok=True):
    lib = pka.load_library()
    return lib.pka_attn_verify_paged(FAKE, FAKE, ctypes.byref(c), FAKE, 8, FAKE, None, n, nq, max_kv, 8, 0.0, 0,
                                     FAKE, 1 << 30, None)


def test_verify_validation():
    assert verify(cache(), nq=0) == -1
    assert verify(cache(), nq=65) == -1
    assert verify(cache(), nq=5, max_kv=4) == -1          # fewer keys than rows
    assert verify(cache(), max_kv=129) == -1              # beyond max_blocks * 16
    assert verify(cache(dtype=pka.PKA_F32), nq=2) == -2   # 16-bit pools only
    assert verify(cache(), n=0) == 0


def test_verify_workspace_sizes():
    lib = pka.load_library()
    for args in [(64, 32, 32, 128, 2048, 0), (16, 64, 8, 128, 32768, 0), (3, 8, 2, 64, 500, 3)]:
        B, hq, hkv, d, kv, sp = args
        assert lib.pka_verify_workspace_size(B, 1, hq, hkv, d, kv, sp, pka.PKA_BF16) == \
            lib.pka_decode_workspace_size(B, hq, hkv, d, kv, sp, pka.PKA_BF16)
    # explicit splits: partials grow with the rows
    a = lib.pka_verify_workspace_size(8, 1, 8, 2, 128, 1000, 4, pka.PKA_BF16)
    b = lib.pka_verify_workspace_size(8, 5, 8, 2, 128, 1000, 4, pka.PKA_BF16)
    assert b >= 5 * a - 512 and b > a
    assert lib.pka_verify_workspace_size(8, 0, 8, 2, 128, 1000, 4, pka.PKA_BF16) == 0
    assert lib.pka_verify_workspace_size(8, 5, 8, 2, 128, 1000, 4, pka.PKA_F32) == 0
