"""Paged-KV attention with slot-mapped append for AMD MI355X (gfx950).

Thin ctypes binding over ``libpka.so`` (C ABI in ``include/pka.h``).  The
binding only marshals arguments: torch tensors supply device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing or a call
fails, an exception is raised.

Entry points (same names as the C ABI without the ``pka_`` prefix):
  kv_append, kv_append_rope, kv_copy_blocks, attn_prefill_varlen, attn_decode_paged,
  attn_decode_paged_noalloc, attn_verify_paged, attn_mixed_step, decode_workspace_size,
  verify_workspace_size, mixed_workspace_size; and BlockManager, over the
  host block manager (pka_bm_*).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpka.so")

PKA_F32 = 0
PKA_BF16 = 1
PKA_F16 = 2
PKA_FP8_E4M3 = 3  # pools only: OCP E4M3 codes with per-kv-head fp32 scales
BLOCK_SIZE = 16
ROPE_HALF = 0         # rotation pair j = dims (j, j + d/2)
ROPE_INTERLEAVED = 1  # rotation pair j = dims (2j, 2j + 1)

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration",
          -3: "workspace missing or too small", -4: "kernel launch failed", -5: "too few free blocks",
          -6: "split partials exceed the fixed device scratch"}
PKA_ERR_NO_BLOCKS = -5
PKA_ERR_SCRATCH_LIMIT = -6
NOALLOC_SCRATCH_BYTES = 32 << 20  # PKA_NOALLOC_SCRATCH_BYTES

EXPORTS = ["pka_kv_append", "pka_kv_append_rope", "pka_kv_copy_blocks", "pka_attn_prefill_varlen", "pka_attn_decode_paged",
           "pka_attn_decode_paged_noalloc",
           "pka_attn_verify_paged", "pka_attn_mixed_step", "pka_decode_workspace_size",
           "pka_verify_workspace_size", "pka_mixed_workspace_size",
           "pka_status_string", "pka_version", "pka_bm_create", "pka_bm_destroy", "pka_bm_append",
           "pka_bm_release", "pka_bm_tables", "pka_bm_free_blocks", "pka_bm_seq_len"]


class PkaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class KVCacheDesc(ctypes.Structure):
    """Mirror of ``pka_kv_cache``."""
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpka.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_attention_append_amd.build`")
    # torch first: its HIP runtime must be the one libpka.so binds to.  Loaded
    # the other way round, the process would hold the system runtime beside
    # torch's, and kernels launched here would not see torch's allocations.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.pka_kv_append.argtypes = [ctypes.POINTER(KVCacheDesc), P, P, P, I32, P]
    lib.pka_kv_append_rope.argtypes = [ctypes.POINTER(KVCacheDesc), P, P, P, P, I32, P, P, I32, F, I32, P]
    lib.pka_kv_copy_blocks.argtypes = [ctypes.POINTER(KVCacheDesc), ctypes.POINTER(KVCacheDesc), P, I32, P]
    lib.pka_attn_prefill_varlen.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P]
    lib.pka_attn_decode_paged.argtypes = [P, P, ctypes.POINTER(KVCacheDesc), P, I32, P, P, I32, I32, I32,
                                          F, I32, P, SZ, P]
    lib.pka_attn_decode_paged_noalloc.argtypes = [P, P, ctypes.POINTER(KVCacheDesc), P, I32, P, P, I32, I32, I32,
                                                  F, I32, P]
    lib.pka_attn_verify_paged.argtypes = [P, P, ctypes.POINTER(KVCacheDesc), P, I32, P, P, I32, I32, I32, I32,
                                          F, I32, P, SZ, P]
    lib.pka_verify_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
    lib.pka_verify_workspace_size.restype = SZ
    lib.pka_attn_mixed_step.argtypes = [P, P, ctypes.POINTER(KVCacheDesc), P, P, P, P, P, I32, I32, I32,
                                        F, P, SZ, P]
    lib.pka_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.pka_decode_workspace_size.restype = SZ
    lib.pka_mixed_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pka_mixed_workspace_size.restype = SZ
    lib.pka_status_string.argtypes = [ctypes.c_int]
    lib.pka_status_string.restype = ctypes.c_char_p
    lib.pka_version.restype = ctypes.c_int
    lib.pka_bm_create.argtypes = [I32, I32, I32]
    lib.pka_bm_create.restype = P
    lib.pka_bm_destroy.argtypes = [P]
    lib.pka_bm_destroy.restype = None
    lib.pka_bm_append.argtypes = [P, P, P, I32, P]
    lib.pka_bm_release.argtypes = [P, I32, P, P]
    lib.pka_bm_tables.argtypes = [P, P, I32, P, P]
    lib.pka_bm_free_blocks.argtypes = [P]
    lib.pka_bm_free_blocks.restype = I32
    lib.pka_bm_seq_len.argtypes = [P, I32]
    lib.pka_bm_seq_len.restype = I32
    for fn in ("pka_bm_append", "pka_bm_release", "pka_bm_tables"):
        getattr(lib, fn).restype = ctypes.c_int
    for fn in ("pka_kv_append", "pka_kv_append_rope", "pka_kv_copy_blocks", "pka_attn_prefill_varlen", "pka_attn_decode_paged",
               "pka_attn_decode_paged_noalloc", "pka_attn_verify_paged", "pka_attn_mixed_step"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise PkaError(fn, status)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PKA_BF16
    if t.dtype == torch.float32:
        return PKA_F32
    if t.dtype == torch.float16:
        return PKA_F16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):  # fp8 pools hold raw E4M3 codes
        return PKA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpka must be contiguous")
    return t.data_ptr()


def _host_i32(t):
    """Pointer to host int32 data (a contiguous CPU tensor or numpy array)."""
    import numpy as np
    if hasattr(t, "data_ptr"):
        if t.device.type != "cpu" or t.dtype != _torch().int32 or not t.is_contiguous():
            raise ValueError("host index arrays must be contiguous CPU int32 tensors")
        return t.data_ptr(), t
    a = np.ascontiguousarray(t, dtype=np.int32)
    return a.ctypes.data, a


_raw_stream = None


def _stream(stream, ref=None) -> int:
    """HIP stream handle: ``stream``'s, else the current stream of the device
    holding tensor ``ref`` (else of the current device).  torch's raw-stream
    query is used when it exists: it costs 0.1 us against about 3 us for
    building a Stream object, which matters for launch-bound steps."""
    if stream is not None:
        return stream.cuda_stream
    global _raw_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    idx = ref.device.index if ref is not None and ref.device.index is not None else torch.cuda.current_device()
    if _raw_stream:
        return _raw_stream(idx)
    return torch.cuda.current_stream(idx).cuda_stream


@dataclass
class KVCache:
    """A paged KV cache: two torch device buffers in the library's pool layout.

    Each pool holds ``num_blocks * num_kv_heads * 16 * head_dim`` elements;
    the tile of (block, kv head) is contiguous (see include/pka.h).

    fp8 pools (torch.uint8 of E4M3 codes) also carry ``act_dtype`` (PKA_BF16
    or PKA_F16: the dtype of q, new keys/values and outputs) and the device
    fp32 per-kv-head scales ``k_scale`` / ``v_scale``.
    """
    k_pool: "object"
    v_pool: "object"
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    act_dtype: int = 0
    k_scale: "object" = None
    v_scale: "object" = None

    @classmethod
    def allocate(cls, num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda", fill=None,
                 pinned_host: bool = False, act_dtype=None, k_scale=None, v_scale=None):
        """Device pools, or with ``pinned_host`` pinned host pools (a swap
        region that ``kv_copy_blocks`` reads and writes from the GPU).  For an
        fp8 cache pass ``dtype=torch.uint8``, the activation torch dtype and
        the scale tensors."""
        torch = _torch()
        n = num_blocks * num_kv_heads * BLOCK_SIZE * head_dim
        if pinned_host:
            k = torch.empty(n, dtype=dtype, pin_memory=True)
            v = torch.empty(n, dtype=dtype, pin_memory=True)
            if fill is not None:
                k.fill_(fill)
                v.fill_(fill)
        elif fill is None:
            k = torch.empty(n, dtype=dtype, device=device)
            v = torch.empty(n, dtype=dtype, device=device)
        else:
            k = torch.full((n,), fill, dtype=dtype, device=device)
            v = torch.full((n,), fill, dtype=dtype, device=device)
        act = 0
        if act_dtype is not None:
            act = act_dtype if isinstance(act_dtype, int) else _dtype_code(torch.empty(0, dtype=act_dtype))
        return cls(k, v, num_blocks, num_kv_heads, head_dim, act, k_scale, v_scale)

    @property
    def dtype_code(self) -> int:
        return _dtype_code(self.k_pool)

    @property
    def act_code(self) -> int:
        """dtype code of q, new keys/values and outputs."""
        return self.act_dtype if self.dtype_code == PKA_FP8_E4M3 else self.dtype_code

    def desc(self) -> KVCacheDesc:
        return KVCacheDesc(_ptr(self.k_pool), _ptr(self.v_pool), self.num_blocks, BLOCK_SIZE,
                           self.num_kv_heads, self.head_dim, self.dtype_code, self.act_dtype,
                           _ptr(self.k_scale), _ptr(self.v_scale))


def kv_append(cache: KVCache, k_new, v_new, slot_mapping, stream=None):
    """Write ``k_new, v_new [T][Hkv][d]`` into the pools at ``slot_mapping [T]`` (device int32)."""
    lib = load_library()
    desc = cache.desc()
    n = int(slot_mapping.shape[0])
    st = lib.pka_kv_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n,
                           _stream(stream, slot_mapping))
    _check("pka_kv_append", st)


def kv_append_rope(cache: KVCache, k_new, v_new, slot_mapping, positions, q=None, q_out=None,
                   rope_base: float = 10000.0, rope_style: int = ROPE_HALF, stream=None):
    """Append with rotary position embedding: ``k_new`` rows rotated by their
    token's ``positions[t]`` (device int32 ``[T]``) and stored at
    ``slot_mapping``, ``v_new`` stored as is; if ``q`` ``[T][Hq][d]`` is given
    it is rotated into ``q_out`` (default: in place).  Returns ``q_out``."""
    lib = load_library()
    desc = cache.desc()
    n = int(slot_mapping.shape[0])
    if q is not None and q_out is None:
        q_out = q
    hq = int(q.shape[1]) if q is not None else 0
    st = lib.pka_kv_append_rope(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(positions),
                                n, _ptr(q), _ptr(q_out), hq, float(rope_base), int(rope_style),
                                _stream(stream, slot_mapping))
    _check("pka_kv_append_rope", st)
    return q_out


def kv_copy_blocks(src: KVCache, dst: KVCache, block_pairs, stream=None):
    """Copy whole blocks (K and V, all heads): ``block_pairs`` is a device int32
    ``[n][2]`` tensor of (source block in ``src``, destination block in ``dst``).
    Either cache may be a pinned host cache (swap region)."""
    lib = load_library()
    sd, dd = src.desc(), dst.desc()
    n = int(block_pairs.shape[0]) if block_pairs is not None else 0
    st = lib.pka_kv_copy_blocks(ctypes.byref(sd), ctypes.byref(dd), _ptr(block_pairs) if n else None, n,
                                _stream(stream, block_pairs if n else None))
    _check("pka_kv_copy_blocks", st)


def attn_prefill_varlen(q, k, v, cu_seqlens, cu_seqlens_host, scale: float = 0.0, out=None, stream=None):
    """Causal prefill; q ``[T][Hq][d]``, k/v ``[T][Hkv][d]``, cu_seqlens device int32 ``[B+1]``."""
    torch = _torch()
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    hptr, keep = _host_i32(cu_seqlens_host)
    st = lib.pka_attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens), hptr,
                                     int(cu_seqlens.shape[0]) - 1, int(q.shape[1]), int(k.shape[1]),
                                     int(q.shape[2]), _dtype_code(q), float(scale), _stream(stream, q))
    del keep
    _check("pka_attn_prefill_varlen", st)
    return out


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits=0,
                          dtype_code=PKA_BF16) -> int:
    return int(load_library().pka_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                        max_kv_len, num_splits, dtype_code))


def mixed_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_kv_len, dtype_code=PKA_BF16) -> int:
    return int(load_library().pka_mixed_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                       max_kv_len, dtype_code))


def _workspace(nbytes, workspace, device):
    """(workspace, its size in bytes): a new one of ``nbytes`` when none is
    given (none at all for 0 bytes); nbytes < 0 means the caller's workspace
    is passed as it is."""
    if nbytes == 0 and workspace is None:
        return None, 0
    if workspace is None:
        workspace = _torch().empty(nbytes, dtype=_torch().uint8, device=device)
    return workspace, int(workspace.numel() * workspace.element_size())


def attn_decode_paged(q, cache: KVCache, block_tables, kv_lens, max_kv_len: int, scale: float = 0.0,
                      num_splits: int = 0, workspace=None, out=None, stream=None, kv_lens_host=None):
    """Paged decode; q ``[B][Hq][d]``, block_tables device int32 ``[B][max_blocks]``, kv_lens ``[B]``.
    ``kv_lens_host`` (optional, host int32 ``[B]``): the lengths on the host, a
    scheduling hint (longest sequences dispatched first)."""
    torch = _torch()
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    B, hq, d = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    if workspace is None:  # else the library checks the given workspace's size itself
        need = decode_workspace_size(B, hq, cache.num_kv_heads, d, max_kv_len, num_splits, cache.dtype_code)
    workspace, wbytes = _workspace(need if workspace is None else -1, workspace, q.device)
    desc = cache.desc()
    hptr, keep = _host_i32(kv_lens_host) if kv_lens_host is not None else (None, None)
    st = lib.pka_attn_decode_paged(_ptr(q), _ptr(out), ctypes.byref(desc), _ptr(block_tables),
                                   int(block_tables.shape[1]), _ptr(kv_lens), hptr, B, int(max_kv_len), hq,
                                   float(scale), int(num_splits), _ptr(workspace), wbytes, _stream(stream, q))
    del keep
    _check("pka_attn_decode_paged", st)
    return out


def attn_decode_paged_noalloc(q, cache: KVCache, block_tables, kv_lens, max_kv_len: int, scale: float = 0.0,
                              num_splits: int = 0, out=None, stream=None, kv_lens_host=None):
    """Paged decode whose split partials live in the library's fixed device
    scratch (no workspace, nothing allocated by the call; ``out`` is allocated
    here only when not given).  Same arguments and bit-identical results as
    ``attn_decode_paged``; plans needing more than NOALLOC_SCRATCH_BYTES of
    partials raise PkaError with status PKA_ERR_SCRATCH_LIMIT.  Calls that
    overlap on one GPU share the scratch and race."""
    torch = _torch()
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    B, hq = int(q.shape[0]), int(q.shape[1])
    desc = cache.desc()
    hptr, keep = _host_i32(kv_lens_host) if kv_lens_host is not None else (None, None)
    st = lib.pka_attn_decode_paged_noalloc(_ptr(q), _ptr(out), ctypes.byref(desc), _ptr(block_tables),
                                           int(block_tables.shape[1]), _ptr(kv_lens), hptr, B, int(max_kv_len), hq,
                                           float(scale), int(num_splits), _stream(stream, q))
    del keep
    _check("pka_attn_decode_paged_noalloc", st)
    return out


def verify_workspace_size(num_seqs, num_q_per_seq, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                          num_splits=0, dtype_code=PKA_BF16) -> int:
    return int(load_library().pka_verify_workspace_size(num_seqs, num_q_per_seq, num_q_heads, num_kv_heads,
                                                        head_dim, max_kv_len, num_splits, dtype_code))


def attn_verify_paged(q, cache: KVCache, block_tables, kv_lens, max_kv_len: int, scale: float = 0.0,
                      num_splits: int = 0, workspace=None, out=None, stream=None, kv_lens_host=None):
    """Speculative verify: q ``[B][nq][Hq][d]`` (nq = k + 1 rows per sequence at
    the end of its kv_lens[s] keys), block_tables ``[B][max_blocks]``, kv_lens ``[B]``."""
    torch = _torch()
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    B, nq, hq, d = int(q.shape[0]), int(q.shape[1]), int(q.shape[2]), int(q.shape[3])
    if workspace is None:  # else the library checks the given workspace's size itself
        need = verify_workspace_size(B, nq, hq, cache.num_kv_heads, d, max_kv_len, num_splits, cache.dtype_code)
    workspace, wbytes = _workspace(need if workspace is None else -1, workspace, q.device)
    desc = cache.desc()
    hptr, keep = _host_i32(kv_lens_host) if kv_lens_host is not None else (None, None)
    st = lib.pka_attn_verify_paged(_ptr(q), _ptr(out), ctypes.byref(desc), _ptr(block_tables),
                                   int(block_tables.shape[1]), _ptr(kv_lens), hptr, B, nq, int(max_kv_len), hq,
                                   float(scale), int(num_splits), _ptr(workspace), wbytes, _stream(stream, q))
    del keep
    _check("pka_attn_verify_paged", st)
    return out


def attn_mixed_step(q, cache: KVCache, cu_q_lens, cu_q_lens_host, kv_lens, kv_lens_host, block_tables,
                    scale: float = 0.0, workspace=None, out=None, stream=None):
    """Mixed chunked-prefill + decode step over rows packed by ``cu_q_lens``."""
    import numpy as np
    torch = _torch()
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    cptr, keep_c = _host_i32(cu_q_lens_host)
    kptr, keep_k = _host_i32(kv_lens_host)
    B = int(keep_c.shape[0]) - 1
    hq, d = int(q.shape[1]), int(q.shape[2])
    if workspace is None:  # else the library checks the given workspace's size itself
        cu_np = np.asarray(keep_c.numpy() if hasattr(keep_c, "numpy") else keep_c)
        kv_np = np.asarray(keep_k.numpy() if hasattr(keep_k, "numpy") else keep_k)
        dec = (cu_np[1:] - cu_np[:-1]) == 1
        max_dec = int(kv_np[dec].max()) if dec.any() else 1
        need = mixed_workspace_size(B, hq, cache.num_kv_heads, d, max_dec, cache.dtype_code) if dec.any() else 0
        workspace, wbytes = _workspace(need, None, q.device)
    else:
        workspace, wbytes = _workspace(-1, workspace, q.device)
    desc = cache.desc()
    st = lib.pka_attn_mixed_step(_ptr(q), _ptr(out), ctypes.byref(desc), _ptr(cu_q_lens), cptr,
                                 _ptr(kv_lens), kptr, _ptr(block_tables), int(block_tables.shape[1]), B, hq,
                                 float(scale), _ptr(workspace), wbytes, _stream(stream, q))
    del keep_c, keep_k
    _check("pka_attn_mixed_step", st)
    return out


class BlockManager:
    """Host block manager (``pka_bm_*``): block tables, lengths and slot
    mappings for the attention calls.  numpy int32 arrays in and out; host
    memory only."""

    def __init__(self, num_blocks: int, max_seqs: int, max_blocks_per_seq: int):
        self._lib = load_library()
        self.num_blocks, self.max_seqs, self.max_blocks_per_seq = num_blocks, max_seqs, max_blocks_per_seq
        self._h = self._lib.pka_bm_create(num_blocks, max_seqs, max_blocks_per_seq)
        if not self._h:
            raise PkaError("pka_bm_create", -1)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pka_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @staticmethod
    def _i32(a):
        import numpy as np
        return np.ascontiguousarray(np.asarray(a, dtype=np.int32))

    def append(self, seqs, num_new):
        """Grow seqs[i] by num_new[i] tokens; returns the step's slot mapping (int32)."""
        import numpy as np
        seqs, num_new = self._i32(seqs).reshape(-1), self._i32(num_new).reshape(-1)
        if seqs.shape != num_new.shape:
            raise ValueError("seqs and num_new differ in length")
        slots = np.empty(int(num_new.clip(min=0).sum()), np.int32)
        _check("pka_bm_append", self._lib.pka_bm_append(self._h, seqs.ctypes.data, num_new.ctypes.data,
                                                        len(seqs), slots.ctypes.data))
        return slots

    def release(self, seq: int):
        """Free every block of `seq`; returns the freed block ids in table order."""
        import numpy as np
        freed = np.empty(self.max_blocks_per_seq, np.int32)
        n = ctypes.c_int32(0)
        _check("pka_bm_release", self._lib.pka_bm_release(self._h, seq, freed.ctypes.data, ctypes.byref(n)))
        return freed[:n.value].copy()

    def tables(self, seqs):
        """(block_tables [n][max_blocks_per_seq], kv_lens [n]) of `seqs`, int32; -1 past each sequence's blocks."""
        import numpy as np
        seqs = self._i32(seqs).reshape(-1)
        tab = np.empty((len(seqs), self.max_blocks_per_seq), np.int32)
        lens = np.empty(len(seqs), np.int32)
        _check("pka_bm_tables", self._lib.pka_bm_tables(self._h, seqs.ctypes.data, len(seqs), tab.ctypes.data,
                                                        lens.ctypes.data))
        return tab, lens

    @property
    def free_blocks(self) -> int:
        return int(self._lib.pka_bm_free_blocks(self._h))

    def seq_len(self, seq: int) -> int:
        return int(self._lib.pka_bm_seq_len(self._h, seq))
