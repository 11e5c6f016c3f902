"""fp64 CPU oracle for paged-KV attention with slot-mapped append.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library (no kernels, headers, helpers,
constants or pre/post-processing); its inputs come from the seeded generator
in ``paged_kv_attention_append_amd/workloads.py``, which holds none of the
method's arithmetic.

What it computes, and the passages it follows:

* ``attention``  -- causal scaled dot-product attention of every query row
  over the keys/values of its own sequence, read from *contiguous* per-
  sequence K/V in logical order (it never sees blocks, slots or splits).
  Prefill attends over the whole prompt; decode attends one new token over
  the cached past keys/values plus itself (TGI router deep-dive, xxmr.cn,
  section "Prefill, Decode and past key values").  A prefill chunk and the
  running decodes share one forward (same article, the paragraph on prefill
  chunking in "the scheduling loop from the source code").  The pages name
  flash-attention and Paged Attention as the kernels (TGI overview note,
  dongnian.icu, feature list) but print no formula; the oracle is the plain
  definition softmax(Q K^T * scale + causal mask) V, scale = 1/sqrt(d).
* ``paged_layout`` -- the KV pool's layout formula: where the append puts
  each new key/value element, how a block table reads them back, and the
  slot of a sequence position given its block-table row (what the block
  manager hands out).  The
  pages only say the server keeps a GPU region for the KV cache (BlitzScale
  documentation, server components: CacheManager) and that blocks come from
  the router's block allocator (TGI architecture page, "The Router").
* ``brute`` -- an independent pure-Python scalar implementation used only to
  pin ``attention`` on tiny inputs.
* ``fp8`` -- the fp8 KV cache's quantization: OCP E4M3 codes of x / scale
  (nearest, ties to even, saturating at 448) and their decoding.  The pages
  list an fp8 option (TGI architecture page, launcher options) without an
  encoding; the attention oracle then runs on scale * decode(code).

* ``rope`` -- the rotary position embedding applied by the fused append:
  pair j of a head's dims, (j, j + d/2) or (2j, 2j + 1), rotated by
  pos * base^(-2j/d).  The pages enable one position-encoding mode in the
  attention build (BlitzScale documentation, "Build") without defining it;
  the reading is the rotary embedding of the RoFormer paper.

Every function here is pinned by tests under ``tests/`` marked ``not gpu``
(brute force, closed forms, invariants, hand-derived golden fixtures).
"""
