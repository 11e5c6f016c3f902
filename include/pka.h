/*
 * pka.h -- paged-KV attention with slot-mapped append, C ABI.
 *
 * The per-step attention work of a continuous-batching LLM server on one AMD
 * MI355X (gfx950): write the new tokens' keys/values into fixed-size KV
 * blocks, then attend -- causal prefill over prompts packed by cu_seqlens,
 * decode of one new token per running sequence against its own block table,
 * or a mixed step holding prefill chunks and decodes together.
 *
 * Sources for the operations (web pages; no page prints code or formulas):
 *   - Prefill computes attention over the whole prompt; later decode passes
 *     attend only the new token against cached past keys/values: TGI router
 *     deep-dive (xxmr.cn), section "Prefill, Decode and past key values".
 *   - Requests join and leave the batch between forward steps and a finished
 *     request frees all of its memory: same article, "Continuous batching".
 *   - With prefill chunking, new prompts are concatenated with the running
 *     batch and prefilled in the same forward: same article, the prefill
 *     chunking paragraph of the scheduling-loop section.
 *   - The kernels are flash-attention and Paged Attention: TGI overview note
 *     (dongnian.icu), feature list; the v3 server protocol adds paged
 *     attention: TGI architecture page (data-sketchers wiki), model server.
 *   - Fixed-size blocks are handed out by the router's block allocator: TGI
 *     architecture page, "The Router"; the server keeps a GPU KV region:
 *     BlitzScale documentation, server components (CacheManager).
 *   - Head dim 128: BlitzScale documentation, "Build" (kernel generation
 *     flags).
 *
 * Attention computed by every entry point: for a sequence with kv_len keys of
 * which q_len are new this step, query row i (absolute position
 * p = kv_len - q_len + i) attends keys 0..p, its own key included;
 *   o = softmax(scale * q K^T) V, scale = 1/sqrt(head_dim) when scale <= 0.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 *   Pointers: all data pointers are DEVICE pointers unless the name ends in
 *     _host (host memory read during the call).  The caller owns every buffer
 *     and keeps it alive until the stream work has finished; the attention,
 *     append and copy calls allocate nothing, and the library keeps no
 *     mutable global state (thread-safe), except the fixed device scratch of
 *     pka_attn_decode_paged_noalloc (see there).  The one allocation is a
 *     block manager's host memory (pka_bm_create / pka_bm_destroy, below).
 *   Streams: `stream` is a hipStream_t (NULL = default stream).  Every call is
 *     asynchronous on it; the library never synchronises the device.
 *   Dtypes: PKA_F32 (IEEE binary32), PKA_BF16 (bfloat16) or PKA_F16 (IEEE
 *     binary16; the server's --dtype float16: TGI architecture page, launcher
 *     options).  Q, K, V, the pools and the output share one dtype, except
 *     for an fp8 cache (PKA_FP8_E4M3 pools, see pka_kv_cache), whose q, new
 *     keys/values and outputs use its act_dtype (bf16 or fp16).  Scores,
 *     softmax and accumulation are fp32; 16-bit outputs are rounded to
 *     nearest-even.  In the 16-bit paths the softmax weights are rounded to
 *     the dtype before the P*V product and the softmax denominator sums
 *     those rounded weights.
 *   Head dims: 64 or 128.  Block size: 16 tokens.
 *   Errors: every call returns an int status; no exceptions or aborts cross
 *     the ABI.  On a non-zero return nothing has been launched, except for
 *     PKA_ERR_LAUNCH (a HIP launch error reported after enqueueing).
 *   Device-side contract (not checked on the host, since the data lives on
 *     the device): block ids in [0, num_blocks), unique slots per append,
 *     kv_len <= max_blocks_per_seq * 16, kv_len >= 1 for a decode row.  When
 *     violated the kernels clamp indexes to stay inside the buffers they were
 *     given, so results are undefined but no access leaves those buffers.
 *
 * KV pool layout (one pool for K, one for V, both caller-allocated, same
 * layout): [num_blocks][num_kv_heads][16][head_dim], row-major.  The element
 * (block b, kv head g, token offset t in 0..15, dim i) is at
 *     ((b * num_kv_heads + g) * 16 + t) * head_dim + i
 * so each (block, kv head) tile of 16 * head_dim elements is contiguous (4 KiB
 * for bf16, d=128) and each token's row of one head is contiguous (256 B).  A
 * token with slot s is at block s / 16, offset s % 16.  All offsets are
 * computed in 64 bits.
 * ------------------------------------------------------------------------- */
#ifndef PKA_H_
#define PKA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKA_VERSION 4

enum pka_status {
  PKA_OK = 0,
  PKA_ERR_INVALID = -1,     /* null pointer, bad size or inconsistent lengths  */
  PKA_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, block_size != 16, bad dtype */
  PKA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
  PKA_ERR_LAUNCH = -4,      /* HIP reported an error for a kernel launch       */
  PKA_ERR_NO_BLOCKS = -5,   /* block manager: too few free blocks in the pool  */
  PKA_ERR_SCRATCH_LIMIT = -6 /* no-allocation call: partials exceed the fixed scratch */
};

enum pka_dtype { PKA_F32 = 0, PKA_BF16 = 1, PKA_F16 = 2, PKA_FP8_E4M3 = 3 /* pools only */ };

/* Description of a paged KV cache.  k_pool / v_pool are device buffers of
 * num_blocks * num_kv_heads * block_size * head_dim elements each, laid out
 * as documented above.  block_size must be 16.
 *
 * fp8 KV cache (dtype = PKA_FP8_E4M3): each pool element is one byte, an OCP
 * E4M3 code (bias 7, no infinities, S.1111.111 = NaN, largest finite 448).
 * act_dtype (PKA_BF16 or PKA_F16) is then the dtype of q, of the new keys /
 * values given to pka_kv_append and of every output.  k_scale / v_scale are
 * device fp32 arrays [num_kv_heads] (positive, finite): the append stores
 * code = E4M3(x / scale[g]) -- the fp32 quotient rounded to the nearest code,
 * ties to the even code, saturating at +-448 -- and attention uses the key
 * scale[g] * decode(code).  For the other dtypes act_dtype is 0 or equal to
 * dtype and the scales are NULL.  The pages list an fp8 option for the
 * server (TGI architecture page, launcher options) without its encoding. */
typedef struct pka_kv_cache {
  void* k_pool;
  void* v_pool;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;          /* enum pka_dtype: pool elements */
  int32_t act_dtype;      /* fp8 pools: dtype of q, new k/v and outputs; else 0 or dtype */
  const float* k_scale;   /* fp8 pools: device fp32 [num_kv_heads]; else NULL */
  const float* v_scale;
} pka_kv_cache;

/* Slot-mapped append.
 * Copies token t's key and value rows (k_new/v_new are [num_tokens][num_kv_heads]
 * [head_dim], row-major, in the cache's dtype -- its act_dtype for fp8 pools)
 * into the pool slot slot_mapping[t] (device int32 [num_tokens]), bit-exactly
 * (fp8 pools: quantized as described at pka_kv_cache).  A negative slot skips the token
 * (padding); a slot >= num_blocks * 16 is also skipped.  Slots must be unique
 * within a call.  num_tokens == 0 is a no-op.
 * Page reference: past keys/values are cached after prefill and reused by
 * each decode (TGI router deep-dive, "Prefill, Decode and past key values");
 * the cache is made of allocator blocks (TGI architecture page, "The Router").
 * Errors: PKA_ERR_INVALID for null cache/pointers or num_tokens < 0;
 * PKA_ERR_UNSUPPORTED for an unsupported cache description. */
int pka_kv_append(const pka_kv_cache* cache, const void* k_new, const void* v_new,
                  const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* Rotary position embedding styles for pka_kv_append_rope: which head dims
 * form rotation pair j (j < head_dim / 2). */
enum pka_rope_style {
  PKA_ROPE_HALF = 0,        /* dims (j, j + head_dim/2) */
  PKA_ROPE_INTERLEAVED = 1  /* dims (2j, 2j + 1) */
};

/* Slot-mapped append fused with the rotary position embedding (RoPE) of the
 * step's keys and queries.
 * For token t at position positions[t] (device int32 [num_tokens], any
 * integer), rotation pair j of every head row turns by the angle
 * positions[t] * theta_j, theta_j = rope_base^(-2j/head_dim):
 * (a, b) -> (a cos - b sin, a sin + b cos), a and b the pair's two dims.
 * - Keys: k_new rows are rotated and stored at slot_mapping[t] as in
 *   pka_kv_append (fp8 pools: the rotated fp32 value is quantized with
 *   k_scale as described above).  Slots < 0 or >= num_blocks * 16 are skipped.
 * - Values: v_new rows are stored unrotated, as pka_kv_append stores them.
 * - Queries: when q is not NULL, q [num_tokens][num_q_heads][head_dim] is
 *   rotated into q_out (same shape; q_out == q rotates in place), whatever the
 *   token's slot.  q and q_out are both NULL or both non-NULL.
 * Inputs and q_out use the cache's activation dtype; 16-byte aligned.  The
 * angles are evaluated in fp64 and the rotation in fp32: each result is
 * within 2^-22 (|a| + |b|) of the exact rotation before its final rounding.
 * Page reference: the attention build enables one position-encoding mode
 * (BlitzScale documentation, "Build"), read as the rotary embedding of the
 * RoFormer paper; keys are cached after the encoding (TGI router deep-dive,
 * "Prefill, Decode and past key values").
 * Errors: PKA_ERR_INVALID (null cache / k_new / v_new / slot_mapping /
 * positions, num_tokens < 0, misaligned buffers, only one of q and q_out,
 * num_q_heads < 1 with q, rope_base not positive and finite, unknown style);
 * PKA_ERR_UNSUPPORTED for an unsupported cache description. */
int pka_kv_append_rope(const pka_kv_cache* cache, const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, const int32_t* positions, int32_t num_tokens,
                       const void* q, void* q_out, int32_t num_q_heads, float rope_base, int32_t rope_style,
                       void* stream);

/* Block copy between paged pools: copy-on-write inside one pool, swap out to
 * and swap in from a host-memory region.
 * For every pair i < num_pairs of block_pairs (device int32 [num_pairs][2] =
 * {source block, destination block}), the destination block of `dst` receives
 * the K and V contents of the source block of `src` -- all kv heads, all 16
 * slots -- bit-exactly.  src and dst must agree in num_kv_heads, head_dim,
 * dtype and block_size; they may describe the same pools.  Each pool may be
 * device memory or pinned host memory (hipHostMalloc / a pinned torch
 * tensor), which the kernel reads or writes across the host link; pageable
 * host memory is rejected.  A pair with either id outside [0, num_blocks) of
 * its cache is skipped.  The pairs run in parallel: destinations must be
 * distinct, and when src and dst share a pool no destination may also be a
 * source of the same call (otherwise the result is undefined).
 * num_pairs == 0 is a no-op.
 * Page reference: the server's cache manager holds a GPU KV region and a CPU
 * KV region (BlitzScale documentation, server components: CacheManager); a
 * finished request frees its blocks (TGI router deep-dive, "Continuous
 * batching").
 * Errors: PKA_ERR_INVALID (null caches or pairs, num_pairs < 0, mismatched
 * caches, a pool that is neither device memory nor pinned host memory);
 * PKA_ERR_UNSUPPORTED for an unsupported cache description. */
int pka_kv_copy_blocks(const pka_kv_cache* src, const pka_kv_cache* dst, const int32_t* block_pairs,
                       int32_t num_pairs, void* stream);

/* Varlen causal prefill over prompts packed by cu_seqlens.
 * q/out: [T][num_q_heads][head_dim]; k/v: [T][num_kv_heads][head_dim], where
 * T = cu_seqlens_host[num_seqs]; prompt s owns rows cu[s]..cu[s+1]-1 and
 * attends only its own tokens with a causal mask.  cu_seqlens (device) and
 * cu_seqlens_host (host) hold the same num_seqs+1 int32 values; cu[0] == 0,
 * non-decreasing.  The host copy sizes the launch.
 * Page reference: prefill is the first full pass over the prompt (TGI router
 * deep-dive, "Prefill, Decode and past key values"); the batch is ragged,
 * indexed by a ragged index pointer (BlitzScale documentation, server
 * components: ragged_indptr).
 * The launch shape (32 or 48 query rows per wave) is chosen from the amount
 * of work; the environment variable PKA_PREFILL_UNIT_ROWS = 32 or 48 fixes
 * it (both give the same output bit for bit).
 * Errors: PKA_ERR_INVALID (null pointers, num_seqs < 0, heads < 1,
 * num_q_heads % num_kv_heads != 0, cu not starting at 0 or decreasing);
 * PKA_ERR_UNSUPPORTED (dtype, head_dim). */
int pka_attn_prefill_varlen(const void* q, const void* k, const void* v, void* out,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, float scale, void* stream);

/* Paged decode: one query token per sequence.
 * q/out: [num_seqs][num_q_heads][head_dim].  Sequence s attends its kv_lens[s]
 * keys (device int32 [num_seqs], this step's token included and already
 * appended), read through block_tables[s][0..] (device int32
 * [num_seqs][max_blocks_per_seq]).  max_kv_len (host) must be >= every
 * kv_lens[s] and sizes the split plan.
 * kv_lens_host (optional, host int32 [num_seqs], NULL allowed): the same
 * lengths on the host, a scheduling hint: with it (up to 1024 sequences) the
 * work is dispatched longest sequence first and the automatic plan takes
 * fewer, longer chunks, which shortens the end of the launch.  Any order
 * computes the same attention, so a stale hint costs time, never accuracy;
 * the workspace size does not depend on it.
 * Split context: the key range of a sequence is cut into fixed-size chunks
 * processed in parallel; per-chunk (o, max, sum) partials go to `workspace` and
 * a second pass merges them with a log-sum-exp rescale.  num_splits = 0 picks
 * the count automatically; >= 1 caps the chunks per sequence.  workspace must
 * hold pka_decode_workspace_size(...) bytes for the same arguments (it may be
 * NULL when that size is 0).
 * Page reference: decode attends the new token only, against the cached past
 * keys/values (TGI router deep-dive, "Prefill, Decode and past key values");
 * generation is memory bound (same article, "Continuous batching").
 * Errors: PKA_ERR_INVALID, PKA_ERR_UNSUPPORTED, PKA_ERR_WORKSPACE. */
int pka_attn_decode_paged(const void* q, void* out, const pka_kv_cache* cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs, int32_t max_kv_len,
                          int32_t num_q_heads, float scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch of pka_attn_decode_paged_noalloc (32 MiB
 * per GPU the library runs on, held until the process ends). */
#define PKA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Paged decode that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments, results and
 * errors are those of pka_attn_decode_paged without workspace /
 * workspace_bytes; the same kernels run with the same split plan, so the
 * output is bit-identical to pka_attn_decode_paged's.  The split partials
 * go to a fixed PKA_NOALLOC_SCRATCH_BYTES device array of the library (one
 * per GPU; the GPU is the current device, which must be the stream's).
 * Plans whose partials need more than that (pka_decode_workspace_size(...)
 * > PKA_NOALLOC_SCRATCH_BYTES) are rejected with PKA_ERR_SCRATCH_LIMIT before
 * anything is launched.  No memory is allocated or freed by the call.  Every
 * call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads) race
 * and give undefined results; calls ordered on one stream are safe.  Nothing
 * in the scratch needs to start at zero (each call writes every partial it
 * reads). */
int pka_attn_decode_paged_noalloc(const void* q, void* out, const pka_kv_cache* cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs,
                                  int32_t max_kv_len, int32_t num_q_heads, float scale, int32_t num_splits,
                                  void* stream);

/* Bytes of workspace pka_attn_decode_paged needs for these arguments (fp32
 * partials, so the same for every 16-bit or fp8 pool dtype; PKA_F32 pools
 * need none, nor does a plan with one chunk per sequence).  dtype is the
 * cache's pool dtype.  Returns 0 for arguments the call would reject.  The
 * size grows with num_seqs and max_kv_len, so a caller sizes the workspace
 * once for its largest batch and longest context, as the server's warmup
 * call sizes the step from the batch limits before serving (TGI architecture
 * page, call-flow diagram: warmup(max_input_tokens, max_batch_prefill_tokens,
 * max_total_tokens, max_batch_size)). */
size_t pka_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_kv_len, int32_t num_splits,
                                 int32_t dtype);

/* Speculative verify: num_q_per_seq (= k + 1, 1..64) new query rows per
 * sequence -- the last accepted token and k draft tokens -- at the end of
 * its kv_lens[s] keys, all already appended.  q/out: [num_seqs][num_q_per_seq]
 * [num_q_heads][head_dim]; row r of sequence s sits at absolute position
 * kv_lens[s] - num_q_per_seq + r and attends keys 0 .. that position (the same
 * bottom-right causal rule as every entry point), so row num_q_per_seq - 1
 * equals a pka_attn_decode_paged row of the same token.  Block tables,
 * kv_lens, kv_lens_host, max_kv_len, split plan and workspace are as in
 * pka_attn_decode_paged (workspace from pka_verify_workspace_size); kv_lens[s]
 * >= num_q_per_seq is a device-side contract (rows that see no key get
 * zeros).  The rows run on the decode unit as extra matrix-core columns
 * (num_q_per_seq * num_q_heads / num_kv_heads per kv head), so they share
 * each K/V block read and get the split-context plan.  bf16 and fp16 only.
 * Page reference: the launcher's speculation option (TGI architecture page,
 * launcher options: --speculate); decode over cached keys/values (TGI router
 * deep-dive, "Prefill, Decode and past key values").
 * Errors: PKA_ERR_INVALID (as decode, num_q_per_seq outside 1..64, max_kv_len <
 * num_q_per_seq); PKA_ERR_UNSUPPORTED (fp32 pools, dims); PKA_ERR_WORKSPACE. */
int pka_attn_verify_paged(const void* q, void* out, const pka_kv_cache* cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs,
                          int32_t num_q_per_seq, int32_t max_kv_len,
                          int32_t num_q_heads, float scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pka_attn_verify_paged needs for these arguments (as
 * pka_decode_workspace_size, and sized once the same way; 0 for arguments the
 * call would reject). */
size_t pka_verify_workspace_size(int32_t num_seqs, int32_t num_q_per_seq, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                 int32_t num_splits, int32_t dtype);

/* Mixed chunked-prefill + decode step, one launch (plus a merge pass when a
 * decode row's keys were split).
 * q/out: [T][num_q_heads][head_dim], T = cu_q_lens_host[num_seqs]; sequence s
 * owns rows cu_q_lens[s]..cu_q_lens[s+1]-1 (q_len_s rows: 1 for a decode, the
 * chunk length for a prefill chunk) and has kv_lens[s] keys in the paged
 * cache, this step's tokens included (append them first, on the same
 * stream).  Row i of s sits at position kv_len_s - q_len_s + i and attends
 * keys 0..that position (bottom-right causal alignment).  Host copies of
 * cu_q_lens and kv_lens size the launch and are validated:
 * 0 <= q_len <= kv_len <= max_blocks_per_seq * 16.
 * workspace must hold pka_mixed_workspace_size(...) bytes.
 * Page reference: with prefill chunking the new prompts run in the same
 * forward as the running decodes (TGI router deep-dive, prefill-chunking
 * paragraph of the scheduling-loop section).
 * Errors: PKA_ERR_INVALID, PKA_ERR_UNSUPPORTED, PKA_ERR_WORKSPACE. */
int pka_attn_mixed_step(const void* q, void* out, const pka_kv_cache* cache,
                        const int32_t* cu_q_lens, const int32_t* cu_q_lens_host,
                        const int32_t* kv_lens, const int32_t* kv_lens_host,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t num_seqs, int32_t num_q_heads, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pka_attn_mixed_step needs (max_kv_len: the largest
 * kv_len of a q_len == 1 row).  Sized once for the largest step, as the
 * server's warmup does (TGI architecture page, call-flow diagram: warmup). */
size_t pka_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_kv_len, int32_t dtype);

/* ---------------------------------------------------------------------------
 * Host block manager: the bookkeeping that produces the block tables, kv_lens
 * and slot mappings the calls above take.  The pages put a block allocator
 * next to the scheduler (TGI architecture page, "The Router": queue,
 * scheduler and block allocator), count the blocks each replica uses
 * (BlitzScale documentation, router: used_blocks) and free everything a
 * query holds once it finishes (TGI router deep-dive, simple continuous
 * batching).  The policy here is this library's own reading: a LIFO free
 * list, so the blocks a finished sequence gives back are the first handed
 * out again.
 *
 * State: num_blocks pool blocks (ids 0 .. num_blocks - 1, all free at first;
 * block 0 is handed out first), max_seqs sequence ids (0 .. max_seqs - 1,
 * each empty at first) and a block-table row of max_blocks_per_seq entries
 * per sequence.  A sequence of length n holds exactly ceil(n / 16) blocks, in
 * table order; its token at position p lives in slot
 *     table[p / 16] * 16 + p % 16.
 * Host memory only (every pointer below is a host pointer); no GPU is used.
 * One manager must not be used from two threads at once; separate managers
 * are independent.  On any non-OK return the manager is unchanged.
 * ------------------------------------------------------------------------- */
typedef struct pka_block_manager pka_block_manager;

/* New manager, or NULL if num_blocks < 1, max_seqs < 1,
 * max_blocks_per_seq < 1, num_blocks or max_blocks_per_seq above
 * INT32_MAX / 16 (slots and lengths are int32), max_seqs * max_blocks_per_seq
 * above 2^31, or memory runs out.  Release with pka_bm_destroy. */
pka_block_manager* pka_bm_create(int32_t num_blocks, int32_t max_seqs, int32_t max_blocks_per_seq);
void pka_bm_destroy(pka_block_manager* bm);

/* Grows sequence seqs[i] by num_new[i] tokens for i in 0 .. n - 1 (the new
 * tokens of one step), taking the blocks they need from the free list in
 * that order, and writes each new token's slot to slots_out, sequence by
 * sequence in the order given and by position within a sequence: slots_out
 * must hold sum(num_new) entries and is the step's slot_mapping.
 * All or nothing: PKA_ERR_NO_BLOCKS if the pool lacks the blocks for the
 * whole step; PKA_ERR_INVALID for a null manager, n < 0, a seq id out of
 * range or repeated, num_new[i] < 0, a length beyond max_blocks_per_seq * 16,
 * or null arrays with n > 0. */
int pka_bm_append(pka_block_manager* bm, const int32_t* seqs, const int32_t* num_new, int32_t n,
                  int32_t* slots_out);

/* Frees every block of sequence seq and sets its length to 0.  The blocks go
 * back on the free list in table order (the sequence's last block is handed
 * out first).  If freed_out is not NULL it receives the freed ids in table
 * order and *num_freed (if not NULL) their count (at most max_blocks_per_seq).
 * Errors: PKA_ERR_INVALID (null manager, seq out of range). */
int pka_bm_release(pka_block_manager* bm, int32_t seq, int32_t* freed_out, int32_t* num_freed);

/* Writes the block-table rows of seqs[0 .. n) to tables_out
 * ([n][max_blocks_per_seq], row-major; entries past a sequence's blocks are
 * -1) and their lengths to kv_lens_out ([n]; may be NULL): the block_tables
 * and kv_lens arguments of the attention calls for those sequences.
 * Errors: PKA_ERR_INVALID (null manager or tables_out with n > 0, n < 0, seq
 * out of range). */
int pka_bm_tables(const pka_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* tables_out,
                  int32_t* kv_lens_out);

/* Free blocks, or -1 for a null manager. */
int32_t pka_bm_free_blocks(const pka_block_manager* bm);

/* Length of sequence seq, or -1 for a null manager or seq out of range. */
int32_t pka_bm_seq_len(const pka_block_manager* bm, int32_t seq);

/* Human-readable name of a status code (static string). */
const char* pka_status_string(int status);

/* PKA_VERSION of the built library. */
int pka_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKA_H_ */
