// C ABI of libpka: argument validation, launch planning, kernel dispatch.
// Every check that can be made on the host is made before anything is
// enqueued, so an error return means no device work was issued (except
// PKA_ERR_LAUNCH).  No function here allocates memory or synchronises.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/pka.h"
#include "pka_internal.h"

using namespace pka;

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;
constexpr int kMaxVerifyRows = 64;  // query rows per sequence in pka_attn_verify_paged

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(int dtype, int head_dim) {
  if (dtype != PKA_F32 && dtype != PKA_BF16 && dtype != PKA_F16) return PKA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKA_ERR_UNSUPPORTED;
  return PKA_OK;
}

int pool_elem_bytes(int dtype) { return dtype == PKA_F32 ? 4 : (dtype == PKA_FP8_E4M3 ? 1 : 2); }

// dtype of q, new k/v and outputs for this cache.
int act_dtype(const pka_kv_cache* c) { return c->dtype == PKA_FP8_E4M3 ? c->act_dtype : c->dtype; }

int check_cache(const pka_kv_cache* c) {
  if (!c) return PKA_ERR_INVALID;
  int st;
  if (c->dtype == PKA_FP8_E4M3) {
    if (c->act_dtype != PKA_BF16 && c->act_dtype != PKA_F16) return PKA_ERR_UNSUPPORTED;
    if (!c->k_scale || !c->v_scale) return PKA_ERR_INVALID;
    st = check_dims(c->act_dtype, c->head_dim);
  } else {
    if (c->act_dtype != 0 && c->act_dtype != c->dtype) return PKA_ERR_INVALID;
    st = check_dims(c->dtype, c->head_dim);
  }
  if (st != PKA_OK) return st;
  if (c->block_size != kBlock) return PKA_ERR_UNSUPPORTED;
  if (c->num_kv_heads < 1 || c->num_blocks < 1) return PKA_ERR_INVALID;
  if ((long long)c->num_blocks * kBlock > 0x7fffffffLL) return PKA_ERR_INVALID;  // slots are int32
  if (!c->k_pool || !c->v_pool || !aligned16(c->k_pool) || !aligned16(c->v_pool)) return PKA_ERR_INVALID;
  return PKA_OK;
}

CacheView view(const pka_kv_cache* c) {
  CacheView v;
  v.k_pool = c->k_pool;
  v.v_pool = c->v_pool;
  v.num_blocks = c->num_blocks;
  v.hkv = c->num_kv_heads;
  v.d = c->head_dim;
  v.dtype = c->dtype;
  v.act_dtype = act_dtype(c);
  v.k_scale = c->k_scale;
  v.v_scale = c->v_scale;
  return v;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

int status_of(hipError_t e) { return e == hipSuccess ? PKA_OK : PKA_ERR_LAUNCH; }

// Checks cu[0] == 0 and monotonicity; returns max step and total.
int scan_cu(const int32_t* cu, int n, int* max_len, long long* total) {
  if (cu[0] != 0) return PKA_ERR_INVALID;
  int mx = 0;
  for (int s = 0; s < n; ++s) {
    const long long len = (long long)cu[s + 1] - cu[s];
    if (len < 0) return PKA_ERR_INVALID;
    if (len > mx) mx = (int)len;
  }
  *max_len = mx;
  *total = cu[n];
  return PKA_OK;
}

}  // namespace

namespace {

// Shape of the prefill unit for one launch (rows per wave, see UnitShape in
// pka_attn_mfma.hip).  The work is counted in 32-key tiles summed over the
// 48-row units; a batch with at most 48 of them per resident 48-row
// workgroup (two per CU) is short enough that the start, the end and the
// granularity of the launch dominate, and runs on 32-row units, three per
// CU (measured: ragged 4096 tokens of prompts up to 893 -10 %, 4 x 1024
// tokens -17 %, 64 x 128 -10 %); more work runs on 48-row units, which read
// each K/V fragment from LDS for more rows (one 8192-token prompt -8 %,
// 8 x 1536 tokens -7 %).
int prefill_rows_per_wave(const int32_t* cu_host, int num_seqs, int G, int heads) {
  // PKA_PREFILL_UNIT_ROWS=32 or 48 fixes the shape (tuning, and the tests,
  // which run every prefill case on both shapes); read on every call.
  if (const char* e = std::getenv("PKA_PREFILL_UNIT_ROWS")) {
    if (std::strcmp(e, "32") == 0) return 2;
    if (std::strcmp(e, "48") == 0) return 3;
  }
  static const int cus = [] {  // compute units of the device (all devices alike on one node)
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = 256;
    }
    return n;
  }();
  const int P = positions_per_wg16(G, 3);
  long long tiles = 0;  // key tiles over the (sequence, 48-row unit) pairs, one head group
  for (int i = 0; i < num_seqs; ++i) {
    const long long len = (long long)cu_host[i + 1] - cu_host[i];
    for (long long r = 0; r < len; r += P) tiles += ((r + P < len ? r + P : len) + kKeyTile - 1) / kKeyTile;
  }
  return tiles * heads <= 48LL * 2 * cus ? 2 : 3;
}

}  // namespace

extern "C" {

int pka_version(void) { return PKA_VERSION; }

const char* pka_status_string(int status) {
  switch (status) {
    case PKA_OK: return "ok";
    case PKA_ERR_INVALID: return "invalid argument";
    case PKA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKA_ERR_WORKSPACE: return "workspace missing or too small";
    case PKA_ERR_LAUNCH: return "kernel launch failed";
    case PKA_ERR_NO_BLOCKS: return "too few free blocks";
    case PKA_ERR_SCRATCH_LIMIT: return "split partials exceed the fixed device scratch";
    default: return "unknown status";
  }
}

int pka_kv_append(const pka_kv_cache* cache, const void* k_new, const void* v_new,
                  const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  int st = check_cache(cache);
  if (st != PKA_OK) return st;
  if (num_tokens < 0) return PKA_ERR_INVALID;
  if (num_tokens == 0) return PKA_OK;
  if (!k_new || !v_new || !slot_mapping || !aligned16(k_new) || !aligned16(v_new)) return PKA_ERR_INVALID;
  const long long chunks = (long long)num_tokens * cache->num_kv_heads * cache->head_dim *
                           pool_elem_bytes(cache->dtype) / 16;
  if ((chunks + kThreads - 1) / kThreads > kMaxGrid) return PKA_ERR_INVALID;
  return status_of(launch_append(view(cache), k_new, v_new, slot_mapping, num_tokens, (hipStream_t)stream));
}

int pka_kv_append_rope(const pka_kv_cache* cache, const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, const int32_t* positions, int32_t num_tokens,
                       const void* q, void* q_out, int32_t num_q_heads, float rope_base, int32_t rope_style,
                       void* stream) {
  int st = check_cache(cache);
  if (st != PKA_OK) return st;
  if (num_tokens < 0) return PKA_ERR_INVALID;
  if (rope_style != PKA_ROPE_HALF && rope_style != PKA_ROPE_INTERLEAVED) return PKA_ERR_INVALID;
  if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return PKA_ERR_INVALID;
  if ((q == nullptr) != (q_out == nullptr)) return PKA_ERR_INVALID;
  if (q && (num_q_heads < 1 || !aligned16(q) || !aligned16(q_out))) return PKA_ERR_INVALID;
  if (num_tokens == 0) return PKA_OK;
  if (!k_new || !v_new || !slot_mapping || !positions || !aligned16(k_new) || !aligned16(v_new))
    return PKA_ERR_INVALID;
  if (num_tokens > kMaxGrid) return PKA_ERR_INVALID;
  const int d = cache->head_dim;
  RopeArgs a = {};
  a.q = q;
  a.q_out = q_out;
  a.hq = q ? num_q_heads : 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.positions = positions;
  for (int j = 0; j < d / 2; ++j) a.theta[j] = std::pow((double)rope_base, -2.0 * j / d);
  return status_of(launch_append_rope(view(cache), a, num_tokens, rope_style == PKA_ROPE_INTERLEAVED,
                                      (hipStream_t)stream));
}

int pka_kv_copy_blocks(const pka_kv_cache* src, const pka_kv_cache* dst, const int32_t* block_pairs,
                       int32_t num_pairs, void* stream) {
  int st = check_cache(src);
  if (st != PKA_OK) return st;
  st = check_cache(dst);
  if (st != PKA_OK) return st;
  if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim || src->dtype != dst->dtype)
    return PKA_ERR_INVALID;  // (fp8 pools: bytes are copied; the scales are the caller's)
  if (num_pairs < 0) return PKA_ERR_INVALID;
  if (num_pairs == 0) return PKA_OK;
  if (!block_pairs || 2LL * num_pairs > kMaxGrid) return PKA_ERR_INVALID;
  // Every pool must be memory the GPU can address: device memory or pinned
  // host memory.  The kernel takes the device-side address of each.
  CacheView sv = view(src), dv = view(dst);
  void** pools[4] = {&sv.k_pool, &sv.v_pool, &dv.k_pool, &dv.v_pool};
  for (void** pp : pools) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, *pp) != hipSuccess) {
      (void)hipGetLastError();  // clear the sticky error of the failed query
      return PKA_ERR_INVALID;
    }
    if ((attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeHost) || !attr.devicePointer)
      return PKA_ERR_INVALID;
    *pp = attr.devicePointer;
  }
  return status_of(launch_copy_blocks(sv, dv, block_pairs, num_pairs, (hipStream_t)stream));
}

int pka_attn_prefill_varlen(const void* q, const void* k, const void* v, void* out,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t dtype, float scale, void* stream) {
  if (num_seqs < 0) return PKA_ERR_INVALID;
  int st = check_dims(dtype, head_dim);
  if (st != PKA_OK) return st;
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0) return PKA_ERR_INVALID;
  if (!cu_seqlens || !cu_seqlens_host) return PKA_ERR_INVALID;
  int max_len = 0;
  long long total = 0;
  st = scan_cu(cu_seqlens_host, num_seqs, &max_len, &total);
  if (st != PKA_OK) return st;
  if (num_seqs == 0 || total == 0) return PKA_OK;
  if (!q || !k || !v || !out) return PKA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PKA_ERR_INVALID;
  RowsProblem p = {};
  p.q = q;
  p.out = out;
  p.cu_q = cu_seqlens;
  p.kv_lens = nullptr;
  p.k = k;
  p.v = v;
  p.num_seqs = num_seqs;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.d = head_dim;
  p.dtype = dtype;
  p.scale = resolve_scale(scale, head_dim);
  p.paged = false;
  p.max_q_len = max_len;
  const hipStream_t s = (hipStream_t)stream;
  if (dtype == PKA_F32) {
    if (num_seqs > 65535 || num_q_heads > 65535) return PKA_ERR_UNSUPPORTED;
    return status_of(launch_rows_valu(p, s));
  }
  const int G = num_q_heads / num_kv_heads;
  const int heads = num_kv_heads * (G / heads_per_wg(G));
  // Longest-first work map (see TileMap) over units of P positions.
  auto build_map = [&](TileMap& map, int P) {
    int nt[kMapSeqs], seq_of_rank[kMapSeqs];
    for (int i = 0; i < num_seqs; ++i) {
      nt[i] = (cu_seqlens_host[i + 1] - cu_seqlens_host[i] + P - 1) / P;
      seq_of_rank[i] = i;
    }
    std::stable_sort(seq_of_rank, seq_of_rank + num_seqs, [&](int x, int y) { return nt[x] > nt[y]; });
    for (int r = 0; r < num_seqs; ++r) {
      map.row0_of_rank[r] = cu_seqlens_host[seq_of_rank[r]];
      map.q_len_of_rank[r] = cu_seqlens_host[seq_of_rank[r] + 1] - cu_seqlens_host[seq_of_rank[r]];
    }
    map.levels = (max_len + P - 1) / P;
    map.heads = heads;
    map.level_start[0] = 0;
    int count = num_seqs;  // ranks with more than l tiles
    for (int l = 0; l < map.levels; ++l) {
      while (count > 0 && nt[seq_of_rank[count - 1]] <= l) --count;
      map.level_start[l + 1] = map.level_start[l] + count * heads;
    }
  };
  p.prefill_rb = prefill_rows_per_wave(cu_seqlens_host, num_seqs, G, heads);
  // The launch is a level grid: (longest prompt's tile count) x sequences x
  // kv heads x head groups workgroups, or the longest-first work map when the
  // batch fits its tables.
  const int P = positions_per_wg16(G, p.prefill_rb);
  const long long max_tiles = ((long long)max_len + P - 1) / P;
  const long long wgs = max_tiles * num_seqs * heads;
  if (wgs > kMaxGrid) return PKA_ERR_UNSUPPORTED;
  TileMap map;
  map.levels = 0;
  if (num_seqs <= kMapSeqs && max_tiles <= kMapLevels) {
    build_map(map, P);
    p.map = &map;
  }
  return status_of(launch_prefill_mfma(p, s));
}

size_t pka_verify_workspace_size(int32_t num_seqs, int32_t num_q_per_seq, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                 int32_t num_splits, int32_t dtype) {
  if (num_seqs <= 0 || num_q_per_seq < 1 || num_q_per_seq > kMaxVerifyRows) return 0;
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads) return 0;
  if (dtype != PKA_BF16 && dtype != PKA_F16 && dtype != PKA_FP8_E4M3) return 0;  // fp32: no partials
  if (head_dim != 64 && head_dim != 128) return 0;
  const DecodePlan plan = plan_decode(num_seqs, num_q_heads, num_kv_heads, max_kv_len, num_splits, num_q_per_seq);
  return decode_partials_bytes(num_seqs * num_q_per_seq, num_q_heads, head_dim, plan.splits);
}

size_t pka_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_kv_len, int32_t num_splits,
                                 int32_t dtype) {
  return pka_verify_workspace_size(num_seqs, 1, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits, dtype);
}

size_t pka_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_kv_len, int32_t dtype) {
  return pka_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_kv_len, 0, dtype);
}

}  // extern "C"

namespace {

// Fixed device scratch of pka_attn_decode_paged_noalloc: the split partials
// of its decode live here instead of in a caller workspace, so that call
// allocates nothing.  Each GPU holds its own copy until the process ends.  In
// host code `scratch` only names the symbol: its device address on the
// current GPU comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[PKA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call on that device, then cached).
int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PKA_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKA_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return PKA_ERR_LAUNCH;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return PKA_OK;
}

// Paged decode of nq query rows per sequence (1: decode; k + 1: speculative
// verify), row r of sequence s at q/out row s * nq + r.
int decode_rows(const void* q, void* out, const pka_kv_cache* cache, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs,
                int32_t nq, int32_t max_kv_len,
                int32_t num_q_heads, float scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                void* stream, bool use_scratch = false) {
  int st = check_cache(cache);
  if (st != PKA_OK) return st;
  if (num_seqs < 0 || num_splits < 0 || nq < 1 || nq > kMaxVerifyRows) return PKA_ERR_INVALID;
  const int hkv = cache->num_kv_heads;
  if (num_q_heads < 1 || num_q_heads % hkv != 0) return PKA_ERR_INVALID;
  if (num_seqs == 0) return PKA_OK;
  if (!q || !out || !block_tables || !kv_lens || !aligned16(q) || !aligned16(out)) return PKA_ERR_INVALID;
  if (max_blocks_per_seq < 1 || max_kv_len < nq || (long long)max_kv_len > (long long)max_blocks_per_seq * kBlock)
    return PKA_ERR_INVALID;
  const int d = cache->head_dim;
  const hipStream_t s = (hipStream_t)stream;
  if (cache->dtype == PKA_F32) {
    if (nq != 1) return PKA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_q_heads > 65535) return PKA_ERR_UNSUPPORTED;
    RowsProblem p = {};
    p.q = q;
    p.out = out;
    p.cu_q = nullptr;
    p.kv_lens = kv_lens;
    p.cache = view(cache);
    p.block_tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.hq = num_q_heads;
    p.hkv = hkv;
    p.d = d;
    p.dtype = PKA_F32;
    p.scale = resolve_scale(scale, d);
    p.paged = true;
    p.max_q_len = 1;
    return status_of(launch_rows_valu(p, s));
  }
  DecodeProblem p = {};
  p.nq = nq;
  // With host lengths the units go out longest sequence first (a scheduling
  // hint only: any order gives the same result).
  SeqOrder order;
  order.n = 0;
  if (kv_lens_host && num_seqs <= kMaxOrderSeqs) {
    int idx[kMaxOrderSeqs];
    for (int i = 0; i < num_seqs; ++i) idx[i] = i;
    std::stable_sort(idx, idx + num_seqs, [&](int x, int y) { return kv_lens_host[x] > kv_lens_host[y]; });
    for (int i = 0; i < num_seqs; ++i) order.seq[i] = (uint16_t)idx[i];
    order.n = num_seqs;
    p.order = &order;
  }
  p.plan = plan_decode(num_seqs, num_q_heads, hkv, max_kv_len, num_splits, nq,
                       order.n > 0 ? kLongestFirst : kIndexOrder);
  const long long wgs = (long long)num_seqs * hkv * p.plan.row_groups * p.plan.splits;
  if (wgs > kMaxGrid) return PKA_ERR_UNSUPPORTED;
  const size_t need = decode_partials_bytes(num_seqs * nq, num_q_heads, d, p.plan.splits);
  if (need > 0) {
    if (use_scratch) {  // the fixed device scratch instead of a caller workspace
      if (need > PKA_NOALLOC_SCRATCH_BYTES) return PKA_ERR_SCRATCH_LIMIT;
      const int sst = scratch_address(&workspace);
      if (sst != PKA_OK) return sst;
      workspace_bytes = PKA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKA_ERR_WORKSPACE;
    const size_t n = (size_t)num_seqs * nq * num_q_heads * p.plan.splits;
    p.part_o = static_cast<float*>(workspace);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(n * d * sizeof(float)));
  }
  p.q = q;
  p.out = out;
  p.cu_q = nullptr;
  p.kv_lens = kv_lens;
  p.block_tables = block_tables;
  p.max_blocks = max_blocks_per_seq;
  p.cache = view(cache);
  p.num_seqs = num_seqs;
  p.hq = num_q_heads;
  p.scale = resolve_scale(scale, d);
  hipError_t e = launch_decode_mfma(p, s);
  if (e != hipSuccess) return PKA_ERR_LAUNCH;
  return status_of(launch_decode_reduce(p, s));
}

}  // namespace

extern "C" {

int pka_attn_decode_paged_noalloc(const void* q, void* out, const pka_kv_cache* cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs,
                                  int32_t max_kv_len, int32_t num_q_heads, float scale, int32_t num_splits,
                                  void* stream) {
  // Arguments are checked and the plan made first; the scratch address is
  // looked up only when the plan has partials (and only if they fit).
  return decode_rows(q, out, cache, block_tables, max_blocks_per_seq, kv_lens, kv_lens_host, num_seqs, 1, max_kv_len,
                     num_q_heads, scale, num_splits, nullptr, 0, stream, /*use_scratch=*/true);
}

int pka_attn_decode_paged(const void* q, void* out, const pka_kv_cache* cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs, int32_t max_kv_len,
                          int32_t num_q_heads, float scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_rows(q, out, cache, block_tables, max_blocks_per_seq, kv_lens, kv_lens_host, num_seqs, 1, max_kv_len,
                     num_q_heads,
                     scale, num_splits, workspace, workspace_bytes, stream);
}

int pka_attn_verify_paged(const void* q, void* out, const pka_kv_cache* cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* kv_lens, const int32_t* kv_lens_host, int32_t num_seqs,
                          int32_t num_q_per_seq, int32_t max_kv_len,
                          int32_t num_q_heads, float scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_rows(q, out, cache, block_tables, max_blocks_per_seq, kv_lens, kv_lens_host, num_seqs, num_q_per_seq,
                     max_kv_len,
                     num_q_heads, scale, num_splits, workspace, workspace_bytes, stream);
}

int pka_attn_mixed_step(const void* q, void* out, const pka_kv_cache* cache,
                        const int32_t* cu_q_lens, const int32_t* cu_q_lens_host,
                        const int32_t* kv_lens, const int32_t* kv_lens_host,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t num_seqs, int32_t num_q_heads, float scale,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != PKA_OK) return st;
  if (num_seqs < 0) return PKA_ERR_INVALID;
  const int hkv = cache->num_kv_heads;
  if (num_q_heads < 1 || num_q_heads % hkv != 0) return PKA_ERR_INVALID;
  if (!cu_q_lens || !cu_q_lens_host || !kv_lens || !kv_lens_host || !block_tables) return PKA_ERR_INVALID;
  if (max_blocks_per_seq < 1) return PKA_ERR_INVALID;
  int max_q = 0;
  long long total = 0;
  st = scan_cu(cu_q_lens_host, num_seqs, &max_q, &total);
  if (st != PKA_OK) return st;
  const long long cap = (long long)max_blocks_per_seq * kBlock;
  const int G = num_q_heads / hkv;
  const int P = positions_per_wg(G);
  // Short multi-row sequences (speculative verify rows: a few query rows at
  // the end of a long context) run on two-column-group decode units, which
  // read each K/V block once for all q_len * G <= 32 columns of a kv head,
  // instead of on 32-row tiles that would leave most matrix rows idle.
  int short_max_q = cache->dtype == PKA_F32 ? 1 : std::min(kMaxVerifyRows, 32 / G);
  int n_short = 0, max_short_kv = 1, max_short_q = 1;
  if (short_max_q >= 2) {
    for (int i = 0; i < num_seqs; ++i) {
      const int ql = cu_q_lens_host[i + 1] - cu_q_lens_host[i];
      if (ql >= 2 && ql <= short_max_q) ++n_short;
    }
    if (n_short > kMaxOrderSeqs || num_seqs > 65536) n_short = 0;  // beyond the order table: tiles
  }
  if (n_short == 0) short_max_q = 1;
  long long tiles = 0;
  int n_dec = 0, max_dec_kv = 1, first_dec = -1, last_dec = -1;
  for (int i = 0; i < num_seqs; ++i) {
    const int ql = cu_q_lens_host[i + 1] - cu_q_lens_host[i];
    const int kv = kv_lens_host[i];
    if (kv < ql || (long long)kv > cap) return PKA_ERR_INVALID;
    if (ql == 1) {
      ++n_dec;
      if (kv > max_dec_kv) max_dec_kv = kv;
      if (first_dec < 0) first_dec = i;
      last_dec = i;
    } else if (ql > 1 && ql <= short_max_q) {
      if (kv > max_short_kv) max_short_kv = kv;
      if (ql > max_short_q) max_short_q = ql;
    } else if (ql > 1) {
      tiles += ((long long)ql + P - 1) / P;
    }
  }
  if (num_seqs == 0 || total == 0) return PKA_OK;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return PKA_ERR_INVALID;
  const int d = cache->head_dim;
  const hipStream_t s = (hipStream_t)stream;
  RowsProblem rp = {};
  rp.q = q;
  rp.out = out;
  rp.cu_q = cu_q_lens;
  rp.kv_lens = kv_lens;
  rp.cache = view(cache);
  rp.block_tables = block_tables;
  rp.max_blocks = max_blocks_per_seq;
  rp.num_seqs = num_seqs;
  rp.hq = num_q_heads;
  rp.hkv = hkv;
  rp.d = d;
  rp.dtype = act_dtype(cache);
  rp.scale = resolve_scale(scale, d);
  rp.paged = true;
  rp.max_q_len = max_q;
  if (cache->dtype == PKA_F32) {
    if (num_seqs > 65535 || num_q_heads > 65535) return PKA_ERR_UNSUPPORTED;
    return status_of(launch_rows_valu(rp, s));
  }
  rp.num_tiles = (int)tiles;
  rp.num_decode_seqs = n_dec;
  rp.max_decode_kv = max_dec_kv;
  rp.decode_base = (n_dec > 0 && last_dec - first_dec + 1 == n_dec) ? first_dec : -1;
  rp.short_max_q = short_max_q;
  DecodeProblem dp = {};
  // Decode rows longest first (see decode_rows): the k-th decode unit of a
  // split level takes sequence dorder.seq[k].
  SeqOrder dorder;
  dorder.n = 0;
  if (n_dec > 0 && n_dec <= kMaxOrderSeqs && num_seqs <= 65536) {
    int idx[kMaxOrderSeqs];
    int m = 0;
    for (int i = 0; i < num_seqs; ++i)
      if (cu_q_lens_host[i + 1] - cu_q_lens_host[i] == 1) idx[m++] = i;
    std::stable_sort(idx, idx + m, [&](int x, int y) { return kv_lens_host[x] > kv_lens_host[y]; });
    for (int i = 0; i < m; ++i) dorder.seq[i] = (uint16_t)idx[i];
    dorder.n = m;
    dp.order = &dorder;
  }
  dp.plan = plan_decode(num_seqs, num_q_heads, hkv, max_dec_kv, 0, 1,
                        dorder.n > 0 ? kLongestFirstMixed : kIndexOrder);
  const long long wgs = tiles * hkv * (G / heads_per_wg(G)) +
                        (long long)n_dec * hkv * dp.plan.row_groups * dp.plan.splits;
  if (wgs > kMaxGrid || (long long)n_short * hkv > kMaxGrid) return PKA_ERR_UNSUPPORTED;
  const size_t need = n_dec > 0 ? decode_partials_bytes(num_seqs, num_q_heads, d, dp.plan.splits) : 0;
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKA_ERR_WORKSPACE;
    const size_t n = (size_t)num_seqs * num_q_heads * dp.plan.splits;
    dp.part_o = static_cast<float*>(workspace);
    dp.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(n * d * sizeof(float)));
  }
  dp.q = q;
  dp.out = out;
  dp.cu_q = cu_q_lens;
  dp.kv_lens = kv_lens;
  dp.block_tables = block_tables;
  dp.max_blocks = max_blocks_per_seq;
  dp.cache = view(cache);
  dp.num_seqs = num_seqs;
  dp.hq = num_q_heads;
  dp.scale = rp.scale;
  if (n_dec == 0) dp.plan.splits = 1;  // no decode rows: nothing to merge
  hipError_t e = launch_mixed_mfma(rp, dp, s);
  if (e != hipSuccess || n_short == 0) return status_of(e);
  // The short multi-row sequences, longest context first, one unsplit unit
  // per (sequence, kv head) holding all its rows x grouped heads as columns.
  SeqOrder sorder;
  {
    int idx[kMaxOrderSeqs];
    int m = 0;
    for (int i = 0; i < num_seqs; ++i) {
      const int ql = cu_q_lens_host[i + 1] - cu_q_lens_host[i];
      if (ql >= 2 && ql <= short_max_q) idx[m++] = i;
    }
    std::stable_sort(idx, idx + m, [&](int x, int y) { return kv_lens_host[x] > kv_lens_host[y]; });
    for (int i = 0; i < m; ++i) sorder.seq[i] = (uint16_t)idx[i];
    sorder.n = m;
  }
  DecodeProblem sp = dp;
  sp.num_seqs = n_short;
  sp.nq = -1;  // rows per sequence from cu_q
  sp.plan.col_groups = max_short_q * G > 16 ? 2 : 1;
  sp.plan.row_groups = 1;
  sp.plan.splits = 1;
  sp.plan.chunk = (max_short_kv + kBlock - 1) / kBlock * kBlock;
  sp.part_o = nullptr;
  sp.part_ml = nullptr;
  sp.order = &sorder;
  return status_of(launch_decode_mfma(sp, s));
}

}  // extern "C"
