// Internal declarations shared by the HIP translation units of libpka.
// gfx950 (CDNA4) only: wave64, MFMA bf16 / fp16 with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pka {

constexpr int kBlock = 16;          // tokens per KV block
constexpr int kKeyTile = 32;        // keys per LDS tile of the prefill and tile units
constexpr int kThreads = 256;       // 4 waves per workgroup in every kernel

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;  // 16-byte chunk in registers
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// ---------------------------------------------------------------------------
// Split-context plan for paged decode rows.
//
// The keys of a decode row are cut into chunks of `chunk` tokens (a multiple
// of 16); sequence s uses ceil(kv_len_s / chunk) <= splits chunks.  One
// workgroup processes one (sequence, kv head, row group, chunk) unit.  The
// automatic rule (num_splits = 0) is in plan_decode; `splits` is monotone in
// max_kv_len, so a workspace sized for a larger max_kv_len is always large
// enough.
// ---------------------------------------------------------------------------
struct DecodePlan {
  int col_groups;  // 16-column MFMA groups per unit (2 only for multi-row verify above 16 columns)
  int row_groups;  // ceil(G / 16): MFMA row tiles of 16 query heads per kv head
  int splits;      // upper bound of chunks per sequence (partials dimension)
  int chunk;       // tokens per chunk
};

// nq query rows per sequence (speculative verify) make nq * G MFMA columns
// per kv head; above 16 columns a unit carries two 16-column groups, so each
// K/V block is read once for up to 32 columns.
// Dispatch order of the decode units, which the automatic plan depends on.
enum DecodeSchedule {
  kIndexOrder = 0,      // sequences in index order (no host lengths)
  kLongestFirst = 1,    // longest sequence first (decode, verify)
  kLongestFirstMixed = 2  // longest first, sharing the launch with prefill-chunk tiles
};

inline DecodePlan plan_decode(int num_seqs, int hq, int hkv, int max_kv_len, int num_splits, int nq = 1,
                              DecodeSchedule sched = kIndexOrder) {
  DecodePlan p;
  const int g = hq / hkv;
  p.col_groups = (nq > 1 && nq * g > 16) ? 2 : 1;
  p.row_groups = (nq * g + 16 * p.col_groups - 1) / (16 * p.col_groups);
  const long long units = (long long)num_seqs * hkv * p.row_groups;
  const int kv = max_kv_len < 1 ? 1 : max_kv_len;
  int s;
  if (num_splits >= 1) {
    const int cap = (kv + kBlock - 1) / kBlock;
    s = num_splits < cap ? num_splits : cap;
  } else {
    // Enough units to keep the 768 resident workgroup slots of the chip busy
    // through the last round (about 1024), and, while there are fewer than
    // 4096 (sequence, kv head) units, up to 4 chunks of at least 512 tokens so
    // that ragged batches end in short units.  Chunks never drop below 64
    // tokens.  Measured on gfx950: 64 x MHA 32/32 decode at kv U{128..2048}
    // is fastest at 4 splits, 128 x GQA 32/8 at 3-4, 16 x GQA 64/8 at 32768
    // keys at 8.
    // Multi-row verify units carry up to 32 query columns (more partial
    // traffic per split) at two workgroups per CU: about one unit per resident
    // slot (512) and no granularity splits.  Measured on 64 x 5 rows, GQA
    // 32/8, kv U{128..2048}: 1 split 70.5 us, 2: 76.1, 4: 79.5, 8: 92.2.
    // Dispatched longest sequence first, the launch already ends on the
    // shortest units: about one unit per resident slot (512) and no
    // granularity splits.  Measured: 64 x MHA 181.6 us at 1 split against
    // 185-195 at 2-4; 128 x GQA 32/8 102.9 against 110-118; 16 x GQA 64/8 at
    // 32768 keys 321 us at 4 against 327-341 at 8-16.  Beside prefill-chunk
    // tiles (the mixed step), which hold slots for long stretches, up to 2
    // chunks of at least 1024 tokens: 128 decodes + 2 x 1024-row chunks 154 us
    // against 165 at one split and 167 in index order.
    const bool sorted = sched != kIndexOrder;
    const long long slots = (nq > 1 || sched == kLongestFirst) ? 512 : 1024;
    const long long balance = units > 0 ? (slots + units - 1) / units : 1;
    const int gran_tokens = sorted ? 1024 : 512, gran_max = sched == kLongestFirst ? 1 : (sorted ? 2 : 4);
    const long long gran_n = (kv + gran_tokens - 1) / gran_tokens;
    const long long gran = (nq == 1 && units < 4096) ? (gran_n < gran_max ? gran_n : gran_max) : 1;
    const long long target = balance > gran ? balance : gran;
    const int cap = (kv + 63) / 64;
    s = (int)(target < cap ? target : cap);
  }
  if (s < 1) s = 1;
  int chunk = (kv + s - 1) / s;
  chunk = (chunk + kBlock - 1) / kBlock * kBlock;
  p.chunk = chunk;
  p.splits = s;
  return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: partial outputs [B][Hq][S][D] fp32, then (m, l) pairs [B][Hq][S].
inline size_t decode_partials_bytes(int num_seqs, int hq, int d, int splits) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)num_seqs * hq * splits;
  return align256(n * d * sizeof(float)) + align256(n * 2 * sizeof(float));
}

// ---------------------------------------------------------------------------
// Kernel launchers (defined next to their kernels).  They assume validated
// arguments and return the HIP error of the launch.
// ---------------------------------------------------------------------------
struct CacheView {
  void* k_pool;
  void* v_pool;
  int num_blocks;
  int hkv;
  int d;
  int dtype;      // pool elements: 0 f32, 1 bf16, 2 f16, 3 fp8 e4m3
  int act_dtype;  // q, new k/v and outputs: dtype, or 1 / 2 for fp8 pools
  const float* k_scale;  // fp8 pools: [hkv]
  const float* v_scale;
};

hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         const int32_t* slots, int num_tokens, hipStream_t stream);
hipError_t launch_copy_blocks(const CacheView& src, const CacheView& dst, const int32_t* pairs, int num_pairs,
                              hipStream_t stream);

// Append with rotary position embedding: the caller fills the token-side
// fields and theta; the launcher fills the pool fields from the cache.
constexpr int kMaxRopePairs = 64;  // d / 2 for d <= 128
struct RopeArgs {
  const void* q;            // [T][hq][d] or nullptr (no q rows)
  void* q_out;              // may equal q
  const void* k_new;        // [T][hkv][d]
  const void* v_new;
  void* kpool;
  void* vpool;
  const int32_t* slots;     // [T]
  const int32_t* positions; // [T]
  const float* k_scale;     // fp8 pools
  const float* v_scale;
  long long num_slots;
  int hq;
  int hkv;
  double theta[kMaxRopePairs];  // base^(-2j/d), j < d/2
};
hipError_t launch_append_rope(const CacheView& c, RopeArgs a, int num_tokens, bool interleaved,
                              hipStream_t stream);

// Longest-first work map of a prefill launch, built on the host from
// cu_seqlens_host and passed by value in the kernel arguments.  Sequences are
// ranked by tile count (most first, ties by index); level l holds the l-th
// tile from the end of every sequence with more than l tiles, i.e. ranks
// 0 .. count_l - 1, each with `heads` workgroups (kv heads x head groups).
// Workgroup ids level_start[l] .. level_start[l+1] - 1 are level l, so the
// grid has exactly one workgroup per (sequence, tile, head group) and the
// tiles with the most keys start first.  Each rank's first row and length
// travel with the map, so a workgroup starts its Q and K/V loads without
// reading cu_seqlens first.  levels == 0: no map (batches beyond the table
// sizes use the plain level grid, whose ids past a sequence's tile count exit
// at once).
constexpr int kMapSeqs = 256;
constexpr int kMapLevels = 128;
struct TileMap {
  int levels;
  int heads;
  int level_start[kMapLevels + 1];
  int row0_of_rank[kMapSeqs];   // first packed row of the rank's sequence
  int q_len_of_rank[kMapSeqs];  // its length
};

// Attention over query rows packed by cu_q (device).  kv source is either
// the contiguous packed k/v (prefill: keys = the rows of the same sequence)
// or the paged cache.
struct RowsProblem {
  const void* q;
  void* out;
  const int32_t* cu_q;       // device [B+1]
  const int32_t* kv_lens;    // device [B] (paged) or nullptr (prefill: kv_len = q_len)
  const void* k;             // prefill only: packed [T][Hkv][D]
  const void* v;
  CacheView cache;           // paged only
  const int32_t* block_tables;
  int max_blocks;
  int num_seqs;
  int hq;
  int hkv;
  int d;
  int dtype;
  float scale;
  bool paged;
  int max_q_len;             // host-known, sizes some launches
  const TileMap* map;        // host: prefill work map, or nullptr
  int num_tiles;             // host-known: sum over tile-type sequences of tiles
  int num_decode_seqs;       // host-known: sequences routed to the decode path
  int max_decode_kv;         // host-known: largest kv_len of decode-path rows
  int decode_base;           // host-known: first decode sequence if the decode
                             // sequences are contiguous, else -1
  int prefill_rb;            // prefill: 16-row blocks per wave of the prefill unit (2 or 3)
  int short_max_q;           // mixed step: sequences with 2..short_max_q rows run
                             // on decode units in a launch of their own (1: none)
};

// Packed prefill on the 16-row-block unit (work map p.map, or the level grid).
hipError_t launch_prefill_mfma(const RowsProblem& p, hipStream_t stream);
hipError_t launch_rows_valu(const RowsProblem& p, hipStream_t stream);  // fp32 only

// Dispatch order of the decode units' sequences: rank r (longest first)
// processes sequence seq[r]; n == 0 keeps the sequences in index order.
constexpr int kMaxOrderSeqs = 1024;
struct SeqOrder {
  int n;
  uint16_t seq[kMaxOrderSeqs];
};

struct DecodeProblem {
  const void* q;
  void* out;
  const int32_t* cu_q;       // nullptr: row of sequence s is s
  const int32_t* kv_lens;
  const int32_t* block_tables;
  int max_blocks;
  CacheView cache;
  int num_seqs;
  int hq;
  float scale;
  DecodePlan plan;
  int nq;                    // query rows per sequence (0 or 1: one; -1: from cu_q, per sequence)
  float* part_o;
  float* part_ml;
  const SeqOrder* order;     // nullptr: index order
};

hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeProblem& p, hipStream_t stream);
hipError_t launch_mixed_mfma(const RowsProblem& rp, const DecodeProblem& dp, hipStream_t stream);

// Tiles of the MFMA prefill/chunk path: 32 query rows per wave, 4 waves per
// workgroup; heads_per_wg query heads of one kv head share each K/V tile.
inline int heads_per_wg(int g) { return (g % 4 == 0) ? 4 : ((g % 2 == 0) ? 2 : 1); }
inline int positions_per_wg(int g) { return 32 * 4 / heads_per_wg(g); }
// The 16-row-block prefill unit: 16 rb rows per wave (rb = 2 or 3), 4 waves.
inline int positions_per_wg16(int g, int rb) { return 16 * rb * 4 / heads_per_wg(g); }

}  // namespace pka
