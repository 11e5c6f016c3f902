// Host block manager: block tables, lengths and slot mappings for the
// attention calls.  A LIFO free list of pool blocks; sequence s of length n
// holds ceil(n / 16) blocks and its token at position p sits in slot
// table[p / 16] * 16 + p % 16.  The pages place a block allocator beside the
// router's queue and scheduler (TGI architecture page, "The Router") and free
// what a finished query holds (TGI router deep-dive, simple continuous
// batching); the LIFO policy is this library's reading.  Host memory only.
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/pka.h"

struct pka_block_manager {
  int32_t num_blocks;
  int32_t max_seqs;
  int32_t max_blocks;            // block-table row width
  std::vector<int32_t> free;     // stack: back() is handed out next
  std::vector<int32_t> len;      // [max_seqs] tokens
  std::vector<int32_t> table;    // [max_seqs][max_blocks], -1 past a sequence's blocks
  std::vector<int32_t> held;     // [max_seqs] blocks held
};

namespace {

constexpr int32_t kBlockTokens = 16;

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + kBlockTokens - 1) / kBlockTokens); }

}  // namespace

extern "C" {

pka_block_manager* pka_bm_create(int32_t num_blocks, int32_t max_seqs, int32_t max_blocks_per_seq) {
  if (num_blocks < 1 || max_seqs < 1 || max_blocks_per_seq < 1) return nullptr;
  // Slots (block * 16 + offset) and sequence lengths are int32.
  if (num_blocks > INT32_MAX / kBlockTokens || max_blocks_per_seq > INT32_MAX / kBlockTokens) return nullptr;
  if ((int64_t)max_seqs * max_blocks_per_seq > (int64_t)1 << 31) return nullptr;
  pka_block_manager* bm = new (std::nothrow) pka_block_manager;
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->max_seqs = max_seqs;
    bm->max_blocks = max_blocks_per_seq;
    bm->free.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free[i] = num_blocks - 1 - i;  // block 0 on top
    bm->len.assign(max_seqs, 0);
    bm->held.assign(max_seqs, 0);
    bm->table.assign((size_t)max_seqs * max_blocks_per_seq, -1);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pka_bm_destroy(pka_block_manager* bm) { delete bm; }

int pka_bm_append(pka_block_manager* bm, const int32_t* seqs, const int32_t* num_new, int32_t n,
                  int32_t* slots_out) {
  if (!bm || n < 0) return PKA_ERR_INVALID;
  if (n == 0) return PKA_OK;
  if (!seqs || !num_new || !slots_out) return PKA_ERR_INVALID;
  // Validate the whole step and count the blocks it needs before changing anything.
  std::vector<char> seen;
  try {
    seen.assign(bm->max_seqs, 0);
  } catch (...) {
    return PKA_ERR_INVALID;
  }
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    if (s < 0 || s >= bm->max_seqs || seen[s] || num_new[i] < 0) return PKA_ERR_INVALID;
    seen[s] = 1;
    const int64_t grown = (int64_t)bm->len[s] + num_new[i];
    if (grown > (int64_t)bm->max_blocks * kBlockTokens) return PKA_ERR_INVALID;
    need += blocks_for(grown) - bm->held[s];
  }
  if (need > (int64_t)bm->free.size()) return PKA_ERR_NO_BLOCKS;
  int64_t out = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    int32_t* row = &bm->table[(size_t)s * bm->max_blocks];
    const int32_t p0 = bm->len[s], p1 = p0 + num_new[i];
    for (int32_t want = blocks_for(p1); bm->held[s] < want; ++bm->held[s]) {
      row[bm->held[s]] = bm->free.back();
      bm->free.pop_back();
    }
    for (int32_t p = p0; p < p1; ++p) slots_out[out++] = row[p / kBlockTokens] * kBlockTokens + p % kBlockTokens;
    bm->len[s] = p1;
  }
  return PKA_OK;
}

int pka_bm_release(pka_block_manager* bm, int32_t seq, int32_t* freed_out, int32_t* num_freed) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return PKA_ERR_INVALID;
  int32_t* row = &bm->table[(size_t)seq * bm->max_blocks];
  const int32_t h = bm->held[seq];
  for (int32_t j = 0; j < h; ++j) {  // the free list has room: every block is either held or free
    if (freed_out) freed_out[j] = row[j];
    bm->free.push_back(row[j]);
    row[j] = -1;
  }
  if (num_freed) *num_freed = h;
  bm->held[seq] = 0;
  bm->len[seq] = 0;
  return PKA_OK;
}

int pka_bm_tables(const pka_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* tables_out,
                  int32_t* kv_lens_out) {
  if (!bm || n < 0) return PKA_ERR_INVALID;
  if (n == 0) return PKA_OK;
  if (!seqs || !tables_out) return PKA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (seqs[i] < 0 || seqs[i] >= bm->max_seqs) return PKA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* row = &bm->table[(size_t)seqs[i] * bm->max_blocks];
    for (int32_t j = 0; j < bm->max_blocks; ++j) tables_out[(size_t)i * bm->max_blocks + j] = row[j];
    if (kv_lens_out) kv_lens_out[i] = bm->len[seqs[i]];
  }
  return PKA_OK;
}

int32_t pka_bm_free_blocks(const pka_block_manager* bm) { return bm ? (int32_t)bm->free.size() : -1; }

int32_t pka_bm_seq_len(const pka_block_manager* bm, int32_t seq) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return -1;
  return bm->len[seq];
}

}  // extern "C"
