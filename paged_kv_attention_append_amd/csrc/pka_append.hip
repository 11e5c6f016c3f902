// Slot-mapped append of new keys/values into the paged KV pools.
//
// The pools are token-major ([block][kv head][16][d]), so a token's row of one
// head is head_dim contiguous elements both in the input ([T][Hkv][d]) and in
// its pool slot.  One thread moves one 16-byte chunk of K and the same chunk
// of V; consecutive threads take consecutive chunks of a row, then the next
// head, then the next token, so every wave reads and writes whole 256-byte
// rows (bf16, d = 128) with 16-byte accesses.
#include "pka_internal.h"

namespace pka {
namespace {

template <int CPR>  // 16-byte chunks per row: head_dim * element_bytes / 16
__global__ __launch_bounds__(kThreads) void append_kernel(
    uint4* __restrict__ kpool, uint4* __restrict__ vpool, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int32_t* __restrict__ slots, long long num_chunks, int hkv,
    long long num_slots) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_chunks) return;
  const int c = (int)(i % CPR);
  const long long row = i / CPR;  // (token, head) row of the input
  const int g = (int)(row % hkv);
  const long long tok = row / hkv;
  const long long slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const long long dst = (((slot >> 4) * hkv + g) * kBlock + (slot & 15)) * CPR + c;
  const uint4 kv = k_new[i];
  const uint4 vv = v_new[i];
  kpool[dst] = kv;
  vpool[dst] = vv;
}

template <int CPR>
hipError_t launch_t(const CacheView& c, const void* k_new, const void* v_new, const int32_t* slots,
                    int num_tokens, hipStream_t stream) {
  const long long chunks = (long long)num_tokens * c.hkv * CPR;
  const long long blocks = (chunks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((append_kernel<CPR>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<uint4*>(c.k_pool), static_cast<uint4*>(c.v_pool),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), slots, chunks, c.hkv,
                     (long long)c.num_blocks * kBlock);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         const int32_t* slots, int num_tokens, hipStream_t stream) {
  const int row_bytes = c.d * (c.dtype == 1 ? 2 : 4);
  switch (row_bytes / 16) {
    case 8: return launch_t<8>(c, k_new, v_new, slots, num_tokens, stream);
    case 16: return launch_t<16>(c, k_new, v_new, slots, num_tokens, stream);
    default: return launch_t<32>(c, k_new, v_new, slots, num_tokens, stream);
  }
}

}  // namespace pka
