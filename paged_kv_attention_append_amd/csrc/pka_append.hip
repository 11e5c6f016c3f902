// Writes into the paged KV pools: the slot-mapped append of new keys/values,
// and whole-block copies between pools (copy-on-write, swap out / swap in).
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

// Block copy.  In the pool layout one block of one pool (all kv heads, all
// 16 slots) is `chunks` contiguous 16-byte chunks, so workgroup w copies block
// pairs[w / 2] of pool w % 2 (K, V) as one contiguous run: every wave moves
// whole 1 KiB spans with 16-byte non-temporal accesses (the data is not read
// again by this launch; the destination may be host memory).
__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ kdst, u32x4* __restrict__ vdst,
                                                        const u32x4* __restrict__ ksrc, const u32x4* __restrict__ vsrc,
                                                        const int32_t* __restrict__ pairs, int chunks, int src_blocks,
                                                        int dst_blocks) {
  const long long pair = blockIdx.x >> 1;
  const int pool = blockIdx.x & 1;
  const int sb = pairs[2 * pair], db = pairs[2 * pair + 1];
  if (sb < 0 || sb >= src_blocks || db < 0 || db >= dst_blocks) return;
  const u32x4* src = (pool ? vsrc : ksrc) + (long long)sb * chunks;
  u32x4* dst = (pool ? vdst : kdst) + (long long)db * chunks;
  constexpr int U = 4;  // independent loads in flight per thread
  int c = threadIdx.x;
  for (; c + (U - 1) * kThreads < chunks; c += U * kThreads) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + c + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], dst + c + u * kThreads);
  }
  for (; c < chunks; c += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + c), dst + c);
}

}  // namespace

hipError_t launch_copy_blocks(const CacheView& src, const CacheView& dst, const int32_t* pairs, int num_pairs,
                              hipStream_t stream) {
  const int es = src.dtype == 0 ? 4 : 2;
  const int chunks = src.hkv * kBlock * src.d * es / 16;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(2LL * num_pairs)), dim3(kThreads), 0, stream,
                     static_cast<u32x4*>(dst.k_pool), static_cast<u32x4*>(dst.v_pool),
                     static_cast<const u32x4*>(src.k_pool), static_cast<const u32x4*>(src.v_pool), pairs, chunks,
                     src.num_blocks, dst.num_blocks);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         const int32_t* slots, int num_tokens, hipStream_t stream) {
  const int row_bytes = c.d * (c.dtype == 0 ? 4 : 2);
  switch (row_bytes / 16) {
    case 8: return launch_t<8>(c, k_new, v_new, slots, num_tokens, stream);
    case 16: return launch_t<16>(c, k_new, v_new, slots, num_tokens, stream);
    default: return launch_t<32>(c, k_new, v_new, slots, num_tokens, stream);
  }
}

}  // namespace pka
