// Slot-mapped append of new keys/values into the paged KV pools.
//
// Each wave copies 16 consecutive new tokens of one kv head.  Lane l owns
// token (l % 16) of the group and 16-byte dim groups (l / 16) + 4k.  K is
// stored in 16-byte dim groups with the 16 tokens of a block adjacent
// (layout in include/pka.h), so when the 16 tokens fill one block a wave
// store instruction writes 4 contiguous 256-byte runs.  V is stored
// dim-major inside a tile, so the lane scatters its 16 bytes element by
// element; lanes 0..15 then write the 16 consecutive token slots of one dim
// (32 contiguous bytes for bf16) and the L2 merges the partial lines before
// they reach HBM.
#include "pka_internal.h"

namespace pka {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(
    T* __restrict__ kpool, T* __restrict__ vpool, const T* __restrict__ k_new,
    const T* __restrict__ v_new, const int32_t* __restrict__ slots, int num_tokens, int hkv,
    long long num_slots) {
  constexpr int X = 16 / sizeof(T);  // elements per 16-byte group
  constexpr int NG = D / X;          // 16-byte groups per row
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const long long groups = (num_tokens + 15) / 16;
  if (wave >= groups * hkv) return;
  const int g = (int)(wave % hkv);
  const long long tok = (wave / hkv) * 16 + (lane & 15);
  if (tok >= num_tokens) return;
  const long long slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const long long blk = slot >> 4;
  const int off = (int)(slot & 15);
  const T* ks = k_new + (tok * hkv + g) * D;
  const T* vs = v_new + (tok * hkv + g) * D;
  T* kt = kpool + (blk * hkv + g) * (long long)(kBlock * D);
  T* vt = vpool + (blk * hkv + g) * (long long)(kBlock * D);
#pragma unroll
  for (int j = lane >> 4; j < NG; j += 4) {
    const uint4 kv = *reinterpret_cast<const uint4*>(ks + j * X);
    *reinterpret_cast<uint4*>(kt + (j * kBlock + off) * X) = kv;
    const uint4 vv = *reinterpret_cast<const uint4*>(vs + j * X);
    const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int e = 0; e < X; ++e) vt[(j * X + e) * kBlock + off] = ve[e];
  }
}

template <typename T, int D>
hipError_t launch_t(const CacheView& c, const void* k_new, const void* v_new, const int32_t* slots,
                    int num_tokens, hipStream_t stream) {
  const long long waves = (long long)((num_tokens + 15) / 16) * c.hkv;
  const long long blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((append_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<T*>(c.k_pool), static_cast<T*>(c.v_pool),
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), slots, num_tokens,
                     c.hkv, (long long)c.num_blocks * kBlock);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         const int32_t* slots, int num_tokens, hipStream_t stream) {
  if (c.dtype == 1) {
    return c.d == 128 ? launch_t<uint16_t, 128>(c, k_new, v_new, slots, num_tokens, stream)
                      : launch_t<uint16_t, 64>(c, k_new, v_new, slots, num_tokens, stream);
  }
  return c.d == 128 ? launch_t<uint32_t, 128>(c, k_new, v_new, slots, num_tokens, stream)
                    : launch_t<uint32_t, 64>(c, k_new, v_new, slots, num_tokens, stream);
}

}  // namespace pka
