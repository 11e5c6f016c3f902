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

// fp8 (OCP E4M3) code of x / scale: the fp32 quotient (IEEE division) rounded
// to the nearest code, ties to the even code, magnitudes from 448 up
// saturating to 448 (code 0x7E).  Inputs are finite.
__device__ __forceinline__ unsigned e4m3_code(float x, float scale) {
  const float q = x / scale;
  const unsigned b = __builtin_bit_cast(unsigned, q);
  const unsigned sign = (b >> 31) << 7;
  const unsigned a = b & 0x7fffffffu;
  unsigned code;
  if (a >= 0x43e00000u) {                 // |q| >= 448
    code = 0x7e;
  } else if (a < 0x3c800000u) {           // |q| < 2^-6: subnormal codes m * 2^-9, m = 0..8
    code = (unsigned)__builtin_rintf(__builtin_bit_cast(float, a) * 512.f);  // rint: ties to even m
  } else {                                // normal: keep 3 mantissa bits, nearest-even on the rest
    const unsigned r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // (fp32 exponent << 3) | mantissa, carried
    code = r - ((127u - 7u) << 3);        // rebias the exponent from 127 to 7
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

// Widen 16-bit elements (the low or high half of a word) to fp32.
template <bool F16>
__device__ __forceinline__ float widen(unsigned w, int hi) {
  const unsigned h = hi ? (w >> 16) : (w & 0xffffu);
  if (F16) return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
  return __builtin_bit_cast(float, h << 16);
}

// fp8 pools: one thread quantizes 16 consecutive elements (32 input bytes,
// 16 pool bytes) of one (token, head) row of K and of V.
template <bool F16>
__global__ __launch_bounds__(kThreads) void append_fp8_kernel(
    u32x4* __restrict__ kpool, u32x4* __restrict__ vpool, const u32x4* __restrict__ k_new,
    const u32x4* __restrict__ v_new, const int32_t* __restrict__ slots, long long num_chunks, int hkv,
    long long num_slots, int cpr, const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_chunks) return;
  const int c = (int)(i % cpr);
  const long long row = i / cpr;  // (token, head) row of the input
  const int g = (int)(row % hkv);
  const long long tok = row / hkv;
  const long long slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const long long dst = (((slot >> 4) * hkv + g) * kBlock + (slot & 15)) * cpr + c;
  const float ks = k_scale[g], vs = v_scale[g];
  const u32x4 k0 = k_new[2 * i], k1 = k_new[2 * i + 1];
  const u32x4 v0 = v_new[2 * i], v1 = v_new[2 * i + 1];
  u32x4 ko, vo;
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {  // output word wd holds elements 4 wd .. 4 wd + 3
    const unsigned ka = wd < 2 ? k0[2 * wd] : k1[2 * wd - 4], kb = wd < 2 ? k0[2 * wd + 1] : k1[2 * wd - 3];
    const unsigned va = wd < 2 ? v0[2 * wd] : v1[2 * wd - 4], vb = wd < 2 ? v0[2 * wd + 1] : v1[2 * wd - 3];
    ko[wd] = e4m3_code(widen<F16>(ka, 0), ks) | (e4m3_code(widen<F16>(ka, 1), ks) << 8) |
             (e4m3_code(widen<F16>(kb, 0), ks) << 16) | (e4m3_code(widen<F16>(kb, 1), ks) << 24);
    vo[wd] = e4m3_code(widen<F16>(va, 0), vs) | (e4m3_code(widen<F16>(va, 1), vs) << 8) |
             (e4m3_code(widen<F16>(vb, 0), vs) << 16) | (e4m3_code(widen<F16>(vb, 1), vs) << 24);
  }
  kpool[dst] = ko;
  vpool[dst] = vo;
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
  const int es = src.dtype == 0 ? 4 : (src.dtype == 3 ? 1 : 2);
  const int chunks = src.hkv * kBlock * src.d * es / 16;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(2LL * num_pairs)), dim3(kThreads), 0, stream,
                     static_cast<u32x4*>(dst.k_pool), static_cast<u32x4*>(dst.v_pool),
                     static_cast<const u32x4*>(src.k_pool), static_cast<const u32x4*>(src.v_pool), pairs, chunks,
                     src.num_blocks, dst.num_blocks);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         const int32_t* slots, int num_tokens, hipStream_t stream) {
  if (c.dtype == 3) {
    const int cpr = c.d / 16;
    const long long chunks = (long long)num_tokens * c.hkv * cpr;
    const long long blocks = (chunks + kThreads - 1) / kThreads;
    if (c.act_dtype == 2)
      hipLaunchKernelGGL((append_fp8_kernel<true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                         static_cast<u32x4*>(c.k_pool), static_cast<u32x4*>(c.v_pool),
                         static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new), slots, chunks, c.hkv,
                         (long long)c.num_blocks * kBlock, cpr, c.k_scale, c.v_scale);
    else
      hipLaunchKernelGGL((append_fp8_kernel<false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                         static_cast<u32x4*>(c.k_pool), static_cast<u32x4*>(c.v_pool),
                         static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new), slots, chunks, c.hkv,
                         (long long)c.num_blocks * kBlock, cpr, c.k_scale, c.v_scale);
    return hipGetLastError();
  }
  const int row_bytes = c.d * (c.dtype == 0 ? 4 : 2);
  switch (row_bytes / 16) {
    case 8: return launch_t<8>(c, k_new, v_new, slots, num_tokens, stream);
    case 16: return launch_t<16>(c, k_new, v_new, slots, num_tokens, stream);
    default: return launch_t<32>(c, k_new, v_new, slots, num_tokens, stream);
  }
}

}  // namespace pka
