// Writes into the paged KV pools: the slot-mapped append of new keys/values
// (plain, quantizing to fp8 E4M3, or with the rotary position embedding), and
// whole-block copies between pools (copy-on-write, swap out / swap in).
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
// whole 1 KiB spans with 16-byte accesses, eight loads in flight per thread
// (a whole 32 KiB block of a GQA-8, d = 128 bf16 pool in one round).  The
// source is read once (non-temporal loads); the stores are ordinary: with
// non-temporal stores the device-to-device copy ran at 5.1 instead of 6.3
// TB/s, and swaps to or from pinned host memory, bound by the host link, are
// the same either way.
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
  constexpr int U = 8;  // independent loads in flight per thread
  int c = threadIdx.x;
  for (; c + (U - 1) * kThreads < chunks; c += U * kThreads) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + c + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) dst[c + u * kThreads] = x[u];
  }
  for (; c < chunks; c += kThreads) dst[c] = __builtin_nontemporal_load(src + c);
}

// ---------------------------------------------------------------------------
// Append with rotary position embedding (RoPE).
//
// Pair j of a head's dims -- (j, j + d/2) in the half pairing, (2j, 2j + 1)
// in the interleaved one -- is rotated by phi = pos * theta_j, theta_j =
// base^(-2j/d): (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
// One workgroup per token.  Its first d/2 threads evaluate cos and sin of the
// token's angles in fp64 (the angle reaches 3e4 rad at long positions, so
// it must not be rounded to fp32 first) and share them through LDS; every
// thread then rotates 8-pair items of the token's K rows (written to the
// pool slot) and q rows (written to q_out) in fp32, and copies 16-element
// chunks of its V rows.  The rotated value is within 2^-22 (|a| + |b|) of
// the exact one before the final rounding to the output type.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

template <int ACT>  // 0 fp32, 1 bf16, 2 fp16: 8 consecutive elements <-> fp32
struct Act;
template <>
struct Act<0> {  // whole-vector loads and stores (element-wise bit casts into vectors miscompile)
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ void load8(const void* p, long long off, float* x) {
    const f32x4* s = reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + off);
    const f32x4 a = s[0], b = s[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
  static __device__ __forceinline__ void store8(void* p, long long off, const float* x) {
    f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(p) + off);
    d[0] = f32x4{x[0], x[1], x[2], x[3]};
    d[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
};
template <>
struct Act<1> {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ void load8(const void* p, long long off, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store8(void* p, long long off, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];  // nearest-even
    *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(p) + off) = v;
  }
};
template <>
struct Act<2> {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ void load8(const void* p, long long off, float* x) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(static_cast<const uint16_t*>(p) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  }
  static __device__ __forceinline__ void store8(void* p, long long off, const float* x) {
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)x[e];  // nearest-even
    *reinterpret_cast<f16x8*>(static_cast<uint16_t*>(p) + off) = v;
  }
};

__device__ __forceinline__ u32x2 e4m3_codes8(const float* x, float scale) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w)
    r[w] = e4m3_code(x[4 * w], scale) | (e4m3_code(x[4 * w + 1], scale) << 8) |
           (e4m3_code(x[4 * w + 2], scale) << 16) | (e4m3_code(x[4 * w + 3], scale) << 24);
  return r;
}

template <int D, int ACT, bool FP8, bool INTERLEAVED>
__global__ __launch_bounds__(kThreads) void append_rope_kernel(RopeArgs a) {
  using A = Act<ACT>;
  constexpr int G16 = D / 16;  // 16-element items per head row (8 rotation pairs each)
  __shared__ float cs[2][D / 2];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < D / 2) {
    double sn, cn;
    sincos((double)a.positions[t] * a.theta[tid], &sn, &cn);
    cs[0][tid] = (float)cn;
    cs[1][tid] = (float)sn;
  }
  const long long slot = a.slots[t];
  const bool write_kv = slot >= 0 && slot < a.num_slots;
  // Pool row (in elements / D) of this token's head 0: ((block * Hkv + g) * 16 + offset), g = 0.
  const long long prow0 = (slot >> 4) * a.hkv * kBlock + (slot & 15);
  __syncthreads();
  const int nk = a.hkv * G16, nq = a.q ? a.hq * G16 : 0;
  for (int it = tid; it < 2 * nk + nq; it += kThreads) {
    if (it < nk + nq) {  // rotate 8 pairs of a K row (it < nk) or a q row
      const bool isk = it < nk;
      if (isk && !write_kv) continue;
      const int r = isk ? it : it - nk;
      const int h = r / G16, g = r % G16;
      const long long row = ((long long)t * (isk ? a.hkv : a.hq) + h) * D;
      const int o_lo = INTERLEAVED ? 16 * g : 8 * g;          // the item's two 8-element runs
      const int o_hi = INTERLEAVED ? 16 * g + 8 : D / 2 + 8 * g;
      float lo[8], hi[8];
      A::load8(isk ? a.k_new : a.q, row + o_lo, lo);
      A::load8(isk ? a.k_new : a.q, row + o_hi, hi);
      float y_lo[8], y_hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // pair j = 8 g + e
        const float c = cs[0][8 * g + e], sn = cs[1][8 * g + e];
        float xa, xb;
        if (INTERLEAVED) {
          xa = e < 4 ? lo[2 * e] : hi[2 * e - 8];
          xb = e < 4 ? lo[2 * e + 1] : hi[2 * e - 7];
        } else {
          xa = lo[e];
          xb = hi[e];
        }
        const float ya = fmaf(xa, c, -(xb * sn)), yb = fmaf(xa, sn, xb * c);
        if (INTERLEAVED) {
          if (e < 4) {
            y_lo[2 * e] = ya;
            y_lo[2 * e + 1] = yb;
          } else {
            y_hi[2 * e - 8] = ya;
            y_hi[2 * e - 7] = yb;
          }
        } else {
          y_lo[e] = ya;
          y_hi[e] = yb;
        }
      }
      if (!isk) {
        A::store8(a.q_out, row + o_lo, y_lo);
        A::store8(a.q_out, row + o_hi, y_hi);
      } else {
        const long long prow = (prow0 + (long long)h * kBlock) * D;
        if constexpr (FP8) {
          const float ks = a.k_scale[h];
          unsigned char* kp = static_cast<unsigned char*>(a.kpool) + prow;
          *reinterpret_cast<u32x2*>(kp + o_lo) = e4m3_codes8(y_lo, ks);
          *reinterpret_cast<u32x2*>(kp + o_hi) = e4m3_codes8(y_hi, ks);
        } else {
          A::store8(a.kpool, prow + o_lo, y_lo);
          A::store8(a.kpool, prow + o_hi, y_hi);
        }
      }
    } else {  // V: 16 consecutive elements of a row, unrotated
      if (!write_kv) continue;
      const int r = it - nk - nq;
      const int h = r / G16, g = r % G16;
      const long long src = ((long long)t * a.hkv + h) * D + 16 * g;
      const long long dst = (prow0 + (long long)h * kBlock) * D + 16 * g;
      if constexpr (FP8) {
        float x[16];
        A::load8(a.v_new, src, x);
        A::load8(a.v_new, src + 8, x + 8);
        const float vs = a.v_scale[h];
        const u32x2 c0 = e4m3_codes8(x, vs), c1 = e4m3_codes8(x + 8, vs);
        *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(a.vpool) + dst) = u32x4{c0[0], c0[1], c1[0], c1[1]};
      } else {  // bit copy
        constexpr int N = 16 * A::kBytes / 16;
        const u32x4* sp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_new) + src * A::kBytes);
        u32x4* dp = reinterpret_cast<u32x4*>(static_cast<char*>(a.vpool) + dst * A::kBytes);
#pragma unroll
        for (int i = 0; i < N; ++i) dp[i] = sp[i];
      }
    }
  }
}

template <int D, int ACT, bool FP8>
hipError_t rope_t(const RopeArgs& a, int num_tokens, bool interleaved, hipStream_t stream) {
  if (interleaved)
    hipLaunchKernelGGL((append_rope_kernel<D, ACT, FP8, true>), dim3(num_tokens), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((append_rope_kernel<D, ACT, FP8, false>), dim3(num_tokens), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t rope_d(const CacheView& c, const RopeArgs& a, int num_tokens, bool interleaved, hipStream_t stream) {
  if (c.dtype == 3)
    return c.act_dtype == 2 ? rope_t<D, 2, true>(a, num_tokens, interleaved, stream)
                            : rope_t<D, 1, true>(a, num_tokens, interleaved, stream);
  if (c.dtype == 2) return rope_t<D, 2, false>(a, num_tokens, interleaved, stream);
  if (c.dtype == 1) return rope_t<D, 1, false>(a, num_tokens, interleaved, stream);
  return rope_t<D, 0, false>(a, num_tokens, interleaved, stream);
}

}  // namespace

hipError_t launch_append_rope(const CacheView& c, RopeArgs a, int num_tokens, bool interleaved,
                              hipStream_t stream) {
  a.kpool = c.k_pool;
  a.vpool = c.v_pool;
  a.k_scale = c.k_scale;
  a.v_scale = c.v_scale;
  a.hkv = c.hkv;
  a.num_slots = (long long)c.num_blocks * kBlock;
  return c.d == 128 ? rope_d<128>(c, a, num_tokens, interleaved, stream)
                    : rope_d<64>(c, a, num_tokens, interleaved, stream);
}

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
