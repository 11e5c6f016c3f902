// Vector-ALU attention rows: the fp32 path of every entry point.
//
// One thread owns one (query row, query head): it keeps q and the output
// accumulator in registers and walks keys 0..p of its sequence with an
// online softmax (running max m, running sum l, rescaled accumulator).  Keys
// come either from the packed prefill K/V or, through the block table, from
// the paged pools.  fp32 configurations are small; this path favours plain
// indexing over speed.
#include "pka_internal.h"

namespace pka {
namespace {

struct ValuArgs {
  const void* q;
  void* out;
  const int32_t* cu_q;
  const int32_t* kv_lens;
  const void* k;
  const void* v;
  const void* kpool;
  const void* vpool;
  const int32_t* block_tables;
  int max_blocks;
  int num_blocks;
  int hq;
  int hkv;
  float scale_log2;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ void store(float* p, float x) { *p = x; }
__device__ __forceinline__ void store(uint16_t* p, float x) {
  *reinterpret_cast<bf16*>(p) = (bf16)x;
}

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(64) void rows_valu_kernel(ValuArgs a) {
  const int seq = blockIdx.y;
  const int head = blockIdx.z;
  const int row0 = a.cu_q ? a.cu_q[seq] : seq;  // decode: one row per sequence
  const int q_len = a.cu_q ? a.cu_q[seq + 1] - row0 : 1;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= q_len) return;
  int kv_len = PAGED ? a.kv_lens[seq] : q_len;
  if (PAGED && kv_len > a.max_blocks * kBlock) kv_len = a.max_blocks * kBlock;
  int pos = kv_len - q_len + i;  // absolute position of this row
  const int g = head / (a.hq / a.hkv);
  const T* qp = static_cast<const T*>(a.q) + ((long long)(row0 + i) * a.hq + head) * D;
  T* op = static_cast<T*>(a.out) + ((long long)(row0 + i) * a.hq + head) * D;
  float qv[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = to_f(qp[x]);
    o[x] = 0.f;
  }
  float m = -1e30f, l = 0.f;
  for (int j = 0; j <= pos; ++j) {
    const T* kr;
    const T* vr;
    if (PAGED) {
      int blk = a.block_tables[(long long)seq * a.max_blocks + j / kBlock];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const long long row = (((long long)blk * a.hkv + g) * kBlock + j % kBlock) * D;
      kr = static_cast<const T*>(a.kpool) + row;
      vr = static_cast<const T*>(a.vpool) + row;
    } else {
      const long long r = ((long long)(row0 + j) * a.hkv + g) * D;
      kr = static_cast<const T*>(a.k) + r;
      vr = static_cast<const T*>(a.v) + r;
    }
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) {
      const float kx = to_f(kr[x]);
      s = fmaf(qv[x], kx, s);
    }
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int x = 0; x < D; ++x) {
      const float vx = to_f(vr[x]);
      o[x] = fmaf(p, vx, o[x] * alpha);
    }
    m = m_new;
  }
  const float inv = pos >= 0 ? 1.f / l : 0.f;
#pragma unroll
  for (int x = 0; x < D; ++x) store(op + x, o[x] * inv);
}

template <typename T, int D>
hipError_t launch_t(const RowsProblem& p, hipStream_t stream) {
  ValuArgs a;
  a.q = p.q;
  a.out = p.out;
  a.cu_q = p.cu_q;
  a.kv_lens = p.kv_lens;
  a.k = p.k;
  a.v = p.v;
  a.kpool = p.cache.k_pool;
  a.vpool = p.cache.v_pool;
  a.block_tables = p.block_tables;
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.cache.num_blocks;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  dim3 grid((p.max_q_len + 63) / 64, p.num_seqs, p.hq);
  if (p.paged)
    hipLaunchKernelGGL((rows_valu_kernel<T, D, true>), grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((rows_valu_kernel<T, D, false>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_valu(const RowsProblem& p, hipStream_t stream) {
  if (p.max_q_len <= 0 || p.num_seqs <= 0) return hipSuccess;
  if (p.dtype == 1)
    return p.d == 128 ? launch_t<uint16_t, 128>(p, stream) : launch_t<uint16_t, 64>(p, stream);
  return p.d == 128 ? launch_t<float, 128>(p, stream) : launch_t<float, 64>(p, stream);
}

}  // namespace pka
