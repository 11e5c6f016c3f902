// Vector-ALU attention rows: the fp32 path of every entry point.
//
// One wave owns one (query row, query head).  Lane l walks keys l, l + 64,
// l + 128, ... of the row's visible range with its own online softmax
// (running max, running sum, rescaled accumulator in registers), so the
// loads of up to 64 keys are in flight at once; the lanes' states are then
// merged with a log-sum-exp rescale: the maximum and the sums across lanes
// by shuffles, the accumulators through LDS, one output dim per lane.  Keys
// come either from the packed prefill K/V or, through the block table, from
// the paged pools.  fp32 configurations are small and launch-bound.
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

template <int D, bool PAGED>
__global__ __launch_bounds__(64) void rows_valu_kernel(ValuArgs a) {
  __shared__ float part[64][D + 1];  // lane-major accumulators for the merge (+1: no bank conflicts)
  const int seq = blockIdx.y;
  const int head = blockIdx.z;
  const int lane = threadIdx.x;
  const int row0 = a.cu_q ? a.cu_q[seq] : seq;  // decode: one row per sequence
  const int q_len = a.cu_q ? a.cu_q[seq + 1] - row0 : 1;
  const int i = blockIdx.x;
  if (i >= q_len) return;
  int kv_len = PAGED ? a.kv_lens[seq] : q_len;
  if (PAGED && kv_len > a.max_blocks * kBlock) kv_len = a.max_blocks * kBlock;
  const int pos = kv_len - q_len + i;  // absolute position of this row: keys 0..pos
  const int g = head / (a.hq / a.hkv);
  const float* qp = static_cast<const float*>(a.q) + ((long long)(row0 + i) * a.hq + head) * D;
  float* op = static_cast<float*>(a.out) + ((long long)(row0 + i) * a.hq + head) * D;
  float qv[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = qp[x];
    o[x] = 0.f;
  }
  float m = -1e30f, l = 0.f;
  for (int j = lane; j <= pos; j += 64) {
    const float* kr;
    const float* vr;
    if (PAGED) {
      int blk = a.block_tables[(long long)seq * a.max_blocks + j / kBlock];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const long long row = (((long long)blk * a.hkv + g) * kBlock + j % kBlock) * D;
      kr = static_cast<const float*>(a.kpool) + row;
      vr = static_cast<const float*>(a.vpool) + row;
    } else {
      const long long r = ((long long)(row0 + j) * a.hkv + g) * D;
      kr = static_cast<const float*>(a.k) + r;
      vr = static_cast<const float*>(a.v) + r;
    }
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) s = fmaf(qv[x], kr[x], s);
    s *= a.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int x = 0; x < D; ++x) o[x] = fmaf(p, vr[x], o[x] * alpha);
    m = m_new;
  }
  // Merge the 64 lanes: M = max of the lanes' maxima, each lane's sum and
  // accumulator scaled by exp2(m - M) (0 for a lane that saw no key).
  float M = m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float f = exp2f(m - M);
  float L = l * f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
#pragma unroll
  for (int x = 0; x < D; ++x) part[lane][x] = o[x] * f;
  __syncthreads();
  const float inv = pos >= 0 ? 1.f / L : 0.f;
  for (int x = lane; x < D; x += 64) {
    float sum = 0.f;
    for (int r = 0; r < 64; ++r) sum += part[r][x];
    op[x] = sum * inv;
  }
}

template <int D>
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
  dim3 grid(p.max_q_len, p.num_seqs, p.hq);  // one wave per (row, head)
  if (p.paged)
    hipLaunchKernelGGL((rows_valu_kernel<D, true>), grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((rows_valu_kernel<D, false>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_valu(const RowsProblem& p, hipStream_t stream) {
  if (p.max_q_len <= 0 || p.num_seqs <= 0) return hipSuccess;
  return p.d == 128 ? launch_t<128>(p, stream) : launch_t<64>(p, stream);
}

}  // namespace pka
