// bf16 attention on the gfx950 matrix cores.
//
// Two work units share this file:
//
// 1. Decode unit -- (sequence, kv head, 16-row group of query heads, key
//    chunk).  Four waves stream the chunk's 16-token blocks (wave w takes
//    blocks w, w+4, ...) straight from HBM into MFMA operands:
//      S^T[16 tok x 16 q]  = K_blk  * Q^T     (mfma 16x16x32, 4x for d=128)
//      O^T[16 dim x 16 q] += V^T_blk * P^T     (mfma 16x16x16, one per 16 dims)
//    The pool layout makes the K operand one contiguous 1 KiB wave load and
//    the V^T operand two contiguous 512 B halves.  Lane (q = l%16, h = l/16)
//    holds scores of tokens 4h..4h+3 for query row q and output dims
//    16nb+4h..+3 of the same row, so the softmax rescale never leaves the
//    lane.  The four waves' (m, l, o) are merged in LDS; a unit that owns the
//    whole sequence writes the output, otherwise it writes a partial that
//    the reduce kernel merges (log-sum-exp).
//
// 2. Tile unit -- 32 query rows per wave, 4 waves per workgroup (positions x
//    query heads of one kv head), 64-key tiles staged in LDS:
//      S^T[32 key x 32 q] = K_tile * Q^T      (mfma 32x32x16)
//      O^T[32 dim x 32 q] += V^T * P^T        (mfma 32x32x16)
//    P^T comes straight from the S^T accumulator registers (the k slots of
//    the PV product follow the accumulator's key order).  V^T fragments are
//    read from a row-major LDS tile with ds_read_b64_tr_b16 (packed prefill
//    K/V) or with plain 8-byte reads from the already transposed paged V
//    tile (mixed step).  Online softmax in the exp2 domain; causal masking by
//    index only on tiles that cross the diagonal or the key end.
//
// Softmax weights are rounded to bf16 for the P*V product and the softmax
// denominator sums those rounded weights, so each output is an exact convex
// combination of value rows up to fp32 accumulation; maxima and accumulators
// are fp32; outputs are rounded to nearest-even bf16.
#include "pka_internal.h"

namespace pka {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1e30f;
constexpr int KT = 64;  // keys per LDS tile

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Vectors of bf16 are always built by float->bf16 conversion or by whole-vector
// bit casts: element-wise short<->bf16 bit casts inside a vector build are
// lowered by this compiler into perms that replicate element 0.
__device__ __forceinline__ bf16x8 concat_bf16(s16x4 lo, s16x4 hi) {
  const s16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------------------
// Decode unit
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const bf16* q;
  bf16* out;
  const int32_t* cu_q;  // nullptr: row of sequence s is s
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const bf16* kpool;
  const bf16* vpool;
  int max_blocks;
  int num_blocks;
  int num_seqs;
  int hq;
  int hkv;
  float scale_log2;
  int chunk;
  int splits;
  int row_groups;
  float* part_o;
  float* part_ml;
};

template <int D>
struct DecodeSmem {
  float m[4][16];
  float l[4][16];
  float o[4][16][D + 4];
};

template <int D>
__device__ void decode_unit(const DecodeArgs& a, int seq, int kvh, int rg, int split, char* smem_raw) {
  DecodeSmem<D>& sm = *reinterpret_cast<DecodeSmem<D>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 4, c16 = lane & 15;
  const int cap = a.max_blocks * kBlock;
  int kv_len = a.kv_lens[seq];
  kv_len = kv_len < 0 ? 0 : (kv_len > cap ? cap : kv_len);
  if (kv_len > a.splits * a.chunk) kv_len = a.splits * a.chunk;
  const int row = a.cu_q ? a.cu_q[seq] : seq;
  const int G = a.hq / a.hkv;
  const int g0 = rg * 16;
  const int ng = (G - g0) < 16 ? (G - g0) : 16;
  const int head0 = kvh * G + g0;
  const int n_split = (kv_len + a.chunk - 1) / a.chunk;
  if (split >= n_split) {
    if (split == 0) {  // no keys: defined zero output
      for (int e = tid; e < ng * D; e += kThreads)
        a.out[((long long)row * a.hq + head0 + e / D) * D + e % D] = (bf16)0.f;
    }
    return;
  }
  const int t0 = split * a.chunk;
  const int t1 = (t0 + a.chunk) < kv_len ? (t0 + a.chunk) : kv_len;
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;

  constexpr int KC = D / 32;  // k-chunks of the 16x16x32 QK product
  constexpr int NB = D / 16;  // 16-dim output blocks
  bf16x8 qf[KC];
  const bool q_ok = c16 < ng;
  const bf16* qp = a.q + ((long long)row * a.hq + head0 + (q_ok ? c16 : 0)) * D;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    bf16x8 z = {};
    qf[c] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * h) : z;
  }
  float m = kNegBig, lsum = 0.f;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = a.block_tables + (long long)seq * a.max_blocks + t0 / kBlock;
  for (int j = w; j < nblk; j += 4) {
    int blk = bt[j];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const long long tile = ((long long)blk * a.hkv + kvh) * (kBlock * D);
    const bf16* kt = a.kpool + tile;
    const bf16* vt = a.vpool + tile;
    bf16x8 ka[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = *reinterpret_cast<const bf16x8*>(kt + (64 * c + lane) * 8);
    s16x4 va[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      va[nb] = *reinterpret_cast<const s16x4*>(vt + (16 * nb + c16) * kBlock + 4 * h);

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qf[c], s, 0, 0, 0);

    const int pos0 = t0 + kBlock * j;
    const bool tail = pos0 + kBlock > t1;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = !tail || (pos0 + 4 * h + r < t1);
      x[r] = ok ? s[r] * a.scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    // The weights enter the P*V product as bf16; the running sum adds the same
    // rounded weights, so the output is an exact convex combination of V rows.
    bf16x4 pbf;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pbf[r] = (bf16)fast_exp2(x[r] - m_new);
      pr[r] = (float)pbf[r];
    }
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    const s16x4 pb = __builtin_bit_cast(s16x4, pbf);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s16x4 v = va[nb];
      if (tail) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (pos0 + 4 * h + r >= t1) v[r] = 0;
      }
      acc[nb] *= alpha;
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pb, acc[nb], 0, 0, 0);
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // Merge the four waves.
  if (h == 0) {
    sm.m[w][c16] = m;
    sm.l[w][c16] = lsum;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    *reinterpret_cast<f32x4*>(&sm.o[w][c16][16 * nb + 4 * h]) = acc[nb];
  __syncthreads();
  const bool whole = (n_split == 1);
  for (int e = tid; e < ng * D; e += kThreads) {
    const int r = e / D, dim = e % D;
    const float M = fmaxf(fmaxf(sm.m[0][r], sm.m[1][r]), fmaxf(sm.m[2][r], sm.m[3][r]));
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = fast_exp2(sm.m[ww][r] - M);
      L += sm.l[ww][r] * f;
      O += sm.o[ww][r][dim] * f;
    }
    const int head = head0 + r;
    if (whole) {
      a.out[((long long)row * a.hq + head) * D + dim] = (bf16)(O / L);
    } else {
      const long long idx = ((long long)seq * a.hq + head) * a.splits + split;
      a.part_o[idx * D + dim] = O;
      if (dim == 0) {
        a.part_ml[2 * idx] = M;
        a.part_ml[2 * idx + 1] = L;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(DecodeSmem<D>)];
  long long id = blockIdx.x;
  const int split = (int)(id % a.splits);
  id /= a.splits;
  const int rg = (int)(id % a.row_groups);
  id /= a.row_groups;
  const int kvh = (int)(id % a.hkv);
  const int seq = (int)(id / a.hkv);
  decode_unit<D>(a, seq, kvh, rg, split, smem);
}

// Merge of split-context partials: one workgroup of 64 lanes per (row, head).
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  const int seq = blockIdx.x / a.hq;
  const int head = blockIdx.x % a.hq;
  int row = seq;
  if (a.cu_q) {
    row = a.cu_q[seq];
    if (a.cu_q[seq + 1] - row != 1) return;
  }
  const int cap = a.max_blocks * kBlock;
  int kv_len = a.kv_lens[seq];
  kv_len = kv_len < 0 ? 0 : (kv_len > cap ? cap : kv_len);
  if (kv_len > a.splits * a.chunk) kv_len = a.splits * a.chunk;
  const int n = (kv_len + a.chunk - 1) / a.chunk;
  if (n <= 1) return;
  const long long base = ((long long)seq * a.hq + head) * a.splits;
  float M = kNegBig;
  for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_ml[2 * (base + s)]);
  float L = 0.f;
  for (int s = 0; s < n; ++s) L += a.part_ml[2 * (base + s) + 1] * fast_exp2(a.part_ml[2 * (base + s)] - M);
  const float inv = 1.f / L;
  for (int dim = threadIdx.x; dim < D; dim += 64) {
    float O = 0.f;
    for (int s = 0; s < n; ++s)
      O += a.part_o[(base + s) * D + dim] * fast_exp2(a.part_ml[2 * (base + s)] - M);
    a.out[((long long)row * a.hq + head) * D + dim] = (bf16)(O * inv);
  }
}

// ---------------------------------------------------------------------------
// Tile unit (prefill and prefill chunks)
// ---------------------------------------------------------------------------
struct TileArgs {
  const bf16* q;
  bf16* out;
  const int32_t* cu_q;
  const int32_t* kv_lens;  // nullptr: kv_len = q_len (packed prefill)
  const bf16* k;           // packed prefill K/V
  const bf16* v;
  const bf16* kpool;       // paged K/V
  const bf16* vpool;
  const int32_t* block_tables;
  int max_blocks;
  int num_blocks;
  int num_seqs;
  int hq;
  int hkv;
  float scale_log2;
  int hp;                  // query heads per workgroup (1, 2 or 4)
};

template <int D>
struct TileSmem {
  static constexpr int KSTR = D + 8;    // K tile row stride (elements)
  static constexpr int VSTR = D + 16;   // row-major V tile stride
  static constexpr int VTSTR = KT + 8;  // transposed V tile stride (rows stay 16-byte aligned)
  static constexpr int VELEMS = (KT * VSTR > D * VTSTR) ? KT * VSTR : D * VTSTR;
  bf16 k[KT * KSTR];
  bf16 v[VELEMS];
};

template <int D, bool PAGED>
__device__ void tile_unit(const TileArgs& a, int seq, int tile, int kvh, int hgrp, char* smem_raw) {
  using SM = TileSmem<D>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.hq / a.hkv;
  const int hp = a.hp;
  const int head = kvh * G + hgrp * hp + (w % hp);
  const int pw = w / hp;
  const int P = 32 * (4 / hp);
  const int row0 = a.cu_q[seq];
  const int q_len = a.cu_q[seq + 1] - row0;
  int kv_len = q_len;
  if (PAGED) {
    kv_len = a.kv_lens[seq];
    const int cap = a.max_blocks * kBlock;
    kv_len = kv_len > cap ? cap : kv_len;
  }
  const int cached = kv_len - q_len;
  const int i0 = tile * P + 32 * pw;
  const int wg_last = ((tile * P + P) < q_len ? (tile * P + P) : q_len) - 1;
  const int kv_end = (cached + wg_last + 1) < kv_len ? (cached + wg_last + 1) : kv_len;
  const bool wave_active = i0 < q_len;
  const int wave_last = (i0 + 31) < (q_len - 1) ? (i0 + 31) : (q_len - 1);
  const int wave_kv_end = wave_active ? ((cached + wave_last + 1) < kv_len ? (cached + wave_last + 1) : kv_len) : 0;
  const int n_kt = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;

  constexpr int KS = D / 16;   // k-steps of the QK product
  constexpr int NB = D / 32;   // 32-dim output blocks
  constexpr int CH = KT * D / 8 / kThreads;  // 16-byte chunks per thread per operand

  const int qi = i0 + l32;
  const bool q_ok = qi < q_len;
  const int my_pos = cached + qi;
  bf16x8 qf[KS];
  {
    const bf16* qp = a.q + ((long long)(row0 + (q_ok ? qi : 0)) * a.hq + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 z = {};
      qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * hh) : z;
    }
  }
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
  float m = kNegBig, lsum = 0.f;

  uint4 kreg[CH], vreg[CH];
  const int nblk_seq = (kv_len + kBlock - 1) / kBlock;
  auto gload = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + kThreads * c;
      const uint4 z = {0u, 0u, 0u, 0u};
      if (!PAGED) {
        const int key = ci / (D / 8), col = ci % (D / 8);
        const int kk = k0 + key;
        if (kk < kv_end) {
          const long long off = ((long long)(row0 + kk) * a.hkv + kvh) * D + col * 8;
          kreg[c] = *reinterpret_cast<const uint4*>(a.k + off);
          vreg[c] = *reinterpret_cast<const uint4*>(a.v + off);
        } else {
          kreg[c] = z;
          vreg[c] = z;
        }
      } else {
        const int bi = ci / (kBlock * D / 8), within = ci % (kBlock * D / 8);
        const int lb = k0 / kBlock + bi;
        if (lb < nblk_seq) {
          int blk = a.block_tables[(long long)seq * a.max_blocks + lb];
          blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
          const long long off = ((long long)blk * a.hkv + kvh) * (kBlock * D) + within * 8;
          kreg[c] = *reinterpret_cast<const uint4*>(a.kpool + off);
          vreg[c] = *reinterpret_cast<const uint4*>(a.vpool + off);
        } else {
          kreg[c] = z;
          vreg[c] = z;
        }
      }
    }
  };
  auto lds_store = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + kThreads * c;
      if (!PAGED) {
        const int key = ci / (D / 8), col = ci % (D / 8);
        *reinterpret_cast<uint4*>(&sm.k[key * SM::KSTR + col * 8]) = kreg[c];
        *reinterpret_cast<uint4*>(&sm.v[key * SM::VSTR + col * 8]) = vreg[c];
      } else {
        const int bi = ci / (kBlock * D / 8), within = ci % (kBlock * D / 8);
        // K: 16-byte dim group jg of token t.
        const int jg = within / kBlock, t = within % kBlock;
        const int key_local = kBlock * bi + t;
        uint4 kv = kreg[c];
        if (k0 + key_local >= kv_len) kv = uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4*>(&sm.k[key_local * SM::KSTR + jg * 8]) = kv;
        // V^T: dim `dim`, tokens 8*half .. 8*half+7 of the block.
        const int dim = within / 2, half = within % 2;
        uint4 vv = vreg[c];
        const int first = k0 + kBlock * bi + 8 * half;
        if (first + 8 > kv_len) {
          uint16_t* e = reinterpret_cast<uint16_t*>(&vv);
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (first + x >= kv_len) e[x] = 0;
        }
        *reinterpret_cast<uint4*>(&sm.v[dim * SM::VTSTR + kBlock * bi + 8 * half]) = vv;
      }
    }
  };

  if (n_kt > 0) {
    gload(0);
    lds_store(0);
  }
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    if (t + 1 < n_kt) gload(t + 1);
    const int k0 = t * KT;
    if (wave_active && k0 < wave_kv_end) {
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.k[(32 * kb + l32) * SM::KSTR + 16 * s + 8 * hh]);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sc[kb], 0, 0, 0);
        }
      }
      // Keys of accumulator element r of key block kb: k0 + 32kb + 8(r/4) + 4hh + r%4.
      const bool need_mask = (k0 + KT - 1 > cached + i0) || (k0 + KT > kv_len);
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[kb][r] * a.scale_log2;
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
            if (key > my_pos || key >= kv_len) x = -INFINITY;
          }
          sc[kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m, tmax);
      const float alpha = fast_exp2(m - m_new);
      float psum = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bf16 p = (bf16)fast_exp2(sc[kb][r] - m_new);
          psum += (float)p;  // sum of the rounded weights (see decode_unit)
          pf[2 * kb + r / 8][r % 8] = p;
        }
      lsum = lsum * alpha + psum;
      m = m_new;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
      // O^T += V^T P^T; k-step s2 covers keys 16*s2 + {4hh..4hh+3, 8+4hh..8+4hh+3}.
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s16x4 lo, hi;
          if (!PAGED) {
            // Row-major V tile; the transpose read gives lane (dim, 4 keys).
            const int g16 = (lane >> 4) & 1, jj = (lane >> 2) & 3, qd = lane & 3;
            const int col = 32 * nb + 16 * g16 + 4 * qd;
            const int key_a = 16 * s2 + 4 * hh + jj;
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&sm.v[key_a * SM::VSTR + col]));
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&sm.v[(key_a + 8) * SM::VSTR + col]));
          } else {
            const bf16* vr = &sm.v[(32 * nb + l32) * SM::VTSTR + 16 * s2 + 4 * hh];
            lo = *reinterpret_cast<const s16x4*>(vr);
            hi = *reinterpret_cast<const s16x4*>(vr + 8);
          }
          const bf16x8 vf = concat_bf16(lo, hi);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], acc[nb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (t + 1 < n_kt) {
      lds_store(t + 1);
      __syncthreads();
    }
  }
  lsum += __shfl_xor(lsum, 32);
  if (q_ok) {
    const float inv = 1.f / lsum;
    bf16* op = a.out + ((long long)(row0 + qi) * a.hq + head) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (bf16)(acc[nb][4 * r4 + x] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * nb + 8 * r4 + 4 * hh) = o4;
      }
  }
}

// Work lookup: the idx-th unit over sequences in order, where sequence s owns
// count(s) units.  All threads of the workgroup call it; the scan runs in LDS.
template <typename CountFn>
__device__ bool find_unit(int num_seqs, int idx, CountFn count, int& seq, int& local, int* scan) {
  const int tid = threadIdx.x;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kThreads) {
    const int s = c0 + tid;
    const int n = s < num_seqs ? count(s) : 0;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int total = scan[kThreads - 1];
    const int want = idx - base;
    if (want < total) {
      const int excl = tid ? scan[tid - 1] : 0;
      __syncthreads();
      if (want >= excl && want < excl + n) {
        scan[kThreads] = s;
        scan[kThreads + 1] = want - excl;
      }
      __syncthreads();
      seq = scan[kThreads];
      local = scan[kThreads + 1];
      return true;
    }
    base += total;
    __syncthreads();
  }
  return false;
}

template <int D, bool PAGED>
struct TileSmemUnion {
  union {
    TileSmem<D> tile;
    DecodeSmem<D> dec;
  };
};

// Packed varlen prefill.  Workgroup id = tile_index * X + x, X = hkv * hgroups.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(TileArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(TileSmem<D>)];
  __shared__ int scan[kThreads + 2];
  const int G = a.hq / a.hkv;
  const int hgroups = G / a.hp;
  const int X = a.hkv * hgroups;
  const int x = blockIdx.x % X;
  const int tidx = blockIdx.x / X;
  const int P = 32 * (4 / a.hp);
  const int32_t* cu = a.cu_q;
  int seq, local;
  if (!find_unit(a.num_seqs, tidx, [&](int s) { return (cu[s + 1] - cu[s] + P - 1) / P; }, seq, local, scan))
    return;
  const int ntiles = (cu[seq + 1] - cu[seq] + P - 1) / P;
  tile_unit<D, false>(a, seq, ntiles - 1 - local, x / hgroups, x % hgroups, smem);
}

// Mixed step: workgroups [0, n_tile_wgs) run prefill-chunk tiles of sequences
// with q_len > 1 (paged K/V); the rest run decode units of q_len == 1 rows.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void mixed_kernel(TileArgs a, DecodeArgs d, int n_tile_wgs) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(TileSmemUnion<D, true>)];
  __shared__ int scan[kThreads + 2];
  const int32_t* cu = a.cu_q;
  if ((int)blockIdx.x < n_tile_wgs) {
    const int G = a.hq / a.hkv;
    const int hgroups = G / a.hp;
    const int X = a.hkv * hgroups;
    const int x = blockIdx.x % X;
    const int tidx = blockIdx.x / X;
    const int P = 32 * (4 / a.hp);
    int seq, local;
    auto cnt = [&](int s) {
      const int ql = cu[s + 1] - cu[s];
      return ql > 1 ? (ql + P - 1) / P : 0;
    };
    if (!find_unit(a.num_seqs, tidx, cnt, seq, local, scan)) return;
    const int ql = cu[seq + 1] - cu[seq];
    const int ntiles = (ql + P - 1) / P;
    tile_unit<D, true>(a, seq, ntiles - 1 - local, x / hgroups, x % hgroups, smem);
  } else {
    long long id = blockIdx.x - n_tile_wgs;
    const int split = (int)(id % d.splits);
    id /= d.splits;
    const int rg = (int)(id % d.row_groups);
    id /= d.row_groups;
    const int kvh = (int)(id % d.hkv);
    const int k = (int)(id / d.hkv);
    int seq, local;
    auto cnt = [&](int s) { return (cu[s + 1] - cu[s]) == 1 ? 1 : 0; };
    if (!find_unit(d.num_seqs, k, cnt, seq, local, scan)) return;
    decode_unit<D>(d, seq, kvh, rg, split, smem);
  }
}

DecodeArgs make_decode_args(const DecodeProblem& p) {
  DecodeArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.out = static_cast<bf16*>(p.out);
  a.cu_q = p.cu_q;
  a.kv_lens = p.kv_lens;
  a.block_tables = p.block_tables;
  a.kpool = static_cast<const bf16*>(p.cache.k_pool);
  a.vpool = static_cast<const bf16*>(p.cache.v_pool);
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.cache.num_blocks;
  a.num_seqs = p.num_seqs;
  a.hq = p.hq;
  a.hkv = p.cache.hkv;
  a.scale_log2 = p.scale * kLog2e;
  a.chunk = p.plan.chunk;
  a.splits = p.plan.splits;
  a.row_groups = p.plan.row_groups;
  a.part_o = p.part_o;
  a.part_ml = p.part_ml;
  return a;
}

TileArgs make_tile_args(const RowsProblem& p) {
  TileArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.out = static_cast<bf16*>(p.out);
  a.cu_q = p.cu_q;
  a.kv_lens = p.paged ? p.kv_lens : nullptr;
  a.k = static_cast<const bf16*>(p.k);
  a.v = static_cast<const bf16*>(p.v);
  a.kpool = static_cast<const bf16*>(p.cache.k_pool);
  a.vpool = static_cast<const bf16*>(p.cache.v_pool);
  a.block_tables = p.block_tables;
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.cache.num_blocks;
  a.num_seqs = p.num_seqs;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.scale_log2 = p.scale * kLog2e;
  a.hp = heads_per_wg(p.hq / p.hkv);
  return a;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream) {
  const DecodeArgs a = make_decode_args(p);
  const long long wgs = (long long)p.num_seqs * p.cache.hkv * p.plan.row_groups * p.plan.splits;
  if (wgs <= 0) return hipSuccess;
  if (p.cache.d == 128)
    hipLaunchKernelGGL((decode_kernel<128>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<64>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeProblem& p, hipStream_t stream) {
  if (p.plan.splits <= 1 || p.num_seqs <= 0) return hipSuccess;
  const DecodeArgs a = make_decode_args(p);
  const long long wgs = (long long)p.num_seqs * p.hq;
  if (p.cache.d == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<128>), dim3((unsigned)wgs), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<64>), dim3((unsigned)wgs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const RowsProblem& p, hipStream_t stream) {
  const TileArgs a = make_tile_args(p);
  const int hgroups = (p.hq / p.hkv) / a.hp;
  const long long wgs = (long long)p.num_tiles * p.hkv * hgroups;
  if (wgs <= 0) return hipSuccess;
  if (p.d == 128)
    hipLaunchKernelGGL((prefill_kernel<128>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<64>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mixed_mfma(const RowsProblem& rp, const DecodeProblem& dp, hipStream_t stream) {
  const TileArgs a = make_tile_args(rp);
  const DecodeArgs d = make_decode_args(dp);
  const int hgroups = (rp.hq / rp.hkv) / a.hp;
  const long long tile_wgs = (long long)rp.num_tiles * rp.hkv * hgroups;
  const long long dec_wgs = (long long)rp.num_decode_seqs * rp.hkv * dp.plan.row_groups * dp.plan.splits;
  const long long wgs = tile_wgs + dec_wgs;
  if (wgs <= 0) return hipSuccess;
  if (rp.d == 128)
    hipLaunchKernelGGL((mixed_kernel<128>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, d,
                       (int)tile_wgs);
  else
    hipLaunchKernelGGL((mixed_kernel<64>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, d,
                       (int)tile_wgs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_reduce(dp, stream);
}

}  // namespace pka
