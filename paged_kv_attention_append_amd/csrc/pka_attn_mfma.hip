// bf16 / fp16 attention on the gfx950 matrix cores.  Every kernel is
// instantiated for both 16-bit element types (traits Bf16, F16 below), and the
// paged paths also for fp8 (E4M3) pools, whose codes are decoded exactly to
// the 16-bit type as they are loaded (FP8 template flag).
//
// Three work units share this file:
//
// 1. Decode unit -- (sequence, kv head, 16-row group of query heads, key
//    chunk).  Four waves stream the chunk's 16-token blocks (wave w takes
//    blocks w, w+4, ...; block ids are prefetched once per unit and the next
//    block's loads are issued before the current block is computed):
//      S^T[16 tok x 16 q]  = K_blk  * Q^T     (mfma 16x16x32, 4x for d=128)
//      O^T[16 dim x 16 q] += V^T_blk * P^T     (mfma 16x16x16, one per 16 dims)
//    K rows go straight from HBM into the A operand; the V block is staged in
//    a wave-private LDS buffer and read back transposed with
//    ds_read_b64_tr_b16.  Every K/V byte of a decode unit is read once, so
//    the block loads are non-temporal (no reuse to keep in L2 or the last-level
//    cache; on gfx950 this raises the random 4 KiB-tile read rate by ~12%).  Lane (q = l%16, h = l/16)
//    holds scores of tokens 4h..4h+3 for query row q and output dims
//    16nb+4h..+3 of the same row, so the softmax rescale never leaves the
//    lane.  The four waves' (m, l, o) are merged in LDS; a unit that owns the
//    whole sequence writes the output, otherwise it writes a partial that
//    the reduce kernel merges (log-sum-exp).  Units go out in sequence
//    order, or longest sequence first when the host gave the lengths.
//
// 2. Prefill unit -- 16-row blocks of query rows per wave (2 or 3 blocks),
//    4 waves per workgroup (positions x query heads of one kv head), 32-key
//    K/V tiles copied by DMA into an LDS ring:
//      S^T[16 key x 16 q] = K_half * Q_b^T     (mfma 16x16x32)
//      O_b^T[16 dim x 16 q] += V^T * P_b^T     (mfma 16x16x32)
//    from the packed prefill K/V or, for the mixed step's chunks, through the
//    block table from the paged pools (bottom-right causal alignment).
//
// 3. Tile unit -- the mixed step's chunks over fp8 pools: 32 query rows per
//    wave, 4 waves per workgroup, 32-key tiles read through the block table,
//    decoded to the 16-bit type and stored to a double-buffered LDS tile:
//      S^T[32 key x 32 q] = K_tile * Q^T      (mfma 32x32x16)
//      O^T[32 dim x 32 q] += V^T * P^T        (mfma 32x32x16)
//    P^T comes straight from the S^T accumulator registers (the k slots of
//    the PV product follow the accumulator's key order).  V^T fragments come
//    from the LDS transpose read (ds_read_b64_tr_b16).  Online softmax in the
//    exp2 domain; causal masking by index only on tiles that cross the
//    diagonal or the key end.
//
// Softmax weights are rounded to the element type for the P*V product and the softmax
// denominator sums those rounded weights, so each output is an exact convex
// combination of value rows up to fp32 accumulation; maxima and accumulators
// are fp32; outputs are rounded to nearest-even in the element type.
#include "pka_internal.h"

namespace pka {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1e30f;
// The running row maximum is only raised when a tile's (block's) maximum
// exceeds it by more than this (log2 units): weights then stay <= 2^8, and
// the O rescale is skipped for most tiles.
constexpr float kLazyRescale = 8.f;
constexpr int KT = kKeyTile;  // keys per LDS tile (a multiple of 32)
constexpr int KB = KT / 32;  // 32-key MFMA blocks per tile

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

// The two 16-bit element types of the matrix-core path.  Both use the same
// MFMA shapes and operand lane layouts; only the instruction, the float
// conversion and the dot product differ.
struct Bf16 {
  using E = __bf16;
  using V8 = bf16x8;
  using V4 = bf16x4;
  using V2 = bf16x2;
  static __device__ __forceinline__ f32x4 mma16x16x32(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma32x32x16(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
  template <bool HI>  // two fp8 (E4M3) codes of one half of w -> exact values
  static __device__ __forceinline__ V2 fp8x2(unsigned w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
  }
};
struct F16 {
  using E = _Float16;
  using V8 = f16x8;
  using V4 = f16x4;
  using V2 = f16x2;
  static __device__ __forceinline__ f32x4 mma16x16x32(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma32x32x16(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
  template <bool HI>
  static __device__ __forceinline__ V2 fp8x2(unsigned w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
  }
};

// Vectors of 16-bit elements are always built by float conversion or by
// whole-vector bit casts: element-wise short<->bf16 bit casts inside a vector
// build are lowered by this compiler into perms that replicate element 0.
template <typename T>
__device__ __forceinline__ typename T::V8 concat16(s16x4 lo, s16x4 hi) {
  const s16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename T::V8, c);
}

// Eight fp8 (OCP E4M3) codes, byte j of w0:w1 = element j, to exact values of
// the 16-bit type (every E4M3 value is exact in bf16 and fp16).  The gfx950
// converters decode OCP E4M3; all 256 codes were checked against the format
// definition on the GPU.
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
template <typename T>
__device__ __forceinline__ typename T::V8 fp8x8(unsigned w0, unsigned w1) {
  const auto p0 = T::template fp8x2<false>(w0), p1 = T::template fp8x2<true>(w0);
  const auto p2 = T::template fp8x2<false>(w1), p3 = T::template fp8x2<true>(w1);
  const auto a = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto b = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Decode unit
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const void* q;  // 16-bit elements of the launch's type
  void* out;
  const int32_t* cu_q;  // nullptr: row of sequence s is s
  const int32_t* kv_lens;
  const int32_t* block_tables;
  const void* kpool;
  const void* vpool;
  int max_blocks;
  int num_blocks;
  int num_seqs;
  int hq;
  int hkv;
  float scale_log2;
  int chunk;
  int splits;
  int row_groups;
  int nq;               // query rows per sequence (1: decode; k + 1: speculative verify);
                        // 0: each sequence's own count, cu_q[s + 1] - cu_q[s] (unsplit units only)
  const float* k_scale;  // fp8 pools: per kv head; nullptr otherwise
  const float* v_scale;
  float* part_o;        // partials of query row r at row r of [rows][Hq][splits]
  float* part_ml;
};

template <int D>
struct DecodeSmem {
  static constexpr int VSTR = D + 16;  // V staging row stride: 4 rows hit disjoint banks
  union {
    uint16_t v[4][kBlock * VSTR];      // one 16-token V block per wave (raw 16-bit elements)
    struct {
      float m[4][16];
      float l[4][16];
      float o[4][16][D + 4];
    } merge;
  };
};

// CG column groups of 16 per unit: CG = 2 lets one unit serve up to 32 query
// columns (speculative verify: rows x heads) from a single read of each K/V
// block, at the cost of a second set of Q fragments and accumulators.
//
// FP8: the pools hold E4M3 codes (one byte per element) and the per-kv-head
// scales k_scale / v_scale.  Codes are decoded exactly to the 16-bit type;
// k_scale joins the score scale and v_scale multiplies the output (both are
// constant over the keys of one head, so this equals attention over the
// scaled values).  K is read 16 bytes at a time, so the QK reduction takes the
// head dims in another order than the 16-bit path: lane group h owns dims
// (D/4) h .. (D/4) h + D/4 - 1 and k-chunk c of it the eight dims from
// (D/4) h + 8 c, and q is loaded in the same order.
template <int D, typename T, int CG, bool FP8>
__device__ void decode_unit(const DecodeArgs& a, int seq, int kvh, int rg, int split, char* smem_raw) {
  using SM = DecodeSmem<D>;
  using E = typename T::E;
  using V8 = typename T::V8;
  using V4 = typename T::V4;
  const E* const q_ptr = static_cast<const E*>(a.q);
  E* const out_ptr = static_cast<E*>(a.out);
  constexpr int ES = FP8 ? 1 : 2;  // bytes per pool element
  const char* const kpool = static_cast<const char*>(a.kpool);
  const char* const vpool = static_cast<const char*>(a.vpool);
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, so its branches are scalar
  const int h = lane >> 4, c16 = lane & 15;
  constexpr int KC = D / 32;        // k-chunks of the 16x16x32 QK product
  constexpr int NB = D / 16;        // 16-dim output blocks
  constexpr int CPR = D * ES / 16;  // 16-byte chunks per token row
  constexpr int TPI = 64 / CPR;     // token rows per wave load instruction
  constexpr int VI = kBlock / TPI;  // V load instructions per block
  constexpr int KL = FP8 ? D / 64 : KC;  // 16-byte K loads per lane per block
  // Dim offset of element 0 of k-chunk c for this lane (see above).
  auto kdim = [&](int c) { return FP8 ? (D / 4) * h + 8 * c : 32 * c + 8 * h; };
  const int G = a.hq / a.hkv;
  const int nq = a.nq > 0 ? a.nq : a.cu_q[seq + 1] - a.cu_q[seq];
  // Query columns of this kv head: column c is query row c / G (of the
  // sequence's nq rows) and query head kvh * G + c % G.  Column group g of row
  // group rg holds columns 16 (CG rg + g) + 0..15, one per MFMA column
  // (lane & 15); ng[g] of them exist.
  const int ncols = nq * G;
  int ng[CG];
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    const int c0 = 16 * (CG * rg + g);
    ng[g] = ncols - c0 < 0 ? 0 : (ncols - c0 < 16 ? ncols - c0 : 16);
  }
  const int t0 = split * a.chunk;

  // Loads that do not depend on kv_len go out first (all indexes clamped into
  // the buffers), so the block ids, the first K/V block and q are in flight
  // while kv_len is fetched: the unit starts streaming after two memory
  // latencies instead of four.
  const int32_t* bt = a.block_tables + (long long)seq * a.max_blocks + t0 / kBlock;
  const int bt_room = a.max_blocks - t0 / kBlock;  // entries left in this row of the table
  int my_n = (a.chunk / kBlock - w + 3) / 4;      // refined once kv_len is known
  auto fetch_ids = [&](int base) {
    const int it = base + lane;
    const int j = w + 4 * it;
    int b = (it < my_n && j < bt_room) ? bt[j] : 0;
    return b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
  };
  int ids = fetch_ids(0);
  const int vrow = lane / CPR, vcol = lane % CPR;
  struct BlockRegs {
    u32x4 k[KL];
    u32x4 v[VI];
  };
  auto load_block = [&](int it) {
    BlockRegs r;
    const int blk = __builtin_amdgcn_readlane(ids, it & 63);
    const long long tile = ((long long)blk * a.hkv + kvh) * (kBlock * D * ES);  // bytes
    const char* kt = kpool + tile;
    const char* vt = vpool + tile;
#pragma unroll
    for (int c = 0; c < KL; ++c)
      r.k[c] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kt + (c16 * D + (FP8 ? kdim(2 * c) : kdim(c))) * ES));
#pragma unroll
    for (int i = 0; i < VI; ++i)
      r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vt + (TPI * i + vrow) * D * ES + 16 * vcol));
    return r;
  };
  BlockRegs cur = load_block(0);  // first block of this wave (clamped id); unused when my_n == 0
  const int row = a.cu_q ? a.cu_q[seq] : seq * a.nq;  // first query row of the sequence
  const int prow = a.cu_q ? seq : seq * a.nq;         // its first row of partials
  int my_qi[CG];                                      // this lane's query row in each group
  V8 qf[CG][KC];
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    // A lane past the last column (its group may be wholly empty: the second
    // group of the last row group when nq * G mod 32 is 1..16) loads column 0
    // of the sequence instead, so every q address stays inside the rows of
    // this sequence; the select below zeroes it and its output is never written.
    const bool q_ok = c16 < ng[g];
    const int col = q_ok ? 16 * (CG * rg + g) + c16 : 0;
    my_qi[g] = col / G;
    const E* qp = q_ptr + ((long long)(row + my_qi[g]) * a.hq + kvh * G + col % G) * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < KC; ++c) {  // unconditional load + select (see tile_unit)
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + kdim(c));
      qf[g][c] = __builtin_bit_cast(V8, q_ok ? v : z);
    }
  }
  const int cap = a.max_blocks * kBlock;
  int kv_len = a.kv_lens[seq];
  kv_len = kv_len < 0 ? 0 : (kv_len > cap ? cap : kv_len);
  if (kv_len > a.splits * a.chunk) kv_len = a.splits * a.chunk;
  const int n_split = (kv_len + a.chunk - 1) / a.chunk;
  if (split >= n_split) {
    if (split == 0) {  // no keys: defined zero output
#pragma unroll
      for (int g = 0; g < CG; ++g)
        for (int e = tid; e < ng[g] * D; e += kThreads) {
          const int col = 16 * (CG * rg + g) + e / D;
          out_ptr[((long long)(row + col / G) * a.hq + kvh * G + col % G) * D + e % D] = (E)0.f;
        }
    }
    return;
  }
  const int t1 = (t0 + a.chunk) < kv_len ? (t0 + a.chunk) : kv_len;
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;
  my_n = nblk > w ? (nblk - w + 3) / 4 : 0;  // this wave takes blocks w, w+4, ...
  int my_last[CG];  // last key this lane's query row sees (causal), per group
#pragma unroll
  for (int g = 0; g < CG; ++g) my_last[g] = kv_len - nq + my_qi[g];

  float m[CG], lsum[CG];
  f32x4 acc[CG][NB];
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    m[g] = kNegBig;
    lsum[g] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[g][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint16_t* vbuf = sm.v[w];
  // Log2-domain score scale and output factor (fp8: per kv head).
  const float sl2 = FP8 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float vsc = FP8 ? a.v_scale[kvh] : 1.f;

  for (int it = 0; it < my_n; ++it) {
    BlockRegs nxt;
    if (it + 1 < my_n) {
      if (((it + 1) & 63) == 0) ids = fetch_ids(it + 1);
      nxt = load_block(it + 1);
    }
    const int pos0 = t0 + kBlock * (w + 4 * it);
    const int valid = t1 - pos0;  // tokens of this block inside the chunk (1..16)

    V8 kf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if constexpr (FP8) {
        const u32x4 wk = cur.k[c / 2];
        kf[c] = fp8x8<T>(wk[2 * (c % 2)], wk[2 * (c % 2) + 1]);
      } else {
        kf[c] = __builtin_bit_cast(V8, cur.k[c]);
      }
    }
    f32x4 s[CG];
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      s[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) s[g] = T::mma16x16x32(kf[c], qf[g][c], s[g]);
    }

    // Stage V as 16-bit elements (rows past the chunk end zeroed: 0 * NaN would
    // poison the product).
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int trow = TPI * i + vrow;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 vv = trow < valid ? cur.v[i] : z;
      if constexpr (FP8) {
        *reinterpret_cast<V8*>(&vbuf[trow * SM::VSTR + 16 * vcol]) = fp8x8<T>(vv[0], vv[1]);
        *reinterpret_cast<V8*>(&vbuf[trow * SM::VSTR + 16 * vcol + 8]) = fp8x8<T>(vv[2], vv[3]);
      } else {
        *reinterpret_cast<u32x4*>(&vbuf[trow * SM::VSTR + 8 * vcol]) = vv;
      }
    }

    s16x4 pb[CG];
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = (4 * h + r < valid && pos0 + 4 * h + r <= my_last[g]) ? s[g][r] * sl2 : -INFINITY;
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      // Lazy maximum: only when some score of the wave exceeds its column's
      // running maximum by more than kLazyRescale (always in a wave's first
      // block) are the columns' block maxima exchanged and the state rescaled;
      // the branch is wave-uniform.
      if (__ballot(mx > m[g] + kLazyRescale) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m[g], mx);
        const float alpha = fast_exp2(m[g] - m_new);
        lsum[g] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[g][nb] *= alpha;
        m[g] = m_new;
      }
      // The weights enter the P*V product rounded to the element type; the
      // running sum adds the same rounded weights, so the output is an exact
      // convex combination of V rows.
      V4 pbf;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pbf[r] = (E)fast_exp2(x[r] - m[g]);
        pr[r] = (float)pbf[r];
      }
      lsum[g] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      pb[g] = __builtin_bit_cast(s16x4, pbf);
    }
    // V^T fragment: lane (dim 16nb + c16, tokens 4h..4h+3) via the LDS transpose read.
    const int jj = (lane >> 2) & 3, qd = lane & 3;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(&vbuf[(4 * h + jj) * SM::VSTR + 16 * nb + 4 * qd]));
#pragma unroll
      for (int g = 0; g < CG; ++g) acc[g][nb] = T::mma16x16x16(va, pb[g], acc[g][nb]);
    }
    cur = nxt;
  }

  // Merge the four waves, one column group at a time (the merge area overlaps
  // the V staging buffers).
  const bool whole = (n_split == 1);
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    float ls = lsum[g];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    __syncthreads();
    if (h == 0) {
      sm.merge.m[w][c16] = m[g];
      sm.merge.l[w][c16] = ls;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4*>(&sm.merge.o[w][c16][16 * nb + 4 * h]) = acc[g][nb];
    __syncthreads();
    for (int e = tid; e < ng[g] * D; e += kThreads) {
      const int r = e / D, dim = e % D;
      const float M = fmaxf(fmaxf(sm.merge.m[0][r], sm.merge.m[1][r]), fmaxf(sm.merge.m[2][r], sm.merge.m[3][r]));
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float f = fast_exp2(sm.merge.m[ww][r] - M);
        L += sm.merge.l[ww][r] * f;
        O += sm.merge.o[ww][r][dim] * f;
      }
      const int col = 16 * (CG * rg + g) + r, qi = col / G, head = kvh * G + col % G;
      if (whole) {  // a row that sees no key (kv_len < nq, a contract violation) gets zeros
        out_ptr[((long long)(row + qi) * a.hq + head) * D + dim] = (E)(L > 0.f ? O / L * vsc : 0.f);
      } else {
        const long long idx = ((long long)(prow + qi) * a.hq + head) * a.splits + split;
        a.part_o[idx * D + dim] = O * vsc;
        if (dim == 0) {
          a.part_ml[2 * idx] = M;
          a.part_ml[2 * idx + 1] = L;
        }
      }
    }
  }
}

// Workgroup id = ((split * B + rank) * Hkv + kvh) * row_groups + rg, where
// rank r is sequence order.seq[r] (longest first) when an order is given,
// else sequence r.  Workgroups are dealt to the 8 XCDs round-robin by id, so
// with the split index slowest each XCD receives the same kv heads of every
// sequence and chunk: equal work per XCD even though only long sequences have
// later chunks.
template <int D, typename T, int CG, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeArgs a, SeqOrder order) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(DecodeSmem<D>)];
  long long id = blockIdx.x;
  const int rg = (int)(id % a.row_groups);
  id /= a.row_groups;
  const int kvh = (int)(id % a.hkv);
  id /= a.hkv;
  const int rank = (int)(id % a.num_seqs);
  const int split = (int)(id / a.num_seqs);
  const int seq = order.n > 0 ? (int)order.seq[rank] : rank;
  decode_unit<D, T, CG, FP8>(a, seq, kvh, rg, split, smem);
}

// Merge of split-context partials (log-sum-exp): one workgroup per (row,
// query head), one thread per output dim; a single pass over the chunks with
// a running maximum, so every chunk's loads are independent of the others.
template <int D, typename T>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
  const int prow = blockIdx.x / a.hq;  // row of partials: sequence prow / nq, its row prow % nq
  const int head = blockIdx.x % a.hq;
  const int seq = prow / a.nq;
  int row = prow;
  if (a.cu_q) {  // mixed step (nq == 1): decode rows only
    row = a.cu_q[seq];
    if (a.cu_q[seq + 1] - row != 1) return;
  }
  const int cap = a.max_blocks * kBlock;
  int kv_len = a.kv_lens[seq];
  kv_len = kv_len < 0 ? 0 : (kv_len > cap ? cap : kv_len);
  if (kv_len > a.splits * a.chunk) kv_len = a.splits * a.chunk;
  const int n = (kv_len + a.chunk - 1) / a.chunk;
  if (n <= 1) return;
  const long long base = ((long long)prow * a.hq + head) * a.splits;
  const float* ml = a.part_ml + 2 * base;
  const float* po = a.part_o + base * D + threadIdx.x;
  float M = kNegBig, L = 0.f, O = 0.f;
#pragma unroll 8
  for (int s = 0; s < n; ++s) {
    const float ms = ml[2 * s], ls = ml[2 * s + 1], os = po[(long long)s * D];
    const float m_new = fmaxf(M, ms);
    const float f_old = fast_exp2(M - m_new), f_new = fast_exp2(ms - m_new);
    L = L * f_old + ls * f_new;
    O = O * f_old + os * f_new;
    M = m_new;
  }
  static_cast<typename T::E*>(a.out)[((long long)row * a.hq + head) * D + threadIdx.x] =
      (typename T::E)(L > 0.f ? O / L : 0.f);
}

// ---------------------------------------------------------------------------
// Tile unit (the mixed step's chunks over fp8 pools) and the arguments of
// both row units
// ---------------------------------------------------------------------------
struct TileArgs {
  const void* q;           // 16-bit elements of the launch's type
  void* out;
  const int32_t* cu_q;
  const int32_t* kv_lens;  // nullptr: kv_len = q_len (packed prefill)
  const void* k;           // packed prefill K/V
  const void* v;
  const void* kpool;       // paged K/V (16-bit elements or fp8 codes)
  const void* vpool;
  const int32_t* block_tables;
  int max_blocks;
  int num_blocks;
  int num_seqs;
  int hq;
  int hkv;
  float scale_log2;
  int hp;                  // query heads per workgroup (1, 2 or 4)
  const float* k_scale;    // fp8 pools: per kv head; nullptr otherwise
  const float* v_scale;
};

template <int D>
struct TileSmem {
  static constexpr int KSTR = D + 8;    // K tile row stride (elements)
  // V tile row stride: a transposed read covers 4 rows x 64 B in each 32-lane
  // half, so rows must sit 64 B apart modulo the 256-byte bank window (D + 16
  // put them 32 B apart: 2-way conflicts, 1.1 conflict cycles per LDS
  // instruction in the prefill's counters; D + 32 counts none).
  static constexpr int VSTR = D + 32;
  uint16_t k[2][KT * KSTR];             // double-buffered: tile t+1 is stored while t is read
  uint16_t v[2][KT * VSTR];             // (decoded 16-bit elements)
};


// E4M3 pools, decoded exactly to the 16-bit type as the tile is stored to
// LDS; k_scale joins the score scale and v_scale the final normalisation, as
// in decode_unit.  row0 and q_len: the sequence's first packed query row and
// its query count (the caller reads them from cu_q).
template <int D, typename T>
__device__ void tile_unit(const TileArgs& a, int seq, int tile, int kvh, int hgrp, char* smem_raw, const int row0,
                          const int q_len) {
  using SM = TileSmem<D>;
  using E = typename T::E;
  using V8 = typename T::V8;
  using V4 = typename T::V4;
  const unsigned char* const k8 = static_cast<const unsigned char*>(a.kpool);
  const unsigned char* const v8 = static_cast<const unsigned char*>(a.vpool);
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, so its branches are scalar
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.hq / a.hkv;
  const int hp = a.hp;
  const int head = kvh * G + hgrp * hp + (w % hp);
  const int pw = w / hp;
  const int P = 32 * (4 / hp);
  const int cap = a.max_blocks * kBlock;
  int kv_len = a.kv_lens[seq];
  kv_len = kv_len > cap ? cap : kv_len;
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

  const int qi = i0 + l32;
  const bool q_ok = qi < q_len;
  const int my_pos = cached + qi;
  V8 qf[KS];
  {
    // Unconditional loads from a clamped row, then a select: the loads stay out
    // of exec-masked branches, which keeps the compiler from waiting on all
    // outstanding global loads at the top of the tile loop.
    const E* qp = static_cast<const E*>(a.q) + ((long long)(row0 + (q_ok ? qi : 0)) * a.hq + head) * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hh);
      qf[s] = __builtin_bit_cast(V8, q_ok ? v : z);
    }
  }
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
  float m = kNegBig, lsum = 0.f;
  const float c2 = a.scale_log2 * a.k_scale[kvh];

  u32x4 kreg, vreg;  // this thread's chunk of the next tile (16 codes of K and of V)
  // A tile spans KT / 16 blocks.  Their ids are read from the block
  // table two tiles ahead of the K/V loads that use them, so the tile loop
  // never waits on a table read before it can issue the next tile's loads.
  static_assert(KT == 2 * kBlock, "two blocks per key tile");
  const int nblk_seq = (kv_len + kBlock - 1) / kBlock;
  // The table is read-only for the whole launch, so it is read through the
  // constant address space: the (uniform) entries become scalar loads that do
  // not queue behind the K/V vector loads.  Raw ids are kept and clamped at use.
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr bt_row = (const_i32_ptr)(a.block_tables + (long long)seq * a.max_blocks);
  struct TileIds {
    int b[2];
  };
  auto load_ids = [&](int t) {
    TileIds r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int bi = 2 * t + j;
      r.b[j] = (t < n_kt && bi < nblk_seq) ? bt_row[bi] : 0;
    }
    return r;
  };
  // Thread tid loads chunk tid of a tile: key tid / (D/16), the 16 codes from
  // dim 16 (tid % (D/16)).  Keys past the keys this workgroup needs are
  // zero-filled (never loaded).
  constexpr int C8 = KT * D / 16;  // 16-byte chunks (16 elements) per tile and operand
  static_assert(C8 <= kThreads, "one chunk per thread");
  auto gload = [&](int t, const TileIds& ids) {
    const int key = tid / (D / 16), col = tid % (D / 16);
    const int kk = t * KT + key;
    const u32x4 z = {0u, 0u, 0u, 0u};
    kreg = z;
    vreg = z;
    if (tid < C8 && kk < kv_end && kk / kBlock < nblk_seq) {
      int blk = key < kBlock ? ids.b[0] : ids.b[1];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const long long off = (((long long)blk * a.hkv + kvh) * kBlock + kk % kBlock) * D + col * 16;
      kreg = *reinterpret_cast<const u32x4*>(k8 + off);
      vreg = *reinterpret_cast<const u32x4*>(v8 + off);
    }
  };
  auto lds_store = [&](int buf) {
    if (tid < C8) {
      const int key = tid / (D / 16), col = tid % (D / 16);
      *reinterpret_cast<V8*>(&sm.k[buf][key * SM::KSTR + col * 16]) = fp8x8<T>(kreg[0], kreg[1]);
      *reinterpret_cast<V8*>(&sm.k[buf][key * SM::KSTR + col * 16 + 8]) = fp8x8<T>(kreg[2], kreg[3]);
      *reinterpret_cast<V8*>(&sm.v[buf][key * SM::VSTR + col * 16]) = fp8x8<T>(vreg[0], vreg[1]);
      *reinterpret_cast<V8*>(&sm.v[buf][key * SM::VSTR + col * 16 + 8]) = fp8x8<T>(vreg[2], vreg[3]);
    }
  };

  TileIds ids_next, ids_later;  // block ids of tiles t + 2 and t + 3
  if (n_kt > 0) {
    gload(0, load_ids(0));
    ids_next = load_ids(2);
    ids_later = load_ids(3);
    lds_store(0);
    if (n_kt > 1) gload(1, load_ids(1));
  }
  __syncthreads();
  const typename T::V2 ones = {(E)1.f, (E)1.f};
  for (int t = 0; t < n_kt; ++t) {
    const int cb = t & 1;
    const int k0 = t * KT;
    if (wave_active && k0 < wave_kv_end) {
      // Scheduling hint: interleave the LDS fragment reads with the MFMAs
      // (measured 1-4 % faster when this unit also served 16-bit prefill).
      __builtin_amdgcn_iglp_opt(1);
      const uint16_t* kb_lds = sm.k[cb];
      const uint16_t* vb_lds = sm.v[cb];
      f32x16 sc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const V8 ka = *reinterpret_cast<const V8*>(&kb_lds[(32 * kb + l32) * SM::KSTR + 16 * s + 8 * hh]);
          sc[kb] = T::mma32x32x16(ka, qf[s], sc[kb]);
        }
      }
      // Keys of accumulator element r of key block kb: k0 + 32kb + 8(r/4) + 4hh + r%4.
      const bool need_mask = (k0 + KT - 1 > cached + i0) || (k0 + KT > kv_len);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
            if (key > my_pos || key >= kv_len) sc[kb][r] = -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sc[kb][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c2;
      if (tmax > m + kLazyRescale) {
        const float alpha = fast_exp2(m - tmax);
        lsum *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
        m = tmax;
      }
      const float neg_m = -m;
      V8 pf[2 * KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pf[2 * kb + r / 8][r % 8] = (E)fast_exp2(fmaf(sc[kb][r], c2, neg_m));
      // Row sum of the rounded weights (they are what the P*V product uses).
      float psum = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 2 * KB; ++s2) {
        psum = T::dot2(__builtin_shufflevector(pf[s2], pf[s2], 0, 1), ones, psum);
        psum = T::dot2(__builtin_shufflevector(pf[s2], pf[s2], 2, 3), ones, psum);
        psum = T::dot2(__builtin_shufflevector(pf[s2], pf[s2], 4, 5), ones, psum);
        psum = T::dot2(__builtin_shufflevector(pf[s2], pf[s2], 6, 7), ones, psum);
      }
      lsum += psum;
      // O^T += V^T P^T; k-step s2 covers keys 16*s2 + {4hh..4hh+3, 8+4hh..8+4hh+3}.
      const int g16 = (lane >> 4) & 1, jj = (lane >> 2) & 3, qd = lane & 3;
#pragma unroll
      for (int s2 = 0; s2 < 2 * KB; ++s2) {
        const int key_a = 16 * s2 + 4 * hh + jj;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // Row-major V tile; the transpose read gives lane (dim, 4 keys).
          const int col = 32 * nb + 16 * g16 + 4 * qd;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_lds[key_a * SM::VSTR + col]));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_lds[(key_a + 8) * SM::VSTR + col]));
          acc[nb] = T::mma32x32x16(concat16<T>(lo, hi), pf[s2], acc[nb]);
        }
      }
    }
    if (t + 1 < n_kt) {
      lds_store(cb ^ 1);             // buffer cb^1 was last read in tile t-1
      if (t + 2 < n_kt) gload(t + 2, ids_next);
      ids_next = ids_later;
      ids_later = load_ids(t + 4);
    }
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 32);
  // Output: lane (row i0 + l32, dims 32nb + 8r4 + 4hh .. +3) is staged in
  // LDS (every wave is past the loop's last barrier, so the tiles are free)
  // and stored as 16-byte chunks of whole rows.
  constexpr int OSTR = D + 8;  // staging row stride (elements)
  static_assert(4 * 32 * OSTR * 2 <= (int)sizeof(SM), "staging fits the tiles");
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem_raw) + w * 32 * OSTR;
  {
    const float inv = a.v_scale[kvh] / lsum;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        V4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (E)(acc[nb][4 * r4 + x] * inv);
        *reinterpret_cast<V4*>(&stg[l32 * OSTR + 32 * nb + 8 * r4 + 4 * hh]) = o4;
      }
  }
  constexpr int CPR8 = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < 32 * CPR8 / 64; ++k) {
    const int ci = 64 * k + lane;
    const int rr = ci / CPR8, cc = ci % CPR8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stg[rr * OSTR + 8 * cc]);
    const int row = i0 + rr;
    if (row < q_len)
      *reinterpret_cast<u32x4*>(static_cast<E*>(a.out) + ((long long)(row0 + row) * a.hq + head) * D + 8 * cc) = v;
  }
}

// LDS ring of the prefill unit: R slots, each one K tile and one V tile
// of KT unpadded key rows, filled by global_load_lds (no staging registers,
// no LDS store instructions).  Chunk c (16 bytes) of key row r sits at chunk
// position c ^ ring_swz<D>(r).  The swizzle is chosen for how gfx950's LDS
// serves the two read shapes, as measured with SQ_LDS_BANK_CONFLICT on the
// bare patterns: a ds_read_b128 takes 8 consecutive lanes per pass over 32
// banks (K fragments: 8 rows x one chunk each), a transposed 64-bit read 16
// lanes per pass over 32 banks (V: 4 rows x 32 bytes); the map below leaves
// both without conflicts (the plain rotation c ^ rot(r) that spreads rows
// over 64 banks left the K reads 2-way, 2 % of the long-prompt time).
template <int D, int R>
struct RingSmem {
  static constexpr int ROWB = 2 * D;       // bytes per key row (16-bit elements)
  static constexpr int TILEB = KT * ROWB;  // bytes per operand tile
  char slot[R][2][TILEB];
};
template <int D>
__device__ __forceinline__ int ring_swz(int r) {
  return D == 128 ? (((r & 3) << 1) | ((r >> 2) & 1) | ((r & 4) << 1)) : ((((r & 3) << 1) ^ (((r >> 2) & 1) * 3)) & 7);
}
// One wave-wide global_load_lds_dwordx4: lane l copies 16 bytes from
// base + voff to LDS byte lds + 16 l.  Written as inline assembly so that
// the compiler, which cannot tell ring slots apart, does not wait for the
// whole DMA queue before every transposed LDS read; the kernel counts these
// loads itself (vmcnt) before the barrier that publishes a tile.
// The compiler does not insert hazard wait states for operands of inline
// assembly: an SALU write of M0 needs one before an LDS DMA reads it, and a
// VALU write of an SGPR (say a readfirstlane) five before a vector-memory
// instruction reads it as its address.  The s_nop 4 provides both.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);  // uniform; readfirstlane lets the compiler see that
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(reinterpret_cast<const void*>(bs)),
               "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
               : "memory");
}
// s_waitcnt with at most N vector-memory operations outstanding and the LDS
// queue drained (vmcnt[3:0], expcnt[6:4] left open, lgkmcnt[11:8] = 0).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((7 << 4) | N);
}

// Prefill unit with 16-row matrix blocks: 48 query rows per wave as three
// 16-row blocks, 4 waves per workgroup (positions x query heads of one kv
// head), 32-key K/V tiles in the LDS ring above:
//   S^T[16 key x 16 q] = K_half * Q_b^T        (mfma 16x16x32, per 16-key half)
//   O_b^T[16 dim x 16 q] += V^T * P_b^T         (mfma 16x16x32, K = the 32 keys)
// Every K and V^T fragment read from LDS feeds the three blocks, and the
// blocks are independent accumulation chains, so a wave has three times the
// matrix work per fragment and per dependency of a one-block wave.  Lane
// (q = l % 16, g = l / 16) holds, for each block, the scores of keys
// 4g..4g+3 and 16+4g..16+4g+3 of tile row q; those eight keys, in that order,
// are the lane's k-slots 8g..8g+7 of the P*V product, whose V^T operand is
// read with two transposed LDS reads per 16 dims.  The registers (Q 48, O 96,
// scores 24) fit two waves per SIMD.  The softmax is that of tile_unit:
// exp2 domain, weights rounded to the element type and summed as rounded.
// The running maximum of a row is set by the first tile and raised only when
// a lane's sum of weights exceeds 2^16 (or is not finite), which sends the
// wave through the rescale; so every weight stays <= 2^16 and the common path
// computes no row maxima.
// Unit shapes: RB 16-row blocks per wave (RB = 3: 48 rows, 218 VGPRs, two
// workgroups per CU, a four-slot ring; RB = 2: 32 rows, three workgroups per
// CU, a three-slot ring).  The host picks one per launch (see
// prefill_rows_per_wave): the 48-row unit reads each K/V fragment from LDS
// for three row blocks, the 32-row one holds more workgroups per CU, which
// start, finish and fill the chip at a finer grain.
template <int RB>
struct UnitShape {
  static constexpr int kWaveRows = 16 * RB;
  static constexpr int kRing = RB == 3 ? 4 : 3;
  static constexpr int kPerCU = RB == 3 ? 2 : 3;
};
constexpr float kWeightSumLimit = 65536.f;

template <int D, typename T, int RB, bool PAGED = false>
__device__ void prefill16_unit(const TileArgs& a, int seq, int tile, int kvh, int hgrp, char* smem_raw, int row0,
                               int q_len) {
  // The unit's coordinates are workgroup-uniform (callers may find them
  // through LDS, where the compiler cannot see that).
  seq = __builtin_amdgcn_readfirstlane(seq);
  tile = __builtin_amdgcn_readfirstlane(tile);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  hgrp = __builtin_amdgcn_readfirstlane(hgrp);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  q_len = __builtin_amdgcn_readfirstlane(q_len);
  constexpr int kRB = RB;
  constexpr int kWaveRows = UnitShape<RB>::kWaveRows;
  constexpr int kRing = UnitShape<RB>::kRing;
  using SM = RingSmem<D, kRing>;
  using E = typename T::E;
  using V8 = typename T::V8;
  using V4 = typename T::V4;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, so its branches are scalar
  const int c16 = lane & 15, g = lane >> 4;
  const int G = a.hq / a.hkv;
  const int hp = a.hp;
  const int head = kvh * G + hgrp * hp + (w % hp);
  const int P = kWaveRows * (4 / hp);  // positions per workgroup
  // Keys: the sequence's own rows (packed K/V), or its kv_len cached tokens
  // of which the last q_len are these rows (paged; kv_len capped by the
  // block table's width).  Row i sees keys 0 .. cached + i.
  int kv_len = q_len;
  if (PAGED) {
    kv_len = __builtin_amdgcn_readfirstlane(a.kv_lens[seq]);
    const int cap = a.max_blocks * kBlock;
    kv_len = kv_len > cap ? cap : kv_len;
  }
  const int cached = kv_len - q_len;
  const int i0 = tile * P + kWaveRows * (w / hp);
  const int wg_end = (tile * P + P) < q_len ? (tile * P + P) : q_len;  // rows of the workgroup
  const int kv_end = (cached + wg_end) < kv_len ? (cached + wg_end) : kv_len;  // keys it needs
  const int n_kt = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;
  const int wave_end = i0 < q_len ? ((i0 + kWaveRows) < q_len ? (i0 + kWaveRows) : q_len) : 0;
  const int wave_kv = wave_end > 0 ? ((cached + wave_end) < kv_len ? (cached + wave_end) : kv_len) : 0;
  const int n_wt = (wave_kv + KT - 1) / KT;  // tiles this wave computes

  constexpr int KC = D / 32;  // 32-dim k-steps of the QK product
  constexpr int NB = D / 16;  // 16-dim output blocks
  constexpr int CH = KT * D / 8 / kThreads;  // 16-byte chunks per thread per operand

  // Q of block b, k-step c: lane (row i0 + 16b + c16, dims 32c + 8g .. +7).
  // Unconditional loads from a clamped row, then a select (see tile_unit).
  V8 qf[kRB][KC];
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    const int row = i0 + 16 * b + c16;
    const bool ok = row < q_len;
    const E* qp = static_cast<const E*>(a.q) + ((long long)(row0 + (ok ? row : 0)) * a.hq + head) * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * g);
      qf[b][c] = __builtin_bit_cast(V8, ok ? v : z);
    }
  }
  f32x4 acc[NB][kRB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int b = 0; b < kRB; ++b) acc[nb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kRB], lsum[kRB];  // lsum: this lane's share of the row sum (its eight keys of each tile)
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    m[b] = kNegBig;
    lsum[b] = 0.f;
  }
  const float c2 = a.scale_log2;

  // DMA of tile t into slot t % kRing.  The tile's K (and V) bytes are 1 KiB
  // pieces, one per wave instruction: piece p = w IPO + j holds key rows
  // p RPI .. p RPI + RPI - 1, and lane l fills chunk position l % CPR of row
  // rr[j] = p RPI + l / CPR with the logical chunk cc[j] that position holds.
  // Rows past the workgroup's keys read its last key row instead (their
  // scores are masked, so they only have to be finite).  Paged K/V: the
  // RPI rows of one instruction lie in one 16-token block (RPI divides 16),
  // so the instruction reads from one block base plus the lane's row and
  // chunk; a tile's two block ids are read from the table one tile ahead of
  // the DMA that uses them.
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;       // key rows per wave instruction (1 KiB)
  constexpr int IPO = KT / RPI / 4;   // instructions per operand, wave and tile
  constexpr int IPW = 2 * IPO;        // per wave and tile, K and V
  static_assert(IPO >= 1 && KT % (4 * RPI) == 0, "tile split over the four waves");
  const long long rstride = (long long)a.hkv * D;  // elements between key rows
  int rr[IPO], cc[IPO];
  uint32_t voff[IPO];
#pragma unroll
  for (int j = 0; j < IPO; ++j) {
    rr[j] = (w * IPO + j) * RPI + lane / CPR;
    cc[j] = (lane % CPR) ^ ring_swz<D>(rr[j]);
    voff[j] = (uint32_t)((rr[j] * rstride + cc[j] * 8) * (long long)sizeof(E));
  }
  const size_t tile_bytes = (size_t)KT * rstride * sizeof(E);
  const long long head_off = PAGED ? (long long)kvh * kBlock * D : ((long long)row0 * a.hkv + kvh) * D;  // elements
  const char* const kbase = static_cast<const char*>(PAGED ? a.kpool : a.k) + head_off * (long long)sizeof(E);
  const char* const vbase = static_cast<const char*>(PAGED ? a.vpool : a.v) + head_off * (long long)sizeof(E);
  const size_t blk_bytes = (size_t)a.hkv * kBlock * D * sizeof(E);  // one pool block, all kv heads
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr bt_row = (const_i32_ptr)(PAGED ? a.block_tables + (long long)seq * a.max_blocks : nullptr);
  const int last_blk = (kv_end - 1) / kBlock;
  struct TileIds {
    int b0, b1;
  };
  auto load_ids = [&](int t) {
    TileIds r = {0, 0};
    if (PAGED && t < n_kt) {
      r.b0 = bt_row[2 * t < last_blk ? 2 * t : last_blk];
      r.b1 = bt_row[2 * t + 1 < last_blk ? 2 * t + 1 : last_blk];
    }
    return r;
  };
  const uint32_t lds_slot = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(sm.slot[0][0]);
  auto issue = [&](int t, const TileIds& ids) {
    const int last = kv_end - 1 - t * KT;  // last row of the tile that the workgroup needs
#pragma unroll
    for (int j = 0; j < IPO; ++j) {
      const uint32_t dst = lds_slot + (uint32_t)((t % kRing) * 2 * SM::TILEB + (w * IPO + j) * 1024);
      const int r = rr[j] < last ? rr[j] : last;  // the lane's (clamped) tile row
      if constexpr (PAGED) {
        const int p0 = (w * IPO + j) * RPI;        // the instruction's first row
        int blk = (p0 < last ? p0 : last) < kBlock ? ids.b0 : ids.b1;
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        const uint32_t o = (uint32_t)(((r % kBlock) * D + cc[j] * 8) * (int)sizeof(E));
        dma16(kbase + (size_t)blk * blk_bytes, o, dst);
        dma16(vbase + (size_t)blk * blk_bytes, o, dst + SM::TILEB);
      } else {
        const uint32_t o = last < KT - 1 ? (uint32_t)((r * rstride + cc[j] * 8) * (long long)sizeof(E)) : voff[j];
        dma16(kbase + (size_t)t * tile_bytes, o, dst);
        dma16(vbase + (size_t)t * tile_bytes, o, dst + SM::TILEB);
      }
    }
  };
  // The Q loads complete before the first DMA is issued, so that the
  // compiler's own wait for them (which cannot count the DMA) is a no-op.
  wait_vm<0>();
  for (int t = 0; t < kRing - 1 && t < n_kt; ++t) issue(t, load_ids(t));
  TileIds ids_next = load_ids(kRing - 1);  // the next tile to issue
  // Per-lane LDS read offsets within a slot.  K: row 16h + c16, logical
  // chunk 4c + g.  V (transposed reads): row 16h' + 4g + jj, elements
  // 16nb + 4qd .. +3 = logical chunk 2nb + qd/2, byte 8 (qd & 1).
  const int jj = (lane >> 2) & 3, qd = lane & 3;
  uint32_t koff[KC], voffr[NB];
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = c16 * SM::ROWB + (((4 * c + g) ^ ring_swz<D>(c16)) << 4);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    voffr[nb] = (4 * g + jj) * SM::ROWB + (((2 * nb + (qd >> 1)) ^ ring_swz<D>(4 * g + jj)) << 4) + 8 * (qd & 1);
  const typename T::V2 ones = {(E)1.f, (E)1.f};
  for (int t = 0; t < n_kt; ++t) {
    // Tile t has landed for this wave once at most the loads of the tiles
    // issued after it are outstanding; the barrier extends that to the
    // workgroup, and orders every wave's reads of slot (t - 1) % kRing (tile
    // t - 1) before the DMA that refills it with tile t + kRing - 1.
    static_assert(kRing == 3 || kRing == 4, "at most two tiles issued after the current one");
    const int ahead = n_kt - 1 - t;
    if (kRing == 4 && ahead >= 2) wait_vm<2 * IPW>();
    else if (ahead >= 1) wait_vm<IPW>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + kRing - 1 < n_kt) {
      issue(t + kRing - 1, ids_next);
      ids_next = load_ids(t + kRing);
    }
    const int k0 = t * KT;
    if (t < n_wt) {
      const char* kb_lds = sm.slot[t % kRing][0];
      const char* vb_lds = sm.slot[t % kRing][1];
      // Scores: s[h][b] lane (q c16, keys k0 + 16h + 4g + r).
      f32x4 s[2][kRB];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < kRB; ++b) s[h][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const V8 ka = *reinterpret_cast<const V8*>(kb_lds + 16 * h * SM::ROWB + koff[c]);
#pragma unroll
          for (int b = 0; b < kRB; ++b) s[h][b] = T::mma16x16x32(ka, qf[b][c], s[h][b]);
        }
      }
      // Causal mask by index, only on tiles that reach past the wave's first row.
      if (k0 + KT - 1 > cached + i0) {
#pragma unroll
        for (int b = 0; b < kRB; ++b) {
          const int lim = cached + i0 + 16 * b + c16 - k0 - 4 * g;  // key offset 16h + r visible iff <= lim
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * h + r > lim) s[h][b][r] = -INFINITY;
        }
      }
      // Row maximum of this tile for block b (the four lanes of the row).
      auto tile_max = [&](int b) {
        float mx = fmaxf(fmaxf(fmaxf(s[0][b][0], s[0][b][1]), fmaxf(s[0][b][2], s[0][b][3])),
                         fmaxf(fmaxf(s[1][b][0], s[1][b][1]), fmaxf(s[1][b][2], s[1][b][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        return mx * c2;
      };
      V8 pf[kRB];
      float ps[kRB];
      // Weights exp2(s c2 - m) rounded to the element type (slot 4h + r), and
      // the lane's sum of the rounded weights.
      auto weights = [&](int b) {
        const float neg_m = -m[b];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) pf[b][4 * h + r] = (E)fast_exp2(fmaf(s[h][b][r], c2, neg_m));
        float sum = T::dot2(__builtin_shufflevector(pf[b], pf[b], 0, 1), ones, 0.f);
        sum = T::dot2(__builtin_shufflevector(pf[b], pf[b], 2, 3), ones, sum);
        sum = T::dot2(__builtin_shufflevector(pf[b], pf[b], 4, 5), ones, sum);
        ps[b] = T::dot2(__builtin_shufflevector(pf[b], pf[b], 6, 7), ones, sum);
      };
      if (t == 0) {
#pragma unroll
        for (int b = 0; b < kRB; ++b) m[b] = fmaxf(tile_max(b), kNegBig);  // the accumulators are still zero
      }
      bool over = false;
#pragma unroll
      for (int b = 0; b < kRB; ++b) {
        weights(b);
        over |= !(ps[b] <= kWeightSumLimit);
      }
      if (__ballot(over) != 0) {  // rare: raise the running maxima that need it
#pragma unroll
        for (int b = 0; b < kRB; ++b) {
          const float m_new = fmaxf(m[b], tile_max(b));
          const float alpha = fast_exp2(m[b] - m_new);
          lsum[b] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[nb][b] *= alpha;
          m[b] = m_new;
          weights(b);
        }
      }
#pragma unroll
      for (int b = 0; b < kRB; ++b) lsum[b] += ps[b];
      // O_b^T += V^T P_b^T: lane (dim 16nb + c16, k-slots 8g..8g+7 = keys
      // 4g..4g+3, 16+4g..16+4g+3) by two transposed reads.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb_lds + voffr[nb]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb_lds + 16 * SM::ROWB + voffr[nb]));
        const V8 va = concat16<T>(lo, hi);
#pragma unroll
        for (int b = 0; b < kRB; ++b) acc[nb][b] = T::mma16x16x32(va, pf[b], acc[nb][b]);
      }
    }
  }
  // Output: lane (row i0 + 16b + c16, dims 16nb + 4g .. +3) is staged in
  // LDS (the ring is free once every wave is past its last tile) and stored
  // as whole 16-byte chunks of whole rows.
  constexpr int OSTR = D + 8;  // staging row stride (elements): rows 16 bytes apart in the banks
  static_assert(4 * kWaveRows * OSTR * 2 <= (int)sizeof(SM), "staging fits the ring");
  __syncthreads();
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem_raw) + w * kWaveRows * OSTR;
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    float ls = lsum[b];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    const float inv = 1.f / ls;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      V4 o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (E)(acc[nb][b][r] * inv);
      *reinterpret_cast<V4*>(&stg[(16 * b + c16) * OSTR + 16 * nb + 4 * g]) = o4;
    }
  }
  constexpr int CPR8 = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < kWaveRows * CPR8 / 64; ++k) {
    const int ci = 64 * k + lane;
    const int rr = ci / CPR8, cc = ci % CPR8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stg[rr * OSTR + 8 * cc]);
    const int row = i0 + rr;
    if (row < q_len)
      *reinterpret_cast<u32x4*>(static_cast<E*>(a.out) + ((long long)(row0 + row) * a.hq + head) * D + 8 * cc) = v;
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

template <int D>
struct TileSmemUnion {
  union {
    TileSmem<D> tile;
    RingSmem<D, UnitShape<2>::kRing> ring;
    DecodeSmem<D> dec;
  };
};

// Packed varlen prefill on the 16-row-block unit, longest-first.  With a work
// map (TileMap) the grid has one workgroup per (sequence, tile, head group),
// level by level.  Without one (batches beyond the map's tables), workgroup
// id = level * X + x with x = (seq * hkv + kvh) * hgroups + hgrp: level 0
// holds the last tile of every sequence long enough to have max_tiles tiles,
// the next level the tiles before them, and so on; ids past a sequence's own
// tile count exit at once.  In both layouts a workgroup's XCD (ids are dealt
// to the 8 XCDs round-robin) depends only on its head group when kv heads x
// head groups is a multiple of 8, so every tile of one (sequence, head group)
// shares its K/V in one XCD's L2.
template <int D, typename T, int RB>
__global__ __launch_bounds__(kThreads, UnitShape<RB>::kPerCU) void prefill16_kernel(TileArgs a, int max_tiles,
                                                                                     TileMap map) {
  __shared__ __attribute__((aligned(1024))) char smem[sizeof(RingSmem<D, UnitShape<RB>::kRing>)];
  const int G = a.hq / a.hkv;
  const int hgroups = G / a.hp;
  const int P = UnitShape<RB>::kWaveRows * (4 / a.hp);
  int level, hx, row0, q_len;
  if (map.levels > 0) {
    const int id = blockIdx.x;
    int lo = 0, hi = map.levels;  // level_start[lo] <= id < level_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (map.level_start[mid] <= id) lo = mid;
      else hi = mid;
    }
    const int r = id - map.level_start[lo];
    const int rank = r / map.heads;
    row0 = map.row0_of_rank[rank];
    q_len = map.q_len_of_rank[rank];
    hx = r % map.heads;
    level = lo;
  } else {
    const int X = a.num_seqs * a.hkv * hgroups;
    const int x = blockIdx.x % X;
    level = blockIdx.x / X;
    const int seq = x / (hgroups * a.hkv);
    hx = x % (hgroups * a.hkv);
    row0 = a.cu_q[seq];
    q_len = a.cu_q[seq + 1] - row0;
  }
  const int ntiles = (q_len + P - 1) / P;
  const int tile = (map.levels > 0 ? ntiles : max_tiles) - 1 - level;
  if (tile < 0 || tile >= ntiles) return;
  prefill16_unit<D, T, RB>(a, 0, tile, hx / hgroups, hx % hgroups, smem, row0, q_len);
}

// Mixed step: prefill-chunk tiles (sequences with q_len > 1, paged K/V; the
// 32-row prefill unit for 16-bit pools, the tile unit for fp8 pools, both 32
// rows per wave) and decode units (q_len == 1) in one grid.  Chunk tile j (most keys first) is
// workgroup j * stride, decode units fill the ids between and after.  With
// stride = the number of this kernel's workgroups a CU holds (made odd, see
// mixed_t), the first fill
// of the chip puts about one tile on every CU beside decode units, so a tile
// has the CU's matrix cores mostly to itself and the decode units keep the
// HBM busy; the remaining tiles follow within the first round of decode
// units.  A larger stride dispatches the last tiles so late that they run
// alone at the end of the launch; a smaller one stacks tiles on the same CUs.
// The k-th decode unit of a split level takes sequence dorder.seq[k] when the
// host gave the decode rows longest first (dorder.n > 0); otherwise
// decode_base >= 0 says the decode rows are sequences decode_base ..
// decode_base + n_dec_seqs - 1 (the host checked), and failing both each
// workgroup searches cu_q for the k-th decode row.
template <int D, typename T, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void mixed_kernel(TileArgs a, DecodeArgs d, int n_tile_wgs, int stride,
                                                             int n_dec_seqs, int decode_base, int short_max_q,
                                                             SeqOrder dorder) {
  __shared__ __attribute__((aligned(1024))) char smem[sizeof(TileSmemUnion<D>)];
  __shared__ int scan[kThreads + 2];
  const int32_t* cu = a.cu_q;
  const int id = blockIdx.x;
  if (id % stride == 0 && id / stride < n_tile_wgs) {
    const int j = id / stride;
    const int G = a.hq / a.hkv;
    const int hgroups = G / a.hp;
    const int X = a.hkv * hgroups;
    const int x = j % X;
    const int tidx = j / X;
    const int P = 32 * (4 / a.hp);
    int seq, local;
    auto cnt = [&](int s) {  // sequences with up to short_max_q rows run on decode units (other launch)
      const int ql = cu[s + 1] - cu[s];
      return ql > short_max_q ? (ql + P - 1) / P : 0;
    };
    if (!find_unit(a.num_seqs, tidx, cnt, seq, local, scan)) return;
    const int r0 = cu[seq];
    const int ql = cu[seq + 1] - r0;
    const int ntiles = (ql + P - 1) / P;
    if constexpr (FP8)
      tile_unit<D, T>(a, seq, ntiles - 1 - local, x / hgroups, x % hgroups, smem, r0, ql);
    else  // the 32-row prefill unit over the pool: the same rows per workgroup as tile_unit
      prefill16_unit<D, T, 2, true>(a, seq, ntiles - 1 - local, x / hgroups, x % hgroups, smem, r0, ql);
  } else {
    const int tiles_before = (id / stride + 1) < n_tile_wgs ? (id / stride + 1) : n_tile_wgs;
    long long k_id = id - tiles_before;  // split slowest, as in decode_kernel
    const int rg = (int)(k_id % d.row_groups);
    k_id /= d.row_groups;
    const int kvh = (int)(k_id % d.hkv);
    k_id /= d.hkv;
    const int n_dec = n_dec_seqs;
    const int k = (int)(k_id % n_dec);
    const int split = (int)(k_id / n_dec);
    int seq = dorder.n > 0 ? (int)dorder.seq[k] : decode_base + k, local;
    auto cnt = [&](int s) { return (cu[s + 1] - cu[s]) == 1 ? 1 : 0; };
    if (dorder.n == 0 && decode_base < 0 && !find_unit(d.num_seqs, k, cnt, seq, local, scan)) return;
    decode_unit<D, T, 1, FP8>(d, seq, kvh, rg, split, smem);
  }
}

DecodeArgs make_decode_args(const DecodeProblem& p) {
  // nq < 0: rows per sequence from cu_q (see DecodeArgs::nq)
  DecodeArgs a;
  a.q = p.q;
  a.out = p.out;
  a.cu_q = p.cu_q;
  a.kv_lens = p.kv_lens;
  a.block_tables = p.block_tables;
  a.kpool = p.cache.k_pool;
  a.vpool = p.cache.v_pool;
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.cache.num_blocks;
  a.num_seqs = p.num_seqs;
  a.hq = p.hq;
  a.hkv = p.cache.hkv;
  a.scale_log2 = p.scale * kLog2e;
  a.chunk = p.plan.chunk;
  a.splits = p.plan.splits;
  a.row_groups = p.plan.row_groups;
  a.nq = p.nq > 0 ? p.nq : (p.nq < 0 ? 0 : 1);
  a.k_scale = p.cache.k_scale;
  a.v_scale = p.cache.v_scale;
  a.part_o = p.part_o;
  a.part_ml = p.part_ml;
  return a;
}

TileArgs make_tile_args(const RowsProblem& p) {
  TileArgs a;
  a.q = p.q;
  a.out = p.out;
  a.cu_q = p.cu_q;
  a.kv_lens = p.paged ? p.kv_lens : nullptr;
  a.k = p.k;
  a.v = p.v;
  a.kpool = p.cache.k_pool;
  a.vpool = p.cache.v_pool;
  a.block_tables = p.block_tables;
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.cache.num_blocks;
  a.num_seqs = p.num_seqs;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.scale_log2 = p.scale * kLog2e;
  a.hp = heads_per_wg(p.hq / p.hkv);
  a.k_scale = p.cache.k_scale;
  a.v_scale = p.cache.v_scale;
  return a;
}

// Launches for one (head dim, element type); the entry points below pick them.
template <int D, typename T, bool FP8>
hipError_t decode_t(const DecodeArgs& a, const SeqOrder& ord, long long wgs, int cg, hipStream_t stream) {
  if (cg == 2)
    hipLaunchKernelGGL((decode_kernel<D, T, 2, FP8>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, ord);
  else
    hipLaunchKernelGGL((decode_kernel<D, T, 1, FP8>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, ord);
  return hipGetLastError();
}
template <int D, typename T>
hipError_t reduce_t(const DecodeArgs& a, long long wgs, hipStream_t stream) {
  hipLaunchKernelGGL((decode_reduce_kernel<D, T>), dim3((unsigned)wgs), dim3(D), 0, stream, a);
  return hipGetLastError();
}
template <int D, typename T>
hipError_t prefill16_t(const TileArgs& a, int rb, long long wgs, int max_tiles, const TileMap& map,
                       hipStream_t stream) {
  if (rb == 2)
    hipLaunchKernelGGL((prefill16_kernel<D, T, 2>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, max_tiles, map);
  else
    hipLaunchKernelGGL((prefill16_kernel<D, T, 3>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, max_tiles, map);
  return hipGetLastError();
}
template <int D, typename T, bool FP8>
hipError_t mixed_t(const TileArgs& a, const DecodeArgs& d, long long tile_wgs, long long wgs, int n_dec, int dec_base,
                   int short_max_q, const SeqOrder& dorder, hipStream_t stream) {
  // Tile stride: the kernel's resident workgroups per CU, capped by the ratio
  // of all to tile workgroups (see mixed_kernel).  The occupancy is a property
  // of this kernel instance on gfx950, asked once (thread-safe static
  // initialisation); a failed query gives 0, i.e. stride 1.
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mixed_kernel<D, T, FP8>, kThreads, 0) != hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
    return n;
  }();
  long long stride = per_cu < 1 ? 1 : per_cu;
  if (tile_wgs > 0 && stride > wgs / tile_wgs) stride = wgs / tile_wgs;
  // Workgroup ids are dealt to the 8 XCDs round-robin: an odd stride spreads
  // the tiles over all of them (and keeps each kv head's tiles on one XCD),
  // an even one crowds them onto 4, 2 or 1 (measured: stride 4 and 8 took
  // 1.5x and 2.4x as long as 3 on the 128-decode + 2-chunk GQA step).
  if (stride % 2 == 0) stride -= 1;
  if (stride < 1) stride = 1;
  hipLaunchKernelGGL((mixed_kernel<D, T, FP8>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a, d, (int)tile_wgs,
                     (int)stride, n_dec, dec_base, short_max_q, dorder);
  return hipGetLastError();
}

// Pool dtype 1 = bf16, 2 = fp16, 3 = fp8 E4M3 with bf16 or fp16 activations
// (act_dtype); the fp32 path has its own kernels.
template <template <int, typename, bool> class Launch, typename... Args>
hipError_t dispatch(const CacheView& c, Args&&... args) {
  const bool f16 = c.act_dtype == 2;
  if (c.dtype == 3) {
    if (f16) return c.d == 128 ? Launch<128, F16, true>::run(args...) : Launch<64, F16, true>::run(args...);
    return c.d == 128 ? Launch<128, Bf16, true>::run(args...) : Launch<64, Bf16, true>::run(args...);
  }
  if (f16) return c.d == 128 ? Launch<128, F16, false>::run(args...) : Launch<64, F16, false>::run(args...);
  return c.d == 128 ? Launch<128, Bf16, false>::run(args...) : Launch<64, Bf16, false>::run(args...);
}
template <int D, typename T, bool FP8>
struct DecodeLaunch {
  static hipError_t run(const DecodeArgs& a, const SeqOrder& ord, long long wgs, int cg, hipStream_t s) {
    return decode_t<D, T, FP8>(a, ord, wgs, cg, s);
  }
};
template <int D, typename T, bool FP8>
struct MixedLaunch {
  static hipError_t run(const TileArgs& a, const DecodeArgs& d, long long tile_wgs, long long wgs, int n_dec,
                        int dec_base, int short_max_q, const SeqOrder& dorder, hipStream_t s) {
    return mixed_t<D, T, FP8>(a, d, tile_wgs, wgs, n_dec, dec_base, short_max_q, dorder, s);
  }
};

}  // namespace

hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream) {
  const DecodeArgs a = make_decode_args(p);
  const long long wgs = (long long)p.num_seqs * p.cache.hkv * p.plan.row_groups * p.plan.splits;
  if (wgs <= 0) return hipSuccess;
  if (p.order) return dispatch<DecodeLaunch>(p.cache, a, *p.order, wgs, p.plan.col_groups, stream);
  SeqOrder none;
  none.n = 0;
  return dispatch<DecodeLaunch>(p.cache, a, none, wgs, p.plan.col_groups, stream);
}

hipError_t launch_decode_reduce(const DecodeProblem& p, hipStream_t stream) {
  if (p.plan.splits <= 1 || p.num_seqs <= 0) return hipSuccess;
  const DecodeArgs a = make_decode_args(p);
  const long long wgs = (long long)p.num_seqs * a.nq * p.hq;
  // The partials are fp32 and already carry v_scale: one reduction per output type.
  if (p.cache.act_dtype == 2)
    return p.cache.d == 128 ? reduce_t<128, F16>(a, wgs, stream) : reduce_t<64, F16>(a, wgs, stream);
  return p.cache.d == 128 ? reduce_t<128, Bf16>(a, wgs, stream) : reduce_t<64, Bf16>(a, wgs, stream);
}

hipError_t launch_prefill_mfma(const RowsProblem& p, hipStream_t stream) {
  const TileArgs a = make_tile_args(p);
  const int hgroups = (p.hq / p.hkv) / a.hp;
  const int P = positions_per_wg16(p.hq / p.hkv, p.prefill_rb);
  const int max_tiles = (p.max_q_len + P - 1) / P;
  TileMap none;
  none.levels = 0;
  const TileMap& map = p.map ? *p.map : none;
  const long long wgs = map.levels > 0 ? (long long)map.level_start[map.levels]
                                       : (long long)max_tiles * p.num_seqs * p.hkv * hgroups;
  if (wgs <= 0) return hipSuccess;
  if (p.dtype == 2)
    return p.d == 128 ? prefill16_t<128, F16>(a, p.prefill_rb, wgs, max_tiles, map, stream)
                      : prefill16_t<64, F16>(a, p.prefill_rb, wgs, max_tiles, map, stream);
  return p.d == 128 ? prefill16_t<128, Bf16>(a, p.prefill_rb, wgs, max_tiles, map, stream)
                    : prefill16_t<64, Bf16>(a, p.prefill_rb, wgs, max_tiles, map, stream);
}

hipError_t launch_mixed_mfma(const RowsProblem& rp, const DecodeProblem& dp, hipStream_t stream) {
  const TileArgs a = make_tile_args(rp);
  const DecodeArgs d = make_decode_args(dp);
  const int hgroups = (rp.hq / rp.hkv) / a.hp;
  const long long tile_wgs = (long long)rp.num_tiles * rp.hkv * hgroups;
  const long long dec_wgs = (long long)rp.num_decode_seqs * rp.hkv * dp.plan.row_groups * dp.plan.splits;
  const long long wgs = tile_wgs + dec_wgs;
  if (wgs <= 0) return launch_decode_reduce(dp, stream);
  SeqOrder none;
  none.n = 0;
  const hipError_t e = dispatch<MixedLaunch>(dp.cache, a, d, tile_wgs, wgs, rp.num_decode_seqs, rp.decode_base,
                                             rp.short_max_q, dp.order ? *dp.order : none, stream);
  if (e != hipSuccess) return e;
  return launch_decode_reduce(dp, stream);
}

}  // namespace pka
