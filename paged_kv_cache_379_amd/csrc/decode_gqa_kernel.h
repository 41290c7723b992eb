// Grouped-query decode on the matrix cores of gfx950 (CDNA4).
//
// Page keys:
//   [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com)
//   [P2] "大模型部署中KV Cache优化策略与显存管理实践教程" (yunthe.com)
//   [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn)
//
// Same computation as paged_decode_kernel ([P1] "PagedAttention注意力计算流程":
// token i of a sequence sits in physical block table[i / 16] at offset i % 16,
// score = scale * q.k, output = softmax-weighted sum of v), for the case the
// pages leave open where G = H / Hkv query heads share each kv head.  One kv
// block then feeds G heads, and per block the work is two small dense products:
//
//   S[16 tokens][16 heads]  = K_blk[16][D] . Q^T[D][16]      (heads padded to 16)
//   O^T[D][16 heads]       += V_blk^T[D][16] . P^T[16][16]
//
// Both run on MFMA with fp32 accumulation.  Lane layouts (checked on the
// device): for v_mfma_f32_16x16x{16,32}, lane l holds A[l%16][k-slice l/16],
// B[k-slice l/16][l%16] and C[4*(l/16)+i][l%16], i < 4.
//
//   * Loads: a block's 16 rows of one kv head ([P1] sketch layout
//     [block][offset][kv head][dim]) are read with whole rows per group of
//     lanes, so every load instruction covers full cache lines, and staged in
//     a per-wave LDS tile.  The MFMA operand layout needs lane l to hold row
//     l%16, i.e. 16 rows x 64 bytes per instruction, which reads from HBM at
//     a much lower rate; LDS turns one layout into the other.  The 16-byte
//     chunks of each row are XOR-swizzled by row so both the row-wise writes
//     and the column-wise reads hit distinct banks.  The next block's loads
//     are in flight while the current block is computed.
//   * K: the LDS read gives lane l 16 bytes of token row l%16, the A operand of
//     S for a 32-element slice of D.  Q^T is the B operand, loaded once, zero
//     for padded heads.  Dims are assigned to (lane group, slot) the same way
//     on both sides, so the sum over D is the plain dot product whatever the
//     order.
//   * S comes out as lane l = (tokens 4*(l/16)+i, head l%16): each lane keeps
//     the running softmax max/sum of head l%16 (replicated over the 4 lane
//     groups), and the same registers are the B operand P^T of the second
//     product.  P goes in as hi + lo halves (16x16x32 with K = 16 tokens x
//     {hi, lo}) so the weights keep ~22 bits instead of 8 (bf16) or 11 (f16).
//   * V rows arrive in the K layout, but O^T needs V^T with tokens along the
//     lane's K slice.  A 16x16x16 MFMA against the identity matrix transposes a
//     16x16 tile exactly (each output is one product by 1.0 plus zeros) into
//     lane l = (tokens 4*(l/16)+i, dim column l%16), which is the A operand.
//   * The accumulator O^T lands as lane l = (dims, head l%16), so rescaling by
//     exp2(m_old - m_new) is a per-lane scalar multiply.
//   * int8 caches ([P2] INT8 KV cache; one fp32 scale per (block, kv head)) are
//     converted exactly to the query's 16-bit format; k_scale joins the score
//     factor and v_scale the softmax weight of the block.
//
// Masked tokens (offset >= valid in the last block) get score -inf by select,
// and their V rows are zeroed before the transpose, so whatever those slots
// hold (NaN included) never reaches the output.
#pragma once

#include "decode_kernel.h"

namespace pkv_dev {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// MFMA wrappers over raw 16-bit operand bits, per query format.
template <int QF> struct Mfma;

template <> struct Mfma<PKV_F16> {
  static constexpr uint32_t kOne = 0x3C00u;
  __device__ __forceinline__ static f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  // Two fp32 values that are exactly representable -> packed bits.
  __device__ __forceinline__ static uint32_t pack_exact(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, y));
  }
  __device__ __forceinline__ static uint32_t bits_rn(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ __forceinline__ static float value(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
  }
};

template <> struct Mfma<PKV_BF16> {
  static constexpr uint32_t kOne = 0x3F80u;
  __device__ __forceinline__ static f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack_exact(float x, float y) {
    return (__float_as_uint(x) >> 16) | (__float_as_uint(y) & 0xFFFF0000u);
  }
  // Round to nearest even (finite, non-negative inputs: softmax weights).
  __device__ __forceinline__ static uint32_t bits_rn(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
  __device__ __forceinline__ static float value(uint32_t bits) { return __uint_as_float(bits << 16); }
};

// Exact conversion of int8 codes to the 16-bit query format.  f16: 0x6400|u is
// 1024 + u for u in [0, 255]; with u = code + 128, subtracting 1152 leaves the
// code.  bf16: the code goes through fp32 (exact, 8 significant bits at most).
template <int QF> __device__ __forceinline__ uint32_t i8pair(uint32_t w, int pair);

template <> __device__ __forceinline__ uint32_t i8pair<PKV_F16>(uint32_t w, int pair) {
  const uint32_t u = (w ^ 0x80808080u) >> (16 * pair);
  const uint32_t h = (u & 0xFFu) | ((u & 0xFF00u) << 8) | 0x64006400u;
  const half2_t v = __builtin_bit_cast(half2_t, h) - half2_t{static_cast<_Float16>(1152.f),
                                                             static_cast<_Float16>(1152.f)};
  return __builtin_bit_cast(uint32_t, v);
}

template <> __device__ __forceinline__ uint32_t i8pair<PKV_BF16>(uint32_t w, int pair) {
  // bytes 2 * pair (low half of the result) and 2 * pair + 1 (high half)
  const float x = static_cast<float>(static_cast<int32_t>(w << (24 - 16 * pair)) >> 24);
  const float y = static_cast<float>(static_cast<int32_t>(w << (16 - 16 * pair)) >> 24);
  return Mfma<PKV_BF16>::pack_exact(x, y);
}

template <int KF, int QF, int D>
struct GqaTile {
  static constexpr int kEB = Format<KF>::kBytes;   // bytes per cache element (2 or 1)
  static constexpr int kE = 16 / kEB;              // elements per 16-byte load
  static constexpr int kLoads = D * kEB / 64;      // 16-byte loads per lane per block, K or V
  static constexpr int kHalves = kE / 8;           // 32-element slices per load (QK^T MFMAs)
  static constexpr int kQuads = kE / 4;            // 4-element slices per load (transposes)
  static constexpr int kRowBytes = D * kEB;        // one token row of one kv head
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kRowsPer256 = 256 / kRowBytes;
  static constexpr int kTileBytes = kBlockSize * kRowBytes;  // a block's K (or V) of one kv head
  static_assert(kRowBytes <= 256 && 256 % kRowBytes == 0, "row of 64, 128 or 256 bytes");
  // LDS chunk of row r that holds global 16-byte chunk c is c ^ swizzle(r): the
  // 16 rows that one column-wise read touches then fall in distinct 16-byte
  // bank groups of each 256-byte bank row.
  __device__ __forceinline__ static int swizzle(int r) { return (r / kRowsPer256) % kLanesPerRow; }
  static_assert(KF == PKV_I8 || KF == QF, "16-bit caches are read in the query's format");
  static_assert(kLoads >= 1 && D * kEB % 64 == 0, "head_dim must fill 64-byte row slices");
};

// The A operand (8 elements) of S for slice `h` of a K load.
template <int KF, int QF>
__device__ __forceinline__ u32x4_t k_operand(const u32x4_t& r, int h) {
  if constexpr (KF == PKV_I8) {
    const uint32_t w0 = h ? r.z : r.x, w1 = h ? r.w : r.y;
    return u32x4_t{i8pair<QF>(w0, 0), i8pair<QF>(w0, 1), i8pair<QF>(w1, 0), i8pair<QF>(w1, 1)};
  } else {
    return r;
  }
}

// 4 elements (slice q) of a V load, in the query's 16-bit format.
template <int KF, int QF>
__device__ __forceinline__ u32x2_t v_quad(const u32x4_t& r, int q) {
  if constexpr (KF == PKV_I8) {
    const uint32_t w = q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
    return u32x2_t{i8pair<QF>(w, 0), i8pair<QF>(w, 1)};
  } else {
    return q == 0 ? u32x2_t{r.x, r.y} : u32x2_t{r.z, r.w};
  }
}

template <int KF, int QF, int D>
struct GqaState {
  using T = GqaTile<KF, QF, D>;
  float m;  // running max of head l%16 (log2 domain)
  float l;  // running sum of head l%16
  f32x4_t acc[T::kLoads][T::kQuads];  // O^T: dims (load, group, quad, i), head l%16
};

// Reductions over the four lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 lane-swap instructions: each call returns the lane's own value and its
// partner's, in an order that is the same for both partners, so every lane of
// a group ends with bit-identical results.
__device__ __forceinline__ float groups_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float groups_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One block's K and V, as each lane loads them: instruction c covers chunks
// 64c .. 64c + 63 of the tile in row order (whole rows per group of lanes).
template <int KF, int QF, int D>
struct GqaStage {
  u32x4_t k[GqaTile<KF, QF, D>::kLoads];
  u32x4_t v[GqaTile<KF, QF, D>::kLoads];
};

template <int KF, int QF, int D>
__device__ __forceinline__ void gqa_load(GqaStage<KF, QF, D>& r, const uint8_t* kbase,
                                         const uint8_t* vbase, int64_t blk_stride, int phys,
                                         const uint32_t (&goff)[GqaTile<KF, QF, D>::kLoads]) {
  using T = GqaTile<KF, QF, D>;
  const uint8_t* kp = kbase + static_cast<int64_t>(phys) * blk_stride;
  const uint8_t* vp = vbase + static_cast<int64_t>(phys) * blk_stride;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c)
    r.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + goff[c]));
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c)
    r.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp + goff[c]));
}

// Staged registers -> the wave's LDS tiles (K tile, then V tile); lane l of
// instruction c writes bytes 16 * (64c + l), so each row lands contiguously.
template <int KF, int QF, int D>
__device__ __forceinline__ void gqa_stage(uint8_t* tile, const GqaStage<KF, QF, D>& r, int lane) {
  using T = GqaTile<KF, QF, D>;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    *reinterpret_cast<u32x4_t*>(tile + 16 * (64 * c + lane)) = r.k[c];
    *reinterpret_cast<u32x4_t*>(tile + T::kTileBytes + 16 * (64 * c + lane)) = r.v[c];
  }
}

// Scores, online softmax and weighted V sum of one block (valid tokens < 16
// only in the last block of a context).
template <int KF, int QF, int D>
__device__ __forceinline__ void gqa_compute(GqaState<KF, QF, D>& st, const uint8_t* tile,
                                            const uint32_t (&roff)[GqaTile<KF, QF, D>::kLoads],
                                            const u32x4_t (&qop)[GqaTile<KF, QF, D>::kLoads]
                                                                [GqaTile<KF, QF, D>::kHalves],
                                            const u32x2_t ident, int valid, float ksc, float vsc,
                                            int t, int g, float scale_log2) {
  using T = GqaTile<KF, QF, D>;
  using M = Mfma<QF>;
  // Lane (t, g): row t, global chunk 4c + g of the K and V tiles.
  struct {
    u32x4_t k[T::kLoads];
    u32x4_t v[T::kLoads];
  } r;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) r.k[c] = *reinterpret_cast<const u32x4_t*>(tile + roff[c]);
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c)
    r.v[c] = *reinterpret_cast<const u32x4_t*>(tile + T::kTileBytes + roff[c]);
  // S = K_blk . Q^T
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c)
#pragma unroll
    for (int h = 0; h < T::kHalves; ++h) s = M::k32(k_operand<KF, QF>(r.k[c], h), qop[c][h], s);

  // Online softmax of head t over this block's tokens 4g + i.
  const float sc = scale_log2 * ksc;
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = (4 * g + i < valid) ? s[i] * sc : -INFINITY;
  const float bm = groups_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
  const float mn = fmaxf(st.m, bm);
  const float ms = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(st.m - ms);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - ms);
  st.l = st.l * alpha + groups_sum((p[0] + p[1]) + (p[2] + p[3]));
  st.m = mn;
  if (__ballot(alpha != 1.f) != 0) {  // wave-uniform: skip when no max moved
#pragma unroll
    for (int c = 0; c < T::kLoads; ++c)
#pragma unroll
      for (int q = 0; q < T::kQuads; ++q) st.acc[c][q] *= alpha;
  }

  // P^T operand: tokens 4g + (j % 4), hi part for j < 4 and lo part after.
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = p[i] * vsc;
    hi[i] = M::bits_rn(w);
    lo[i] = M::bits_rn(w - M::value(hi[i]));
  }
  const u32x4_t pop = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), lo[0] | (lo[1] << 16),
                       lo[2] | (lo[3] << 16)};

  // Rows past the context contribute nothing, whatever they hold.
  if (valid < kBlockSize && t >= valid) {
#pragma unroll
    for (int c = 0; c < T::kLoads; ++c) r.v[c] = u32x4_t{0u, 0u, 0u, 0u};
  }

  // O^T += V_blk^T . P^T, one 16-dim tile at a time.
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
#pragma unroll
    for (int q = 0; q < T::kQuads; ++q) {
      const f32x4_t tt = M::k16(v_quad<KF, QF>(r.v[c], q), ident, f32x4_t{0.f, 0.f, 0.f, 0.f});
      const uint32_t t01 = M::pack_exact(tt[0], tt[1]);
      const uint32_t t23 = M::pack_exact(tt[2], tt[3]);
      st.acc[c][q] = M::k32(u32x4_t{t01, t23, t01, t23}, pop, st.acc[c][q]);
    }
  }
}

template <int KF, int QF, int D, int NW>
__global__ void __launch_bounds__(NW * 64) paged_decode_gqa_kernel(DecodeArgs a) {
  using T = GqaTile<KF, QF, D>;

  // Per-wave K/V staging tiles during the loop; the same bytes then hold the
  // waves' accumulators for the final merge.
  constexpr int kStageBytes = NW * 2 * T::kTileBytes;
  constexpr int kMergeBytes = NW * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes];
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];
  float (*s_acc)[16][D] = reinterpret_cast<float (*)[16][D]>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;  // token row in a block; head column of S and O^T
  const int g = lane >> 4;  // lane group

  // Partition-major order: workgroup i runs on XCD i % 8, so consecutive ids
  // must carry comparable work.  With the (sequence, kv head) pair fastest,
  // each XCD sees every partition index and the same kv heads of every
  // sequence (shared prefix blocks of a kv head then meet in one L2), and
  // partitions past short contexts sit at the tail of the grid.
  const int item = blockIdx.x;
  const int nsk = a.num_seqs * a.num_kv_heads;
  const int part = item / nsk;
  const int sk = item - part * nsk;
  const int kvh = sk % a.num_kv_heads;
  const int seq = sk / a.num_kv_heads;
  const int G = a.num_heads / a.num_kv_heads;

  int ctx = a.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > a.max_blocks * kBlockSize ? a.max_blocks * kBlockSize : ctx);
  const int nblk = (ctx + kBlockSize - 1) / kBlockSize;
  const int pb0 = part * a.part_blocks;
  if (pb0 >= nblk && part != 0) return;  // partition past the context
  const int pb1 = min(pb0 + a.part_blocks, nblk);
  const int nparts_seq = (nblk + a.part_blocks - 1) / a.part_blocks;
  const bool direct = nparts_seq <= 1;

  // Q^T operand: head t of this kv head's group, dims (load c, group g, slice h).
  u32x4_t qop[T::kLoads][T::kHalves];
  {
    const bool hv = t < G;
    const int64_t qrow = (static_cast<int64_t>(seq) * a.num_heads + kvh * G + (hv ? t : 0)) * D;
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) + qrow * 2;
#pragma unroll
    for (int c = 0; c < T::kLoads; ++c)
#pragma unroll
      for (int h = 0; h < T::kHalves; ++h) {
        const int d0 = c * 4 * T::kE + T::kE * g + 8 * h;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qb + d0 * 2);
        qop[c][h] = hv ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
  }
  // Identity operand of the transposes: B[k = 4g + j][n = t] = (4g + j == t).
  u32x2_t ident;
  {
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = (4 * g + j == t) ? Mfma<QF>::kOne : 0u;
    ident = u32x2_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }

  GqaState<KF, QF, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c)
#pragma unroll
    for (int q = 0; q < T::kQuads; ++q) st.acc[c][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * D * T::kEB;
  const int64_t blk_stride = row_stride * kBlockSize;
  const int64_t head_off = static_cast<int64_t>(kvh) * T::kRowBytes;
  const uint8_t* kbase = a.key_cache + head_off;
  const uint8_t* vbase = a.value_cache + head_off;
  uint8_t* tile = smem + wave * 2 * T::kTileBytes;
  // Global byte offset (inside a block, from the kv head's row 0) of this
  // lane's chunk in load c, and the LDS offset of its MFMA-layout read c.
  uint32_t goff[T::kLoads], roff[T::kLoads];
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    const int idx = 64 * c + lane;
    const int r = idx / T::kLanesPerRow;
    const int ch = (idx % T::kLanesPerRow) ^ T::swizzle(r);
    goff[c] = static_cast<uint32_t>(r * row_stride + 16 * ch);
    roff[c] = static_cast<uint32_t>(t * T::kRowBytes + 16 * ((4 * c + g) ^ T::swizzle(t)));
  }
  const int32_t* trow = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks;

  // Blocks of this wave: pb0 + wave + NW * k for k < nk.  The loads of block
  // k + 1 are in flight while block k is computed from the LDS tiles.
  const int span = pb1 - pb0 - wave;
  const int nk = span > 0 ? (span + NW - 1) / NW : 0;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int kk = k0 + lane;
    int tb = -1;
    float tks = 1.f, tvs = 1.f;
    if (kk < nk) {
      tb = trow[pb0 + wave + NW * kk];
      if (static_cast<unsigned>(tb) >= static_cast<unsigned>(a.num_blocks)) tb = -1;
      if constexpr (KF == PKV_I8) {
        if (tb >= 0) {
          tks = a.k_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvh];
          tvs = a.v_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvh];
        }
      }
    }
    const int kend = min(64, nk - k0);
    // Physical id of block k of this chunk (0 if the entry is out of range; the
    // block is then fully masked).
    auto phys_of = [&](int k) {
      const int p = __builtin_amdgcn_readlane(tb, k);
      return p < 0 ? 0 : p;
    };
    GqaStage<KF, QF, D> stage;
    gqa_load(stage, kbase, vbase, blk_stride, phys_of(0), goff);
    for (int k = 0; k < kend; ++k) {
      gqa_stage(tile, stage, lane);
      if (k + 1 < kend) gqa_load(stage, kbase, vbase, blk_stride, phys_of(k + 1), goff);
      const int p = __builtin_amdgcn_readlane(tb, k);
      const int j = pb0 + wave + NW * (k0 + k);
      const int valid = p < 0 ? 0 : min(kBlockSize, ctx - j * kBlockSize);
      const float ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tks), k));
      const float vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tvs), k));
      gqa_compute(st, tile, roff, qop, ident, valid, ks, vs, t, g, a.scale_log2);
    }
  }
  __syncthreads();  // the staging tiles become the merge buffer

  // Each wave's state to LDS: lane (t, g) holds dims (c, g, q, i) of head t.
  if (t < G) {
#pragma unroll
    for (int c = 0; c < T::kLoads; ++c)
#pragma unroll
      for (int q = 0; q < T::kQuads; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_acc[wave][t][c * 4 * T::kE + T::kE * g + 4 * q + i] = st.acc[c][q][i];
    if (g == 0) {
      s_m[wave][t] = st.m;
      s_l[wave][t] = st.l;
    }
  }
  __syncthreads();

  // Merge the waves and write the result (or this partition's partial).
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float Mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mx = fmaxf(Mx, s_m[w][h]);
    const float ms = (Mx == -INFINITY) ? 0.f : Mx;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][h] - ms);
      L = fmaf(f, s_l[w][h], L);
      O = fmaf(f, s_acc[w][h][d], O);
    }
    const int64_t sh = static_cast<int64_t>(seq) * a.num_heads + kvh * G + h;
    if (direct) {
      store_elem<QF>(a.out, sh * D + d, L > 0.f ? O / L : 0.f);
    } else {
      const int64_t slot = sh * a.num_parts + part;
      a.ws_acc[slot * D + d] = O;
      if (d == 0) {
        a.ws_ml[slot * 2] = Mx;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

}  // namespace pkv_dev
