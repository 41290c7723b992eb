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
//   S[16 tokens][16 heads] = K_blk[16][D] . Q^T[D][16]        (heads padded to 16)
//   O^T[D][16 cols]       += V_blk^T[D][16 tokens] . P^T[16 tokens][16 cols]
//
// both on MFMA with fp32 accumulation.  Lane layouts (checked on the device):
// for v_mfma_f32_16x16x{16,32}, lane l holds A[l%16][k-slice l/16],
// B[k-slice l/16][l%16] and C[4*(l/16)+i][l%16], i < 4.  Below, t = l%16 and
// g = l/16.
//
//   * Loads: a block's 16 rows of one kv head ([P1] sketch layout
//     [block][offset][kv head][dim]) are read with whole rows per group of
//     lanes, so every 16-byte load instruction covers full cache lines (the
//     MFMA operand layout, 16 rows x 64 bytes per instruction, streams from HBM
//     at a much lower rate).  The rows are staged in a per-wave LDS tile in
//     the query's 16-bit format (int8 codes are converted exactly on the way,
//     [P2] INT8 KV cache), with the row pitches padded (16 bytes for K, 32
//     for V) so that both the row-wise reads of K and the column-wise reads
//     of V hit distinct banks.  The next block's loads are in flight while the current block is
//     computed.
//   * K: lane (t, g) reads 16 bytes of row t, the A operand of S for a
//     32-element slice of D; Q^T is the B operand, loaded once with the same
//     dims per (g, slot), zero for padded heads.
//   * S comes out as lane (t, g) = (tokens 4g+i, head t).  Each lane keeps the
//     running max and sum of head t (replicated over g).  The max used as the
//     exponent base is only raised when a head's scores exceed it by more than
//     2^8 (log2 domain), so the accumulator is rescaled rarely instead of every
//     block; weights are then at most 2^8.
//   * P^T is the B operand of the second product in the same registers.  Its
//     16-bit rounding would cost 8 (bf16) or 11 (f16) bits, so each weight
//     goes in as hi + lo: with G <= 8, column 8 + h gets head h's query as
//     well, so it computes the same scores and softmax state, and carries the
//     lo parts; the two columns are added at the end.  With G = 16 the lo
//     halves take a second MFMA.
//   * V: lane (t, g) reads 16-bit elements (row 4g+j, dim 16c+t), j < 4, from
//     the tile: V^T in the A layout, no transpose needed.  O^T lands as lane
//     (t, g) = (dims 16c+4g+i, column t), so a rescale is a per-lane multiply.
//   * k_scale of an int8 block joins the score factor and v_scale the weights.
//
// Masked tokens (offset >= valid in the last block) get score -inf by select
// and weight exactly 0; their V rows are zeroed in LDS, so whatever those
// slots hold (NaN included) never reaches the output.
#pragma once

#include "decode_kernel.h"

namespace pkv_dev {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Exponent-base slack of the lazy rescale (log2 domain): weights stay <= 2^8.
constexpr float kRescaleSlack = 8.f;

// MFMA wrappers over raw 16-bit operand bits, per query format, and the
// packing of softmax weights (rounded toward zero; the remainder is kept).
template <int QF> struct Mfma;

template <> struct Mfma<PKV_F16> {
  __device__ __forceinline__ static f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  // Packed 16-bit of (x, y), rounded toward zero, and the halves' values.
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, y));
  }
  __device__ __forceinline__ static float lo_value(uint32_t p) {
    return static_cast<float>(__builtin_bit_cast(half2_t, p).x);
  }
  __device__ __forceinline__ static float hi_value(uint32_t p) {
    return static_cast<float>(__builtin_bit_cast(half2_t, p).y);
  }
};

template <> struct Mfma<PKV_BF16> {
  __device__ __forceinline__ static f32x4_t k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  // The upper halves of two fp32 values (bytes 2, 3 of x, then of y).
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
  }
  __device__ __forceinline__ static float lo_value(uint32_t p) { return __uint_as_float(p << 16); }
  __device__ __forceinline__ static float hi_value(uint32_t p) {
    return __uint_as_float(p & 0xFFFF0000u);
  }
};

// Four int8 codes (one dword) -> four exact 16-bit values in two dwords.
// f16: 0x6400 | u is 1024 + u for a byte u; with u = code + 128 (sign bit
// flipped), subtracting 1152 leaves the code.  bf16: through fp32, whose upper
// half holds any |code| <= 127 exactly.
template <int QF> __device__ __forceinline__ u32x2_t i8x4_to_16(uint32_t w);

template <> __device__ __forceinline__ u32x2_t i8x4_to_16<PKV_F16>(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // 64 b1 64 b0
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // 64 b3 64 b2
  const half2_t bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
  return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, lo) - bias),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, hi) - bias)};
}

template <> __device__ __forceinline__ u32x2_t i8x4_to_16<PKV_BF16>(uint32_t w) {
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = static_cast<float>(static_cast<int32_t>(w << (24 - 8 * j)) >> 24);
  return u32x2_t{Mfma<PKV_BF16>::pack(x[0], x[1]), Mfma<PKV_BF16>::pack(x[2], x[3])};
}

// Four FP8 E4M3 codes -> four exact 16-bit values, with the gfx950
// scaled conversions at scale 1 (two codes per instruction; every E4M3 value
// is exactly an f16 and a bf16 value).
template <int QF> __device__ __forceinline__ u32x2_t fp8x4_to_16(uint32_t w);

template <> __device__ __forceinline__ u32x2_t fp8x4_to_16<PKV_F16>(uint32_t w) {
  return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
}

template <> __device__ __forceinline__ u32x2_t fp8x4_to_16<PKV_BF16>(uint32_t w) {
  return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// Four one-byte codes of cache format KF -> 16-bit values of format QF.
template <int KF, int QF>
__device__ __forceinline__ u32x2_t codes4_to_16(uint32_t w) {
  if constexpr (KF == PKV_I8)
    return i8x4_to_16<QF>(w);
  else
    return fp8x4_to_16<QF>(w);
}

// The grouped-query kernel works in tiles of 16 tokens, the MFMA tile height:
// a tile is one 16-token block, half of a 32-token block, or two 8-token
// blocks.
constexpr int kTileRows = 16;

template <int KF, int QF, int D>
struct GqaTile {
  static constexpr int kEB = Format<KF>::kBytes;      // bytes per cache element (2 or 1)
  static constexpr int kSrcRow = D * kEB;             // one token row of one kv head in HBM
  static constexpr int kSrcLanesPerRow = kSrcRow / 16;
  static constexpr int kLoads = kSrcRow / 64;         // 16-byte loads per lane per K (or V) block
  // LDS row pitches (16-bit elements + pad).  K rows are read 16 bytes per
  // lane down a column of rows, so a 16-byte pad puts 16 consecutive rows in
  // distinct banks; V rows are read 8 bytes per lane across 4 columns of
  // 8 consecutive rows (the transposing read), so a 32-byte pad does.
  static constexpr int kPitchK = 2 * D + 16;
  static constexpr int kPitchV = 2 * D + 32;
  static constexpr int kTileK = kTileRows * kPitchK;  // one tile of K in LDS
  static constexpr int kTileV = kTileRows * kPitchV;  // one tile of V, after the K tile
  static constexpr int kSlot = kTileK + kTileV;       // a staged tile: K, then V
  static constexpr int kSlices = D / 32;              // QK^T MFMAs (32 dims each)
  static constexpr int kTiles = D / 16;               // PV MFMAs (16 dims each)
  static_assert(scaled_format(KF) || KF == QF, "16-bit caches are read in the query's format");
  static_assert(kLoads >= 1 && kSrcRow % 64 == 0, "head_dim must fill 64-byte row slices");
};

// One tile's K and V as each lane loads them: load c covers source bytes
// 16 * (64c + lane) of the tile's rows of one kv head, in row order.
template <int KF, int QF, int D>
struct GqaStage {
  u32x4_t k[GqaTile<KF, QF, D>::kLoads];
  u32x4_t v[GqaTile<KF, QF, D>::kLoads];
};

// off_a: byte offset of the tile's first row (block and row within it);
// with two blocks per tile (TWO), rows 8..15 come from off_b instead
// (second[c] says which half this lane's load c reads).
template <int KF, int QF, int D, bool TWO>
__device__ __forceinline__ void gqa_load(GqaStage<KF, QF, D>& r, const uint8_t* kbase,
                                         const uint8_t* vbase, int64_t off_a, int64_t off_b,
                                         const uint32_t (&goff)[GqaTile<KF, QF, D>::kLoads],
                                         const bool (&second)[GqaTile<KF, QF, D>::kLoads]) {
  using T = GqaTile<KF, QF, D>;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    const int64_t off = (TWO && second[c]) ? off_b : off_a;
    r.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kbase + off + goff[c]));
  }
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    const int64_t off = (TWO && second[c]) ? off_b : off_a;
    r.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vbase + off + goff[c]));
  }
}

// Staged registers -> the wave's LDS tiles (K, then V) in 16-bit form.
// soff[c] / voff[c]: LDS byte offset of the 16-bit elements of this lane's
// load c in the K tile / from the start of the V tile.
template <int KF, int QF, int D>
__device__ __forceinline__ void gqa_stage(uint8_t* tile, const GqaStage<KF, QF, D>& r,
                                          const uint32_t (&soff)[GqaTile<KF, QF, D>::kLoads],
                                          const uint32_t (&voff)[GqaTile<KF, QF, D>::kLoads]) {
  using T = GqaTile<KF, QF, D>;
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    if constexpr (scaled_format(KF)) {
      const u32x2_t k0 = codes4_to_16<KF, QF>(r.k[c].x), k1 = codes4_to_16<KF, QF>(r.k[c].y);
      const u32x2_t k2 = codes4_to_16<KF, QF>(r.k[c].z), k3 = codes4_to_16<KF, QF>(r.k[c].w);
      const u32x2_t v0 = codes4_to_16<KF, QF>(r.v[c].x), v1 = codes4_to_16<KF, QF>(r.v[c].y);
      const u32x2_t v2 = codes4_to_16<KF, QF>(r.v[c].z), v3 = codes4_to_16<KF, QF>(r.v[c].w);
      *reinterpret_cast<u32x4_t*>(tile + soff[c]) = u32x4_t{k0.x, k0.y, k1.x, k1.y};
      *reinterpret_cast<u32x4_t*>(tile + soff[c] + 16) = u32x4_t{k2.x, k2.y, k3.x, k3.y};
      *reinterpret_cast<u32x4_t*>(tile + T::kTileK + voff[c]) = u32x4_t{v0.x, v0.y, v1.x, v1.y};
      *reinterpret_cast<u32x4_t*>(tile + T::kTileK + voff[c] + 16) = u32x4_t{v2.x, v2.y, v3.x, v3.y};
    } else {
      *reinterpret_cast<u32x4_t*>(tile + soff[c]) = r.k[c];
      *reinterpret_cast<u32x4_t*>(tile + T::kTileK + voff[c]) = r.v[c];
    }
  }
}

template <int KF, int QF, int D>
struct GqaState {
  float m;  // exponent base of head t (log2 domain): the running max, raised lazily
  float l;  // running sum of head t's weights relative to m
  f32x4_t acc[GqaTile<KF, QF, D>::kTiles];  // O^T: dims 16c + 4g + i, column t
};

// Scores, online softmax and weighted V sum of one tile staged in `tile`
// (rows outside lo <= row < valid are masked).  ksc and vsc are this lane's
// int8/fp8 scales (its tokens 4g .. 4g + 3 lie in one block).  SPLIT: G <= 8
// and the lo halves of the weights use columns 8..15.
template <int KF, int QF, int D, bool SPLIT>
__device__ __forceinline__ void gqa_compute(GqaState<KF, QF, D>& st, uint8_t* tile,
                                            const u32x4_t (&qop)[GqaTile<KF, QF, D>::kSlices],
                                            int lo, int valid, float ksc, float vsc, int t, int g,
                                            float scale_log2) {
  using T = GqaTile<KF, QF, D>;
  using M = Mfma<QF>;
  // Rows outside the attended tokens lo <= offset < valid: zero their V
  // elements (this lane's 16-byte chunks of row t) so the weighted sum never
  // touches those slots.
  if (valid < kTileRows || lo > 0) {
    if (t >= valid || t < lo) {
#pragma unroll
      for (int c = 0; c < T::kSlices; ++c)
        *reinterpret_cast<u32x4_t*>(tile + T::kTileK + t * T::kPitchV + 64 * c + 16 * g) =
            u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // V^T operands, read first so that their latency hides behind the scores
  // and the softmax: lane (t, g) needs V elements (row 4g + j, dim 16c + t),
  // j < 4, in the four 16-bit halves of two registers.  gfx950's transposing
  // LDS read delivers them in one instruction per 16 dims: within each group
  // of 16 lanes, lane 4a + b receives element b of the 8-byte pieces that
  // lanes a, a + 4, a + 8 and a + 12 address (checked on the device), so lane
  // (t, g) addresses row 4g + t / 4, dims 16c + 4 (t % 4) .. + 3.
  u32x2_t vt[T::kTiles];
  {
    typedef short i16x4_lds_t __attribute__((ext_vector_type(4)));
    const uint8_t* vp = tile + T::kTileK + (4 * g + t / 4) * T::kPitchV + 8 * (t % 4);
#pragma unroll
    for (int c = 0; c < T::kTiles; ++c) {
      const i16x4_lds_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_lds_t*)(vp + 32 * c));
      vt[c] = __builtin_bit_cast(u32x2_t, r);
    }
  }

  // S = K_blk . Q^T: lane (t, g) reads row t, dims 32c + 8g .. + 7.
  const uint8_t* krow = tile + t * T::kPitchK + 16 * g;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < T::kSlices; ++c)
    s = M::k32(*reinterpret_cast<const u32x4_t*>(krow + 64 * c), qop[c], s);

  // Online softmax of head t over tokens 4g + i, with a lazily raised base.
  const float sc = scale_log2 * ksc;
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = (4 * g + i < valid && 4 * g + i >= lo) ? s[i] * sc : -INFINITY;
  float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  const bool raise = bm > st.m + kRescaleSlack;  // also true for the first finite block
  if (__ballot(raise) != 0) {                    // wave-uniform
    const float mn = raise ? bm : st.m;
    const float alpha = fast_exp2(st.m - mn);   // 0 when st.m = -inf (acc and l are 0 then)
    st.l *= alpha;
    if (__ballot(raise && st.m != -INFINITY) != 0) {
#pragma unroll
      for (int c = 0; c < T::kTiles; ++c) st.acc[c] *= alpha;
    }
    st.m = mn;
  }
  const float ms = (st.m == -INFINITY) ? 0.f : st.m;
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = fast_exp2(sv[i] - ms);
  {
    float ps = (w[0] + w[1]) + (w[2] + w[3]);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
    ps = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
    st.l += __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] *= vsc;

  // P^T operands: column t, tokens 4g + j.
  u32x2_t p_hi, p_lo;
  if constexpr (SPLIT) {
    // Columns t and t + 8 both hold head t (t < 8): column t takes hi(w) and
    // column t + 8 the remainder lo(w).
    const uint32_t h01 = M::pack(w[0], w[1]), h23 = M::pack(w[2], w[3]);
    const uint32_t l01 = M::pack(w[0] - M::lo_value(h01), w[1] - M::hi_value(h01));
    const uint32_t l23 = M::pack(w[2] - M::lo_value(h23), w[3] - M::hi_value(h23));
    p_hi = t < 8 ? u32x2_t{h01, h23} : u32x2_t{l01, l23};
  } else {
    const uint32_t h01 = M::pack(w[0], w[1]), h23 = M::pack(w[2], w[3]);
    p_hi = u32x2_t{h01, h23};
    p_lo = u32x2_t{M::pack(w[0] - M::lo_value(h01), w[1] - M::hi_value(h01)),
                   M::pack(w[2] - M::lo_value(h23), w[3] - M::hi_value(h23))};
  }

  // O^T += V^T . P^T with the V^T operands read above.
#pragma unroll
  for (int c = 0; c < T::kTiles; ++c) {
    const u32x2_t va = vt[c];
    st.acc[c] = M::k16(va, p_hi, st.acc[c]);
    if constexpr (!SPLIT) st.acc[c] = M::k16(va, p_lo, st.acc[c]);
  }
}

// Two staged tiles A and B (32 consecutive tokens) in one step: the same
// arithmetic as gqa_compute on each, with one softmax update for both (one
// maximum, one rescale decision and one sum over their 32 tokens) and the two
// score products issued together, so the step's dependent chains overlap.
// Sixteen distinct query rows (no SPLIT); lo/valid/scales per tile as in
// gqa_compute.
template <int KF, int QF, int D>
__device__ __forceinline__ void gqa_compute_pair(GqaState<KF, QF, D>& st, uint8_t* tileA,
                                                 uint8_t* tileB,
                                                 const u32x4_t (&qop)[GqaTile<KF, QF, D>::kSlices],
                                                 int loA, int validA, int loB, int validB,
                                                 float kscA, float vscA, float kscB, float vscB,
                                                 int t, int g, float scale_log2) {
  using T = GqaTile<KF, QF, D>;
  using M = Mfma<QF>;
  typedef short i16x4_lds_t __attribute__((ext_vector_type(4)));
  // masked rows' V elements to zero (see gqa_compute)
  auto zero_masked = [&](uint8_t* tile, int lo, int valid) {
    if (valid < kTileRows || lo > 0) {
      if (t >= valid || t < lo) {
#pragma unroll
        for (int c = 0; c < T::kSlices; ++c)
          *reinterpret_cast<u32x4_t*>(tile + T::kTileK + t * T::kPitchV + 64 * c + 16 * g) =
              u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  zero_masked(tileA, loA, validA);
  zero_masked(tileB, loB, validB);
  auto read_vt = [&](const uint8_t* tile, u32x2_t (&vt)[T::kTiles]) {
    const uint8_t* vp = tile + T::kTileK + (4 * g + t / 4) * T::kPitchV + 8 * (t % 4);
#pragma unroll
    for (int c = 0; c < T::kTiles; ++c)
      vt[c] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                              (__attribute__((address_space(3))) i16x4_lds_t*)(vp + 32 * c)));
  };
  // both tiles' V^T operands first, their latency hidden by the scores
  u32x2_t vt[T::kTiles], vtB[T::kTiles];
  read_vt(tileA, vt);
  read_vt(tileB, vtB);

  // both score products, interleaved
  const uint8_t* krowA = tileA + t * T::kPitchK + 16 * g;
  const uint8_t* krowB = tileB + t * T::kPitchK + 16 * g;
  f32x4_t sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < T::kSlices; ++c) {
    sA = M::k32(*reinterpret_cast<const u32x4_t*>(krowA + 64 * c), qop[c], sA);
    sB = M::k32(*reinterpret_cast<const u32x4_t*>(krowB + 64 * c), qop[c], sB);
  }

  const float scA = scale_log2 * kscA, scB = scale_log2 * kscB;
  float sv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = sA[i] * scA;
    sv[4 + i] = sB[i] * scB;
  }
  if (loA > 0 || validA < kTileRows || loB > 0 || validB < kTileRows) {  // wave-uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g + i >= validA || 4 * g + i < loA) sv[i] = -INFINITY;
      if (4 * g + i >= validB || 4 * g + i < loB) sv[4 + i] = -INFINITY;
    }
  }
  float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                   fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  const bool raise = bm > st.m + kRescaleSlack;
  if (__ballot(raise) != 0) {
    const float mn = raise ? bm : st.m;
    const float alpha = fast_exp2(st.m - mn);
    st.l *= alpha;
    if (__ballot(raise && st.m != -INFINITY) != 0) {
#pragma unroll
      for (int c = 0; c < T::kTiles; ++c) st.acc[c] *= alpha;
    }
    st.m = mn;
  }
  const float ms = (st.m == -INFINITY) ? 0.f : st.m;
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = fast_exp2(sv[i] - ms);
  {
    float ps = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
    ps = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
    st.l += __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] *= vscA;
    w[4 + i] *= vscB;
  }
  // O^T += V^T . P^T over the pair's 32 tokens in one 16x16x32 product per
  // 16 dims (and per hi/lo part).  The contraction index k = 8g + j of lane
  // (t, g) stands for token 4g + j of tile A (j < 4) and token 4g + j - 4 of
  // tile B (j >= 4): exactly the V^T elements of the two transposing reads
  // and the weights this lane computed, side by side; the sum over k does not
  // depend on how tokens map to it.
  const uint32_t a01 = M::pack(w[0], w[1]), a23 = M::pack(w[2], w[3]);
  const uint32_t b01 = M::pack(w[4], w[5]), b23 = M::pack(w[6], w[7]);
  const u32x4_t p_hi = {a01, a23, b01, b23};
  const u32x4_t p_lo = {M::pack(w[0] - M::lo_value(a01), w[1] - M::hi_value(a01)),
                        M::pack(w[2] - M::lo_value(a23), w[3] - M::hi_value(a23)),
                        M::pack(w[4] - M::lo_value(b01), w[5] - M::hi_value(b01)),
                        M::pack(w[6] - M::lo_value(b23), w[7] - M::hi_value(b23))};
#pragma unroll
  for (int c = 0; c < T::kTiles; ++c) {
    const u32x4_t va = {vt[c].x, vt[c].y, vtB[c].x, vtB[c].y};
    st.acc[c] = M::k32(va, p_hi, st.acc[c]);
    st.acc[c] = M::k32(va, p_lo, st.acc[c]);
  }
}

// LDS of one grouped-query workgroup: per-wave K/V tiles during the loop,
// whose bytes then hold the waves' accumulators for the final merge, and the
// waves' softmax states.
template <int KF, int QF, int D, int NW>
struct GqaShared {
  static constexpr int kStageBytes = NW * GqaTile<KF, QF, D>::kSlot;
  static constexpr int kAccRow = D + 4;  // padded: the 16 columns' rows start in different banks
  static constexpr int kMergeBytes = NW * 16 * kAccRow * 4;
  static constexpr int kTileBytes = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
  static constexpr int kBytes = kTileBytes + 2 * NW * 16 * 4;
};

// Work item `item` of the grouped-query decode (one kv head of one sequence
// and partition), with `smem` the workgroup's GqaShared bytes (16-byte
// aligned).  Every thread of the workgroup calls it.
template <int KF, int QF, int D, int NW, bool SPLIT, int BS>
__device__ __forceinline__ void gqa_decode_body(const DecodeArgs& a, int item, uint8_t* smem) {
  using T = GqaTile<KF, QF, D>;
  constexpr bool kTwo = BS < kTileRows;                     // two blocks per tile
  constexpr int kTilesPerBlock = BS > kTileRows ? BS / kTileRows : 1;
  static_assert(BS == 8 || BS % kTileRows == 0, "block size");
  const int part_tiles = a.part_tokens / kTileRows;
  // Table entries of tile jj (the second only with two blocks per tile; -1
  // past the table row).
  auto tile_entries = [&](const int32_t* row, int jj, int& ea, int& eb) {
    if constexpr (kTwo) {
      ea = row[2 * jj];
      eb = 2 * jj + 1 < a.max_blocks ? row[2 * jj + 1] : -1;
    } else {
      ea = row[jj / kTilesPerBlock];
      eb = -1;
    }
  };

  using Lds = GqaShared<KF, QF, D, NW>;
  constexpr int kAccRow = Lds::kAccRow;
  float (*s_acc)[16][kAccRow] = reinterpret_cast<float (*)[16][kAccRow]>(smem);
  float (*s_m)[16] = reinterpret_cast<float (*)[16]>(smem + Lds::kTileBytes);
  float (*s_l)[16] = s_m + NW;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  // Partition-major order: workgroup i runs on XCD i % 8, so consecutive ids
  // must carry comparable work.  With the (sequence, kv head) pair fastest,
  // each XCD sees every partition index and the same kv heads of every
  // sequence (shared prefix blocks of a kv head then meet in one L2), and
  // partitions past short contexts sit at the tail of the grid.
  const int nsk = a.num_seqs * a.num_kv_heads;
  const int part = item / nsk;
  const int sk = item - part * nsk;
  const int kvh = sk % a.num_kv_heads;
  const int seq = sk / a.num_kv_heads;
  const int G = a.num_heads / a.num_kv_heads;

  const int32_t* trow = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks;
  // Issued together, before the context length is known, so that the
  // prologue waits for one memory round trip instead of three: this wave's
  // first table entries of the partition (as many as a full table holds;
  // entries past the context are never used), the query, and the length.
  // With a sliding window (or after a shared prefix) the partitions start at
  // a token that depends on the length, so the table is read after it.
  const bool early_table = a.window == 0 && !a.prefix_lens;
  const int max_tiles = (a.max_blocks * BS + kTileRows - 1) / kTileRows;
  int tb_first = -1, tb_first_b = -1;
  if (early_table) {
    const int pt0e = part * part_tiles;
    const int span_full = min(pt0e + part_tiles, max_tiles) - pt0e - wave;
    const int nk_full = span_full > 0 ? (span_full + NW - 1) / NW : 0;
    if (lane < min(64, nk_full)) tile_entries(trow, pt0e + wave + NW * lane, tb_first, tb_first_b);
  }

  // Q^T operand: head t of this kv head's group (head t % 8 when SPLIT, so
  // columns t and t + 8 compute the same scores), dims 32c + 8g .. + 7.
  u32x4_t qop[T::kSlices];
  {
    const int hq = SPLIT ? (t & 7) : t;
    const bool hv = hq < G;
    const int64_t qrow = (static_cast<int64_t>(seq) * a.num_heads + kvh * G + (hv ? hq : 0)) * D;
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) + (qrow + 8 * g) * 2;
#pragma unroll
    for (int c = 0; c < T::kSlices; ++c) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qb + 64 * c);
      qop[c] = hv ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const Span sp = attended_span(a, seq);
  const int ctx = sp.ctx;
  if (part >= sp.nparts && part != 0) return;  // partition past the context
  const int pt0 = sp.origin / kTileRows + part * part_tiles;
  const int pt1 = min(pt0 + part_tiles, (ctx + kTileRows - 1) / kTileRows);
  const bool direct = sp.nparts <= 1 && !a.prefix_lens;

  GqaState<KF, QF, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < T::kTiles; ++c) st.acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * T::kSrcRow;
  const int64_t blk_stride = row_stride * BS;
  const int64_t head_off = static_cast<int64_t>(kvh) * T::kSrcRow;
  const uint8_t* kbase = a.key_cache + head_off;
  const uint8_t* vbase = a.value_cache + head_off;
  uint8_t* tile = smem + wave * T::kSlot;
  // Per load c: global byte offset of this lane's 16 source bytes from the
  // first row of its block's part of the tile, whether that is the tile's
  // second block (two blocks per tile), and the LDS offset of their 16-bit
  // form.
  uint32_t goff[T::kLoads], soff[T::kLoads], voff[T::kLoads];
  bool second[T::kLoads];
#pragma unroll
  for (int c = 0; c < T::kLoads; ++c) {
    const int idx = 64 * c + lane;
    const int r = idx / T::kSrcLanesPerRow;
    const int ch = idx % T::kSrcLanesPerRow;
    second[c] = kTwo && r >= BS;
    goff[c] = static_cast<uint32_t>((kTwo ? r % BS : r) * row_stride + 16 * ch);
    soff[c] = static_cast<uint32_t>(r * T::kPitchK + 16 * ch * (2 / T::kEB));
    voff[c] = static_cast<uint32_t>(r * T::kPitchV + 16 * ch * (2 / T::kEB));
  }

  // Tiles of this wave: pt0 + wave + NW * k for k < nk.  The loads of tile
  // k + 1 are in flight while tile k is computed from the LDS tiles.
  const int span = pt1 - pt0 - wave;
  const int nk = span > 0 ? (span + NW - 1) / NW : 0;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int kk = k0 + lane;
    int tb = -1, tb2 = -1;
    float tks = 1.f, tvs = 1.f, tks2 = 1.f, tvs2 = 1.f;
    if (kk < nk) {
      if (k0 == 0 && early_table) {
        tb = tb_first;
        tb2 = tb_first_b;
      } else {
        tile_entries(trow, pt0 + wave + NW * kk, tb, tb2);
      }
      if (static_cast<unsigned>(tb) >= static_cast<unsigned>(a.num_blocks)) tb = -1;
      if (static_cast<unsigned>(tb2) >= static_cast<unsigned>(a.num_blocks)) tb2 = -1;
      if constexpr (scaled_format(KF)) {
        if (tb >= 0) {
          tks = a.k_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvh];
          tvs = a.v_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvh];
        }
        if (kTwo && tb2 >= 0) {
          tks2 = a.k_scales[static_cast<int64_t>(tb2) * a.num_kv_heads + kvh];
          tvs2 = a.v_scales[static_cast<int64_t>(tb2) * a.num_kv_heads + kvh];
        }
      }
    }
    const int kend = min(64, nk - k0);
    // Byte offsets of tile k's rows (its block, or its two blocks; 0 for an
    // entry outside the pool, whose rows are then masked).
    auto offsets = [&](int k, int64_t& off_a, int64_t& off_b) {
      const int p = __builtin_amdgcn_readlane(tb, k);
      off_a = static_cast<int64_t>(p < 0 ? 0 : p) * blk_stride;
      off_b = 0;
      if constexpr (kTwo) {
        const int p2 = __builtin_amdgcn_readlane(tb2, k);
        off_b = static_cast<int64_t>(p2 < 0 ? 0 : p2) * blk_stride;
      } else if constexpr (kTilesPerBlock > 1) {
        const int jj = pt0 + wave + NW * (k0 + k);
        off_a += static_cast<int64_t>((jj % kTilesPerBlock) * kTileRows) * row_stride;
      }
    };
    // Tile k of this chunk, already staged in LDS: scores, softmax, weighted sum.
    auto compute = [&](int k) {
      const int p = __builtin_amdgcn_readlane(tb, k);
      const int jj = pt0 + wave + NW * (k0 + k);
      int lo = max(0, sp.first - jj * kTileRows);
      int valid = min(kTileRows, ctx - jj * kTileRows);
      float ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tks), k));
      float vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tvs), k));
      if constexpr (kTwo) {
        const int p2 = __builtin_amdgcn_readlane(tb2, k);
        if (p < 0) lo = max(lo, BS);
        if (p2 < 0) valid = min(valid, BS);
        // lane (t, g) holds tokens 4g .. 4g + 3: rows 8..15 (g >= 2) are the
        // second block's
        if (4 * g >= BS) {
          ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tks2), k));
          vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tvs2), k));
        }
      } else {
        if (p < 0) valid = 0;
      }
      gqa_compute<KF, QF, D, SPLIT>(st, tile, qop, lo, valid, ks, vs, t, g, a.scale_log2);
    };
    GqaStage<KF, QF, D> r0;
    int64_t oa, ob;
    offsets(0, oa, ob);
    gqa_load<KF, QF, D, kTwo>(r0, kbase, vbase, oa, ob, goff, second);
    if constexpr (D == 64) {
      // head_dim 64: a tile's rows are few bytes and its compute is short, so
      // the next tile's loads alone cannot cover the memory latency; two
      // register sets keep tiles k + 1 and k + 2 in flight.
      GqaStage<KF, QF, D> r1;
      if (1 < kend) {
        offsets(1, oa, ob);
        gqa_load<KF, QF, D, kTwo>(r1, kbase, vbase, oa, ob, goff, second);
      }
      for (int k = 0; k < kend; k += 2) {
        gqa_stage(tile, r0, soff, voff);
        if (k + 2 < kend) {
          offsets(k + 2, oa, ob);
          gqa_load<KF, QF, D, kTwo>(r0, kbase, vbase, oa, ob, goff, second);
        }
        compute(k);
        if (k + 1 < kend) {
          gqa_stage(tile, r1, soff, voff);
          if (k + 3 < kend) {
            offsets(k + 3, oa, ob);
            gqa_load<KF, QF, D, kTwo>(r1, kbase, vbase, oa, ob, goff, second);
          }
          compute(k + 1);
        }
      }
    } else {
      for (int k = 0; k < kend; ++k) {
        gqa_stage(tile, r0, soff, voff);
        if (k + 1 < kend) {
          offsets(k + 1, oa, ob);
          gqa_load<KF, QF, D, kTwo>(r0, kbase, vbase, oa, ob, goff, second);
        }
        compute(k);
      }
    }
  }
  __syncthreads();  // the staging tiles become the merge buffer

  // Each wave's state to LDS: lane (t, g) holds dims 16c + 4g + i of column t.
#pragma unroll
  for (int c = 0; c < T::kTiles; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[wave][t][16 * c + 4 * g + i] = st.acc[c][i];
  if (g == 0) {
    s_m[wave][t] = st.m;
    s_l[wave][t] = st.l;
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
      const float o = SPLIT ? s_acc[w][h][d] + s_acc[w][h + 8][d] : s_acc[w][h][d];
      O = fmaf(f, o, O);
    }
    const int64_t sh = static_cast<int64_t>(seq) * a.num_heads + kvh * G + h;
    if (direct) {
      store_elem<QF>(a.out, sh * D + d, L > 0.f ? O / L : 0.f);
    } else {  // a partition's (or, after a shared prefix, the rest's) partial
      const int64_t slot = sh * a.num_parts + a.part_base + part;
      a.ws_acc[slot * D + d] = O;
      if (d == 0) {
        a.ws_ml[slot * 2] = Mx;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

template <int KF, int QF, int D, int NW, bool SPLIT, int BS>
__global__ void __launch_bounds__(NW * 64) paged_decode_gqa_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GqaShared<KF, QF, D, NW>::kBytes];
  gqa_decode_body<KF, QF, D, NW, SPLIT, BS>(a, blockIdx.x, smem);
}

}  // namespace pkv_dev
