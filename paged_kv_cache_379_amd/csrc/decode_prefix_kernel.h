// Shared-prefix decode: attention over the blocks that a group of sequences
// shares (forks of one prompt, [P1] "vLLM调度器与PagedAttention协同工作" item
// 2; [P2] "Prefix Cache复用共享前缀的KV Cache"), computed once for all the
// group's query rows instead of once per sequence.
//
// A workgroup takes one kv head of one group, 64 query rows (the group's
// (sequence, query head) pairs of that kv head, 16 per wave as the 16 MFMA
// columns) and one chunk of the prefix.  The four waves load each 16-token
// tile of the prefix together (a quarter each) and stage it once in LDS; the
// tiles go in pairs (double buffered, one barrier per pair), and every wave
// runs the grouped-query arithmetic on a pair at a time (scores, one online
// softmax update for its 32 tokens, weighted V sum) with its own 16 rows.
// The partial (max, sum, accumulator) of each row goes to the
// workspace slot of its chunk; the merge kernel combines the chunks with the
// partials of the rest of each context, which the decode kernels compute (for
// grouped-query heads in the same launch, after the prefix items).
#pragma once

#include "decode_gqa_kernel.h"

namespace pkv_dev {

constexpr int kMaxPrefixGroups = 32;
constexpr int kPrefixWaves = 4;  // 64 query rows per workgroup

struct PrefixArgs {
  DecodeArgs d;  // q, caches, scales, tables, workspace, shapes, scale, prefix_chunk
  int num_groups;
  int group_first[kMaxPrefixGroups];      // group g = sequences group_first[g] ..
  int group_count[kMaxPrefixGroups];      //           group_first[g] + group_count[g] - 1
  int group_prefix[kMaxPrefixGroups];     // tokens the group shares (multiple of max(bs, 16))
  int work_start[kMaxPrefixGroups + 1];   // first workgroup of each group
};

// LDS of one prefix workgroup: two buffers of two K tiles and two V tiles.
template <int KF, int QF, int D>
struct PrefixShared {
  static constexpr int kBytes = 2 * 2 * GqaTile<KF, QF, D>::kSlot;
};

// Prefix work item `item` (group, kv head, row tile, chunk), with `smem` the
// workgroup's PrefixShared bytes (16-byte aligned).  Every thread of the
// workgroup calls it.
template <int KF, int QF, int D, int BS>
__device__ __forceinline__ void prefix_body(const PrefixArgs& pa, int item, uint8_t* smem) {
  using T = GqaTile<KF, QF, D>;
  constexpr int NW = kPrefixWaves;
  constexpr bool kTwo = BS < kTileRows;
  constexpr int kTilesPerBlock = BS > kTileRows ? BS / kTileRows : 1;
  // Lanes of a wave that load: each wave loads 4 of the tile's 16 rows.
  constexpr int kLoadLanes = 4 * T::kSrcLanesPerRow;
  static_assert(kLoadLanes <= 64, "a quarter tile per wave in one load");
  const DecodeArgs& a = pa.d;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  // Group, then (kv head fastest: workgroup i runs on XCD i % 8, so with
  // num_kv_heads a multiple of 8 each kv head's prefix stays in one L2),
  // row tile and chunk.
  int grp = 0;
  while (grp + 1 < pa.num_groups && item >= pa.work_start[grp + 1]) ++grp;
  const int local = item - pa.work_start[grp];
  const int Hkv = a.num_kv_heads;
  const int G = a.num_heads / Hkv;
  const int first_seq = pa.group_first[grp];
  const int rows = pa.group_count[grp] * G;
  const int row_tiles = (rows + 16 * NW - 1) / (16 * NW);
  const int kvh = local % Hkv;
  const int rest = local / Hkv;
  const int rtile = rest % row_tiles;
  const int chunk = rest / row_tiles;
  const int c0 = chunk * a.prefix_chunk;
  const int c1 = min(c0 + a.prefix_chunk, pa.group_prefix[grp]);
  const int ntiles = c1 > c0 ? (c1 - c0) / kTileRows : 0;

  // Column t of this wave: query row r = (member, head) of the group.
  const int r = rtile * 16 * NW + wave * 16 + t;
  const bool rv = r < rows;
  const int seq = first_seq + (rv ? r / G : 0);
  const int hq = rv ? r % G : 0;
  u32x4_t qop[T::kSlices];
  {
    const int64_t qrow = (static_cast<int64_t>(seq) * a.num_heads + kvh * G + hq) * D;
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) + (qrow + 8 * g) * 2;
#pragma unroll
    for (int c = 0; c < T::kSlices; ++c) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qb + 64 * c);
      qop[c] = rv ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // The prefix blocks are those of the group's first sequence.  Lane k holds
  // the table entries (and int8/fp8 scales) of tile c0 / 16 + k.
  const int32_t* trow = a.block_tables + static_cast<int64_t>(first_seq) * a.max_blocks;
  int tb = -1, tb2 = -1;
  float tks = 1.f, tvs = 1.f, tks2 = 1.f, tvs2 = 1.f;
  if (lane < ntiles) {
    const int jj = c0 / kTileRows + lane;
    if constexpr (kTwo) {
      tb = trow[2 * jj];
      tb2 = trow[2 * jj + 1];
    } else {
      tb = trow[jj / kTilesPerBlock];
    }
    if (static_cast<unsigned>(tb) >= static_cast<unsigned>(a.num_blocks)) tb = -1;
    if (static_cast<unsigned>(tb2) >= static_cast<unsigned>(a.num_blocks)) tb2 = -1;
    if constexpr (scaled_format(KF)) {
      if (tb >= 0) {
        tks = a.k_scales[static_cast<int64_t>(tb) * Hkv + kvh];
        tvs = a.v_scales[static_cast<int64_t>(tb) * Hkv + kvh];
      }
      if (kTwo && tb2 >= 0) {
        tks2 = a.k_scales[static_cast<int64_t>(tb2) * Hkv + kvh];
        tvs2 = a.v_scales[static_cast<int64_t>(tb2) * Hkv + kvh];
      }
    }
  }

  // This lane's part of a tile: tile row 4 * wave + lane / lanes-per-row,
  // 16 source bytes at chunk lane % lanes-per-row.
  const int64_t row_stride = static_cast<int64_t>(Hkv) * T::kSrcRow;
  const int64_t blk_stride = row_stride * BS;
  const uint8_t* kbase = a.key_cache + static_cast<int64_t>(kvh) * T::kSrcRow;
  const uint8_t* vbase = a.value_cache + static_cast<int64_t>(kvh) * T::kSrcRow;
  const bool loads = lane < kLoadLanes;
  const int trow_in = 4 * wave + (loads ? lane / T::kSrcLanesPerRow : 0);
  const int tch = loads ? lane % T::kSrcLanesPerRow : 0;
  const uint32_t soff = static_cast<uint32_t>(trow_in * T::kPitchK + 16 * tch * (2 / T::kEB));
  const uint32_t voff = static_cast<uint32_t>(T::kTileK + trow_in * T::kPitchV + 16 * tch * (2 / T::kEB));
  auto src_offset = [&](int k) -> int64_t {
    const int jj = c0 / kTileRows + k;
    if constexpr (kTwo) {
      // tile rows 0..7 come from the first block, 8..15 from the second
      const int pa_ = __builtin_amdgcn_readlane(tb, k);
      const int pb_ = __builtin_amdgcn_readlane(tb2, k);
      const int p = trow_in < BS ? pa_ : pb_;
      return static_cast<int64_t>(p < 0 ? 0 : p) * blk_stride + (trow_in % BS) * row_stride + 16 * tch;
    } else {
      const int p = __builtin_amdgcn_readlane(tb, k);
      const int row0 = (jj % kTilesPerBlock) * kTileRows;
      return static_cast<int64_t>(p < 0 ? 0 : p) * blk_stride + (row0 + trow_in) * row_stride +
             16 * tch;
    }
  };
  // One tile's 16 source bytes of K and of V per loading lane.
  struct TileRegs {
    u32x4_t k, v;
  };
  auto load_tile = [&](TileRegs& r, int k) {
    if (loads) {
      const int64_t off = src_offset(k < ntiles ? k : ntiles - 1);  // clamped: no branch
      r.k = *reinterpret_cast<const u32x4_t*>(kbase + off);
      r.v = *reinterpret_cast<const u32x4_t*>(vbase + off);
    }
  };
  auto stage_tile = [&](uint8_t* tile, const TileRegs& r) {
    if (loads) {
      if constexpr (scaled_format(KF)) {
        const u32x2_t k0 = codes4_to_16<KF, QF>(r.k.x), k1 = codes4_to_16<KF, QF>(r.k.y);
        const u32x2_t k2 = codes4_to_16<KF, QF>(r.k.z), k3 = codes4_to_16<KF, QF>(r.k.w);
        const u32x2_t v0 = codes4_to_16<KF, QF>(r.v.x), v1 = codes4_to_16<KF, QF>(r.v.y);
        const u32x2_t v2 = codes4_to_16<KF, QF>(r.v.z), v3 = codes4_to_16<KF, QF>(r.v.w);
        *reinterpret_cast<u32x4_t*>(tile + soff) = u32x4_t{k0.x, k0.y, k1.x, k1.y};
        *reinterpret_cast<u32x4_t*>(tile + soff + 16) = u32x4_t{k2.x, k2.y, k3.x, k3.y};
        *reinterpret_cast<u32x4_t*>(tile + voff) = u32x4_t{v0.x, v0.y, v1.x, v1.y};
        *reinterpret_cast<u32x4_t*>(tile + voff + 16) = u32x4_t{v2.x, v2.y, v3.x, v3.y};
      } else {
        *reinterpret_cast<u32x4_t*>(tile + soff) = r.k;
        *reinterpret_cast<u32x4_t*>(tile + voff) = r.v;
      }
    }
  };

  GqaState<KF, QF, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < T::kTiles; ++c) st.acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Attended rows lo <= row < valid of tile k and its scales (as in the
  // grouped-query kernel); a tile past the chunk's end attends nothing.
  auto tile_params = [&](int k, int& lo, int& valid, float& ks, float& vs) {
    lo = 0;
    valid = kTileRows;
    ks = 1.f;
    vs = 1.f;
    if (k >= ntiles) {
      valid = 0;
      return;
    }
    const int p = __builtin_amdgcn_readlane(tb, k);
    ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tks), k));
    vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tvs), k));
    if constexpr (kTwo) {
      const int p2 = __builtin_amdgcn_readlane(tb2, k);
      if (p < 0) lo = BS;
      if (p2 < 0) valid = BS;
      if (4 * g >= BS) {
        ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tks2), k));
        vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tvs2), k));
      }
    } else {
      if (p < 0) valid = 0;
    }
  };
  // The tiles go in pairs (2j, 2j + 1), one softmax update per pair; an odd
  // count ends with a pair whose second tile attends nothing.  LDS holds two
  // pairs: pair j is computed from buffer j & 1 while pair j + 1 is staged in
  // the other one and pair j + 2 loads into registers (two tiles in flight).
  constexpr int kPairBytes = 2 * T::kSlot;
  auto compute_pair = [&](int j) {
    uint8_t* pair = smem + (j & 1) * kPairBytes;
    int loA, validA, loB, validB;
    float ksA, vsA, ksB, vsB;
    tile_params(2 * j, loA, validA, ksA, vsA);
    tile_params(2 * j + 1, loB, validB, ksB, vsB);
    gqa_compute_pair<KF, QF, D>(st, pair, pair + T::kSlot, qop, loA, validA, loB, validB, ksA,
                                vsA, ksB, vsB, t, g, a.scale_log2);
  };
  auto stage_pair = [&](int j, const TileRegs& ra, const TileRegs& rb) {
    uint8_t* pair = smem + (j & 1) * kPairBytes;
    stage_tile(pair, ra);
    stage_tile(pair + T::kSlot, rb);
  };

  if (ntiles > 0) {
    const int npairs = (ntiles + 1) / 2;
    TileRegs ra, rb;
    load_tile(ra, 0);
    load_tile(rb, 1);
    stage_pair(0, ra, rb);
    load_tile(ra, 2);
    load_tile(rb, 3);
    __syncthreads();
    for (int j = 0; j < npairs; ++j) {
      compute_pair(j);
      if (j + 1 < npairs) stage_pair(j + 1, ra, rb);
      load_tile(ra, 2 * j + 4);
      load_tile(rb, 2 * j + 5);
      __syncthreads();
    }
  }

  // Row r's partial for this chunk: lane (t, g) holds dims 16c + 4g + i.
  if (rv) {
    const int64_t sh = static_cast<int64_t>(seq) * a.num_heads + kvh * G + hq;
    const int64_t slot = sh * a.num_parts + chunk;
    float* acc = a.ws_acc + slot * D;
#pragma unroll
    for (int c = 0; c < T::kTiles; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[16 * c + 4 * g + i] = st.acc[c][i];
    if (g == 0) {
      a.ws_ml[slot * 2] = st.m;
      a.ws_ml[slot * 2 + 1] = st.l;
    }
  }
}

template <int KF, int QF, int D, int BS>
__global__ void __launch_bounds__(kPrefixWaves * 64) paged_prefix_kernel(PrefixArgs pa) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PrefixShared<KF, QF, D>::kBytes];
  prefix_body<KF, QF, D, BS>(pa, blockIdx.x, smem);
}

// Shared-prefix decode in one launch (grouped-query heads): the n_prefix
// prefix work items first, then the n_rest decode items of the rest of each
// context (pa.d, which writes partials for the merge kernel).  The rest items
// fill the CUs as the prefix items drain, so the tail of the compute-bound
// prefix work overlaps the memory-bound rest instead of waiting for a second
// launch.  (Dealing the two kinds in alternating runs measured slower at long
// prefixes: the rest items then compete with every prefix chunk.)
template <int KF, int QF, int D, bool SPLIT, int BS>
__global__ void __launch_bounds__(kPrefixWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
    paged_prefix_fused_kernel(PrefixArgs pa, int n_prefix) {
  static_assert(kPrefixWaves == 4, "both kinds run on four waves");
  constexpr int kP = PrefixShared<KF, QF, D>::kBytes;
  constexpr int kR = GqaShared<KF, QF, D, 4>::kBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kP > kR ? kP : kR];
  const int i = blockIdx.x;
  if (i < n_prefix)
    prefix_body<KF, QF, D, BS>(pa, i, smem);
  else
    gqa_decode_body<KF, QF, D, 4, SPLIT, BS>(pa.d, i - n_prefix, smem);
}

}  // namespace pkv_dev
