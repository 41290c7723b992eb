// Paged-attention decode kernels for gfx950 (CDNA4), templated on the cache
// format, the query format, head_dim and the query-head group size.
//
// Page keys:
//   [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com)
//   [P2] "大模型部署中KV Cache优化策略与显存管理实践教程" (yunthe.com)
//   [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn)
//
// What is computed ([P1] "PagedAttention注意力计算流程" and its kernel sketch):
// for a sequence's query head, token i of the context lives in physical block
// table[i / bs] at offset i % bs; its score is scale * dot(q, k_i); the output
// is the softmax-weighted sum of the v_i.  [P3] section 三 notes that the
// scattered rows are best walked block by block, reading each block's rows
// contiguously; that is what the wave loop below does.
//
// How it maps onto CDNA4 (this is not the sketch's one-thread-per-token shape):
//   * one workgroup of NW wave64s per (sequence, kv head, context partition);
//     with grouped-query attention the G query heads that share a kv head are
//     all handled by that workgroup, so each K/V row is read from HBM once;
//   * the waves of a workgroup take the partition's blocks round-robin; a wave
//     reads a block's K rows of its kv head with 16-byte loads, LPR lanes per
//     row (a 256-byte fp16 row of head_dim 128 is 16 lanes), RPI rows per load
//     instruction, IPB instructions per block of BS tokens, then the same for V
//     (one-byte rows of head_dim 64 are half a line: there a load row covers
//     two neighbouring kv heads, HR = 2, each lane working for one of them);
//   * each lane holds its E query elements (per head) in registers, the dot
//     product is finished by a DPP butterfly across the LPR lanes of a row;
//   * every row group of a wave (the lanes that share token rows) keeps its own
//     running softmax state (max, sum, E accumulators per head), so a block
//     needs no cross-row traffic at all; the row groups and waves are merged
//     exactly once at the end (shuffles, then LDS);
//   * exp is exp2 with log2(e) folded into the scale; masking is by select, so
//     slots past the context may hold anything (NaN included);
//   * a partition that does not hold the whole context writes (max, sum,
//     unnormalised accumulator) to the workspace and a second kernel merges
//     the partitions of each (sequence, head) with the same exact rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv_dev {

// Block sizes the kernels are built for ([P1] "PagedAttention分页内存管理原理"
// uses 16; 8 and 32 are the neighbours its block-size trade-off discusses).
__host__ __device__ constexpr bool supported_block_size(int bs) {
  return bs == 8 || bs == 16 || bs == 32;
}
// Partitions start at multiples of this many tokens: a whole block and a whole
// 16-token MFMA tile of the grouped-query kernel.
__host__ __device__ constexpr int partition_align(int bs) { return bs > 16 ? bs : 16; }

struct DecodeArgs {
  void* out;
  const void* q;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;   // [B*H][num_parts][2]: running max (log2 domain) and sum
  float* ws_acc;  // [B*H][num_parts][D]: unnormalised accumulators
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int max_blocks;
  int num_blocks;
  int block_size;   // tokens per block (the kernel's BS)
  int align;        // partition_align(block_size)
  int part_tokens;  // tokens per partition, a multiple of align
  int num_parts;    // partitions per sequence in the grid
  int window;       // sliding window in tokens, 0 = the whole context
  int heads_per_item;  // multi-head kernel: kv heads per workgroup (1, 2 or 4)
  // Multi-head kernel: > 0 deals the (at most 64) sequences to the grid's
  // sequence positions by context length in runs of balance_run ranks
  // (balanced_seq); 0 keeps the batch order.
  int balance_run;
  float scale_log2; // scale * log2(e)
  // Shared-prefix decode: the first prefix_lens[s] tokens of sequence s are
  // attended by the prefix kernel, which writes its partials to the first
  // part_base slots of each (sequence, head), prefix_chunk tokens per slot;
  // the decode kernels then take the remaining tokens and always write
  // partials, at slots part_base + p.  prefix_lens is NULL otherwise.
  const int32_t* prefix_lens;
  int part_base;
  int prefix_chunk;
  // Shared-prefix decode with one query head per kv head whose rest of every
  // context is one partition: the multi-head decode kernel merges the prefix
  // chunks itself and stores the output.
  int merge_prefix;
};

// The sequence that sequence position `pos` of the multi-head grid decodes
// when the batch is dealt by context length: ranked longest first (equal
// lengths by index), then taken in runs of a.balance_run ranks whose
// direction alternates.  With one round of workgroups, the items a compute
// unit holds together are C / g sequence positions apart (C compute units, g
// items per sequence, workgroups dealt round-robin); runs of that length give
// every CU long and short contexts alike instead of leaving some CUs all
// long ones.  `len` is sequence `lane`'s context length (lanes below
// a.num_seqs <= 64).  A batch of equal lengths keeps the batch order.  Every
// lane returns the same value.
__device__ __forceinline__ int balanced_seq(const DecodeArgs& a, int pos, int len) {
  const int lane = threadIdx.x & 63;
  const int n = a.num_seqs;
  const int cap = a.max_blocks * a.block_size;
  len = lane < n ? min(max(len, 0), cap) : -1;
  const int first = __builtin_amdgcn_readlane(len, 0);
  if (__ballot(lane < n && len != first) == 0) return pos;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const int run = a.balance_run;
  const int r0 = pos / run * run;
  const int off = pos - r0;
  const int target = ((pos / run) & 1) ? r0 + min(run, n - r0) - 1 - off : r0 + off;
  const uint64_t hit = __ballot(lane < n && rank == target);
  return hit ? static_cast<int>(__builtin_ctzll(hit)) : pos;
}

// The attended part of a sequence's context: its length clamped to the table,
// the first attended token (the last `window` tokens when a sliding window is
// set; the first token after the shared prefix in shared-prefix decode), the
// origin of its partitions (the first token rounded down to the partition
// alignment), the number of partitions that hold tokens, and the number of
// prefix-chunk partials written by the prefix kernel.  Partition p covers
// tokens origin + p * part_tokens onwards.
struct Span {
  int ctx;
  int first;
  int origin;
  int nparts;
  int nchunks;
};

__device__ __forceinline__ Span attended_span(const DecodeArgs& a, int seq) {
  const int cap = a.max_blocks * a.block_size;
  int ctx = a.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  int first = a.window > 0 ? max(0, ctx - a.window) : 0;
  int nchunks = 0;
  if (a.prefix_lens) {
    // at most the part_base chunk slots the workspace holds, whatever the
    // device value says (a value that disagrees with the groups gives a wrong
    // output, never a read outside the workspace)
    const int pl = min(min(max(a.prefix_lens[seq], 0), ctx), a.part_base * a.prefix_chunk);
    first = max(first, pl);
    nchunks = (pl + a.prefix_chunk - 1) / a.prefix_chunk;
  }
  const int origin = first / a.align * a.align;
  const int nparts = ctx > origin ? (ctx - origin + a.part_tokens - 1) / a.part_tokens : 0;
  return Span{ctx, first, origin, nparts, nchunks};
}

template <int F> struct Format;
template <> struct Format<PKV_F32> { static constexpr int kBytes = 4; };
template <> struct Format<PKV_F16> { static constexpr int kBytes = 2; };
template <> struct Format<PKV_BF16> { static constexpr int kBytes = 2; };
template <> struct Format<PKV_I8> { static constexpr int kBytes = 1; };
template <> struct Format<PKV_FP8> { static constexpr int kBytes = 1; };

// Formats whose codes carry a per-(block, kv head) scale.
__host__ __device__ constexpr bool scaled_format(int f) { return f == PKV_I8 || f == PKV_FP8; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// 16 bytes of storage -> 16 / kBytes floats (exact conversions).
template <int F> __device__ __forceinline__ void unpack16(const uint4& r, float* x);

template <> __device__ __forceinline__ void unpack16<PKV_F32>(const uint4& r, float* x) {
  x[0] = __uint_as_float(r.x);
  x[1] = __uint_as_float(r.y);
  x[2] = __uint_as_float(r.z);
  x[3] = __uint_as_float(r.w);
}

template <> __device__ __forceinline__ void unpack16<PKV_F16>(const uint4& r, float* x) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t h = __builtin_bit_cast(half2_t, w[i]);
    x[2 * i] = static_cast<float>(h.x);
    x[2 * i + 1] = static_cast<float>(h.y);
  }
}

template <> __device__ __forceinline__ void unpack16<PKV_BF16>(const uint4& r, float* x) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <> __device__ __forceinline__ void unpack16<PKV_I8>(const uint4& r, float* x) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[4 * i + j] = static_cast<float>(static_cast<int32_t>(w[i] << (24 - 8 * j)) >> 24);
  }
}

// FP8 E4M3 codes -> fp32 with the gfx950 conversion instruction (two codes
// per instruction; exact, every E4M3 value is an fp32 value).
typedef float float2_t __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ void unpack16<PKV_FP8>(const uint4& r, float* x) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
    const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    x[4 * i] = lo.x;
    x[4 * i + 1] = lo.y;
    x[4 * i + 2] = hi.x;
    x[4 * i + 3] = hi.y;
  }
}

// Round-to-nearest-even stores of an fp32 result in the query format.
template <int F> __device__ __forceinline__ void store_elem(void* base, int64_t idx, float v);
template <> __device__ __forceinline__ void store_elem<PKV_F32>(void* base, int64_t idx, float v) {
  static_cast<float*>(base)[idx] = v;
}
template <> __device__ __forceinline__ void store_elem<PKV_F16>(void* base, int64_t idx, float v) {
  static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(v);
}
template <> __device__ __forceinline__ void store_elem<PKV_BF16>(void* base, int64_t idx, float v) {
  uint32_t u = __float_as_uint(v);
  uint16_t b;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    b = 0x7FC0;  // NaN
  } else {
    u += 0x7FFFu + ((u >> 16) & 1u);
    b = static_cast<uint16_t>(u >> 16);
  }
  static_cast<uint16_t*>(base)[idx] = b;
}

// 16-byte load of cache data that is read once: the non-temporal hint keeps
// the stream from displacing reusable lines in the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// E query elements (E * kBytes is a multiple of 16) -> fp32.
template <int QF, int E>
__device__ __forceinline__ void load_q(const void* base, int64_t elem, float* x) {
  constexpr int kPer = 16 / Format<QF>::kBytes;
  static_assert(E % kPer == 0, "query fragment must be whole 16-byte vectors");
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) +
                                                  elem * Format<QF>::kBytes);
#pragma unroll
  for (int v = 0; v < E / kPer; ++v) unpack16<QF>(p[v], x + v * kPer);
}

// DPP row permutations (within 16-lane rows).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (result in every lane).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp<kDppQuadSwap1>(v);
  if constexpr (W >= 4) v += dpp<kDppQuadSwap2>(v);
  if constexpr (W >= 8) v += dpp<kDppRowHalfMirror>(v);
  if constexpr (W >= 16) v += dpp<kDppRowMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16);
  if constexpr (W >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Reduction over lanes that differ only in bits >= log2(FROM) (row groups).
template <int FROM>
__device__ __forceinline__ float across_groups_max(float v) {
#pragma unroll
  for (int off = FROM; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
template <int FROM>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int off = FROM; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// HR: neighbouring kv heads whose rows one load row covers (2 for one-byte
// rows of head_dim 64, so that a load row is a whole 128-byte line).
template <int KF, int QF, int D, int G, int NW, int BS, int HR = 1>
struct DecodeTile {
  static constexpr int kEB = Format<KF>::kBytes;
  static constexpr int kRow = HR * D * kEB;   // bytes of one load row (token, HR kv heads)
  static constexpr int kLPR = kRow / 16;      // lanes per row
  static constexpr int kLPH = kLPR / HR;      // lanes per head within a row
  static constexpr int kRPI = 64 / kLPR;      // rows per load instruction
  // Load instructions per block.  One-byte rows of head_dim 64 give 16 rows
  // per instruction, more than an 8-token block holds: the row groups past
  // the block then re-read the block's rows (rg % BS, so every load stays in
  // the block) and are masked like slots past the context.
  static constexpr int kIPB = kRPI <= BS ? BS / kRPI : 1;
  static constexpr int kE = 16 / kEB;         // elements per lane per load
  static constexpr bool kDupRows = kRPI > BS;
  static constexpr bool kBuilt = kDupRows ? kRPI % BS == 0 : BS % kRPI == 0;
  static_assert(kRow % 16 == 0 && kLPR >= 1 && kLPR <= 64 && 64 % kLPR == 0, "row shape");
};

// Per-lane running softmax state of one row group for G heads.
template <int G, int E>
struct SoftmaxState {
  float m[G];
  float l[G];
  float acc[G][E];
};

// Score, mask and accumulate NBLK blocks whose loads are issued together.
template <int KF, int QF, int D, int G, int NW, int BS, int HR, int NBLK>
__device__ __forceinline__ void process_blocks(
    SoftmaxState<G, DecodeTile<KF, QF, D, G, NW, BS, HR>::kE>& st,
    const float (&qf)[G][DecodeTile<KF, QF, D, G, NW, BS, HR>::kE], const uint8_t* kbase,
    const uint8_t* vbase, int64_t blk_stride, int64_t row_stride, const int (&phys)[NBLK],
    const int (&lo)[NBLK], const int (&valid)[NBLK], const float (&ksc)[NBLK],
    const float (&vsc)[NBLK], int rg, float scale_log2) {
  using T = DecodeTile<KF, QF, D, G, NW, BS, HR>;
  constexpr int E = T::kE, IPB = T::kIPB, RPI = T::kRPI, LPH = T::kLPH;
  uint4 kr[NBLK][IPB], vr[NBLK][IPB];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const uint8_t* kp = kbase + static_cast<int64_t>(phys[b]) * blk_stride;
#pragma unroll
    for (int i = 0; i < IPB; ++i)
      kr[b][i] = load_stream16(kp + static_cast<int64_t>(i * RPI) * row_stride);
  }
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const uint8_t* vp = vbase + static_cast<int64_t>(phys[b]) * blk_stride;
#pragma unroll
    for (int i = 0; i < IPB; ++i)
      vr[b][i] = load_stream16(vp + static_cast<int64_t>(i * RPI) * row_stride);
  }
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    float s[G][IPB];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      float kx[E];
      unpack16<KF>(kr[b][i], kx);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(qf[g][e], kx[e], d);
        s[g][i] = d;
      }
    }
    const float sc = scale_log2 * ksc[b];
    // tokens lo <= offset < valid of the block are attended (lo > 0 only in
    // the first block of a sliding window); offsets >= BS are the re-read
    // rows of T::kDupRows
    const bool partial = T::kDupRows || valid[b] < BS || lo[b] > 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        float v = group_sum<LPH>(s[g][i]) * sc;
        const int off = i * RPI + rg;
        if (partial && (off >= valid[b] || off < lo[b])) v = -INFINITY;
        s[g][i] = v;
      }
    }
    float vx[IPB][E];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      unpack16<KF>(vr[b][i], vx[i]);
      const int off = i * RPI + rg;
      if (partial && (off >= valid[b] || off < lo[b])) {
#pragma unroll
        for (int e = 0; e < E; ++e) vx[i][e] = 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = s[g][0];
#pragma unroll
      for (int i = 1; i < IPB; ++i) bm = fmaxf(bm, s[g][i]);
      const float mn = fmaxf(st.m[g], bm);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(st.m[g] - ms);
      float psum = 0.f;
      float p[IPB];
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        p[i] = fast_exp2(s[g][i] - ms);
        psum += p[i];
      }
      st.l[g] = st.l[g] * alpha + psum;
      st.m[g] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        const float pv = p[i] * vsc[b];
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[g][e] = fmaf(pv, vx[i][e], st.acc[g][e]);
      }
    }
  }
}

// Store the output of (sequence, head) row sh from this workgroup's partial
// (max m, sum l, accumulator o of dimension d, relative to m) merged with the
// nchunks prefix-chunk partials in the workspace.
template <int QF, int D>
__device__ __forceinline__ void store_merged_with_prefix(const DecodeArgs& a, int64_t sh, int d,
                                                         float m, float l, float o, int nchunks) {
  const float* ml = a.ws_ml + sh * a.num_parts * 2;
  const float* acc = a.ws_acc + sh * a.num_parts * D;
  float M = m;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, ml[2 * c]);
  const float ms = (M == -INFINITY) ? 0.f : M;
  const float f0 = fast_exp2(m - ms);
  float L = l * f0, O = o * f0;
  for (int c = 0; c < nchunks; ++c) {
    const float f = fast_exp2(ml[2 * c] - ms);
    L = fmaf(f, ml[2 * c + 1], L);
    O = fmaf(f, acc[static_cast<int64_t>(c) * D + d], O);
  }
  store_elem<QF>(a.out, sh * D + d, L > 0.f ? O / L : 0.f);
}

template <int KF, int QF, int D, int G, int NW, int BS, int HR = 1>
__global__ void __launch_bounds__(NW * 64) paged_decode_kernel(DecodeArgs a) {
  using T = DecodeTile<KF, QF, D, G, NW, BS, HR>;
  constexpr int E = T::kE, LPR = T::kLPR, LPH = T::kLPH;
  // Blocks whose loads are issued together: 32 tokens' worth.
  constexpr int UNROLL = BS >= 32 ? 1 : 32 / BS;
  const int part_blocks = a.part_tokens / BS;

  __shared__ float s_acc[NW][G][HR * D];
  __shared__ float s_m[NW][HR][G];
  __shared__ float s_l[NW][HR][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LPR;
  const int rg = lane / LPR;

  // Partition-major order: workgroup i runs on XCD i % 8, so consecutive ids
  // must carry comparable work.  With the (sequence, kv head) pair fastest,
  // each XCD sees every partition index and the same kv heads of every
  // sequence (shared prefix blocks of a kv head then meet in one L2), and
  // partitions past short contexts sit at the tail of the grid.
  //
  // A workgroup serves hpw neighbouring kv heads of one sequence and
  // partition: wave w takes kv head w % hpw and every (NW / hpw)-th block of
  // the partition from block w / hpw.  The heads' rows of a block are
  // adjacent in the cache, so one CU then reads hpw x head_dim x element
  // bytes of each token row at about the same time instead of one head's
  // 128 or 256 bytes.  With HR = 2 a wave's load rows cover two
  // neighbouring heads (the lanes of a row split between them), so the hpw
  // heads form hpw / 2 such pairs: wave w takes pair w % (hpw / 2).
  const int hpw = a.heads_per_item;
  const int vpw = hpw / HR;           // head groups (single heads or pairs) per workgroup
  const int wph = NW / vpw;
  const int hsub = wave % vpw;
  const int wslot = wave / vpw;
  const int item = blockIdx.x;
  const int gps = a.num_kv_heads / hpw;
  const int nsk = a.num_seqs * gps;
  const int part = item / nsk;
  const int sk = item - part * nsk;
  const int pos = sk / gps;           // sequence position in the grid
  const int kvh0 = (sk - pos * gps) * hpw;
  const int kvw = kvh0 + hsub * HR;   // the wave's first kv head
  const int lhead = sub / LPH;        // this lane's head within the load row
  const int kvh = kvw + lhead;        // this lane's kv head

  // Issued together, before the context length is known, so that the
  // prologue waits for one memory round trip instead of three: this wave's
  // first table entries of the partition (as many as a full table holds;
  // entries past the context are never used), the query, and the length.
  // With a sliding window (or after a shared prefix) the partitions start at
  // a token that depends on the length, so the table is read after it.
  const bool early_table = a.window == 0 && !a.prefix_lens;
  const int32_t* trow;
  int tb_first;
  float qf[G][E];
  Span sp;
  auto prologue = [&](int s) {
    trow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
    tb_first = -1;
    if (early_table) {
      const int pb0e = part * part_blocks;
      const int span_full = min(pb0e + part_blocks, a.max_blocks) - pb0e - wslot;
      const int nk_full = span_full > 0 ? (span_full + wph - 1) / wph : 0;
      if (lane < min(64, nk_full)) tb_first = trow[pb0e + wslot + wph * lane];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      load_q<QF, E>(a.q, (static_cast<int64_t>(s) * a.num_heads + h) * D + (sub % LPH) * E, qf[g]);
    }
    sp = attended_span(a, s);
  };
  // With the length-balanced order every sequence's length is read in the
  // same round trip as the prologue of the batch-order sequence `pos`, whose
  // loads stand when the order keeps it (equal lengths).
  int all_len = -1;
  if (a.balance_run > 0 && lane < a.num_seqs) all_len = a.context_lens[lane];
  int seq = pos;
  prologue(seq);
  if (a.balance_run > 0) {
    const int s = balanced_seq(a, pos, all_len);
    if (s != seq) {
      seq = s;
      prologue(seq);
    }
  }
  const int ctx = sp.ctx;
  if (part >= sp.nparts && part != 0) return;  // partition past the context
  const int pb0 = sp.origin / BS + part * part_blocks;
  const int pb1 = min(pb0 + part_blocks, (ctx + BS - 1) / BS);
  const bool direct = sp.nparts <= 1 && !a.prefix_lens;

  SoftmaxState<G, E> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[g][e] = 0.f;
  }

  constexpr int kHeadBytes = D * T::kEB;
  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * kHeadBytes;
  const int64_t blk_stride = row_stride * BS;
  const int row = T::kDupRows ? rg % BS : rg;
  const int64_t lane_off = static_cast<int64_t>(kvw) * kHeadBytes + sub * 16 + row * row_stride;
  const uint8_t* kbase = a.key_cache + lane_off;
  const uint8_t* vbase = a.value_cache + lane_off;

  // Blocks of this wave: pb0 + wslot + wph * k for k < nk.
  const int span = pb1 - pb0 - wslot;
  const int nk = span > 0 ? (span + wph - 1) / wph : 0;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int kk = k0 + lane;
    int tb = -1;
    // scales of table entry kk for the wave's HR heads (broadcast below,
    // then each lane takes its own head's)
    float tks[HR], tvs[HR];
#pragma unroll
    for (int r = 0; r < HR; ++r) tks[r] = tvs[r] = 1.f;
    if (kk < nk) {
      tb = (k0 == 0 && early_table) ? tb_first : trow[pb0 + wslot + wph * kk];
      if (static_cast<unsigned>(tb) >= static_cast<unsigned>(a.num_blocks)) tb = -1;
      if constexpr (scaled_format(KF)) {
        if (tb >= 0) {
#pragma unroll
          for (int r = 0; r < HR; ++r) {
            tks[r] = a.k_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvw + r];
            tvs[r] = a.v_scales[static_cast<int64_t>(tb) * a.num_kv_heads + kvw + r];
          }
        }
      }
    }
    auto bcast = [&](const float (&v)[HR], int from) {
      float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), from));
      if constexpr (HR == 2) {
        const float y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[1]), from));
        x = lhead ? y : x;
      }
      return x;
    };
    const int kend = min(64, nk - k0);
    int k = 0;
    for (; k + UNROLL <= kend; k += UNROLL) {
      int phys[UNROLL], lo[UNROLL], valid[UNROLL];
      float ks[UNROLL], vs[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int p = __builtin_amdgcn_readlane(tb, k + u);
        const int j = pb0 + wslot + wph * (k0 + k + u);
        phys[u] = p < 0 ? 0 : p;
        lo[u] = max(0, sp.first - j * BS);
        valid[u] = p < 0 ? 0 : min(BS, ctx - j * BS);
        ks[u] = bcast(tks, k + u);
        vs[u] = bcast(tvs, k + u);
      }
      process_blocks<KF, QF, D, G, NW, BS, HR, UNROLL>(st, qf, kbase, vbase, blk_stride, row_stride,
                                                   phys, lo, valid, ks, vs, rg, a.scale_log2);
    }
    for (; k < kend; ++k) {
      const int p = __builtin_amdgcn_readlane(tb, k);
      const int j = pb0 + wslot + wph * (k0 + k);
      int phys[1] = {p < 0 ? 0 : p};
      int lo[1] = {max(0, sp.first - j * BS)};
      int valid[1] = {p < 0 ? 0 : min(BS, ctx - j * BS)};
      float ks[1] = {bcast(tks, k)};
      float vs[1] = {bcast(tvs, k)};
      process_blocks<KF, QF, D, G, NW, BS, HR, 1>(st, qf, kbase, vbase, blk_stride, row_stride, phys,
                                              lo, valid, ks, vs, rg, a.scale_log2);
    }
  }

  // Merge the row groups of this wave (exact rescaling to a common max).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = across_groups_max<LPR>(st.m[g]);
    const float f = fast_exp2(st.m[g] - (M == -INFINITY ? 0.f : M));
    st.l[g] = across_groups_sum<LPR>(st.l[g] * f);
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[g][e] = across_groups_sum<LPR>(st.acc[g][e] * f);
    st.m[g] = M;
  }
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][g][sub * E + e] = st.acc[g][e];
  }
  if (rg == 0 && sub % LPH == 0) {   // the first lane of each head in the row
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[wave][lhead][g] = st.m[g];
      s_l[wave][lhead][g] = st.l[g];
    }
  }
  __syncthreads();

  // Merge the waves of each kv head (head slot hs is half hs % HR of the
  // waves hs / HR, hs / HR + vpw, ...) and write the result (or this
  // partition's partial).
  for (int idx = threadIdx.x; idx < hpw * G * D; idx += NW * 64) {
    const int hs = idx / (G * D);
    const int g = (idx / D) % G;
    const int d = idx % D;
    const int hw = hs / HR, half = hs % HR;
    float M = s_m[hw][half][g];
    for (int w = hw + vpw; w < NW; w += vpw) M = fmaxf(M, s_m[w][half][g]);
    const float ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
    for (int w = hw; w < NW; w += vpw) {
      const float f = fast_exp2(s_m[w][half][g] - ms);
      L = fmaf(f, s_l[w][half][g], L);
      O = fmaf(f, s_acc[w][g][half * D + d], O);
    }
    const int h = (kvh0 + hs) * G + g;
    const int64_t sh = static_cast<int64_t>(seq) * a.num_heads + h;
    if (direct) {
      store_elem<QF>(a.out, sh * D + d, L > 0.f ? O / L : 0.f);
    } else if (a.merge_prefix) {
      store_merged_with_prefix<QF, D>(a, sh, d, M, L, O, sp.nchunks);
    } else {
      const int64_t slot = sh * a.num_parts + a.part_base + part;
      a.ws_acc[slot * D + d] = O;
      if (d == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Merge the partitions of each (sequence, head): one wave per row, kMergeRows
// rows per workgroup.  The lanes read the partials' (max, sum) pairs together
// and two wave reductions give the common exponent base and the sum; then
// every lane sums its D / 64 dims of the accumulators, issuing the loads of
// four partials at a time.
constexpr int kMergeRows = 4;

template <int QF, int D>
__global__ void __launch_bounds__(kMergeRows * 64) paged_decode_reduce_kernel(DecodeArgs a) {
  static_assert(D % 64 == 0, "head_dim must be a multiple of the wave");
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * kMergeRows + (threadIdx.x >> 6);
  if (sh >= static_cast<int64_t>(a.num_seqs) * a.num_heads) return;  // seq * num_heads + head
  const int seq = static_cast<int>(sh / a.num_heads);
  const Span sp = attended_span(a, seq);
  // The partials to merge: the prefix chunks (slots 0 .. nchunks - 1) and the
  // partitions of the rest (slots part_base .. part_base + nparts - 1).
  if (!a.prefix_lens && sp.nparts <= 1) return;  // the decode kernel wrote this output
  const float* ml = a.ws_ml + sh * a.num_parts * 2;
  const float* acc = a.ws_acc + sh * a.num_parts * D;
  auto slot_of = [&](int i) { return i < sp.nchunks ? i : a.part_base + (i - sp.nchunks); };
  const int n = sp.nchunks + sp.nparts;

  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, ml[2 * slot_of(i)]);
  M = across_groups_max<1>(M);
  const float ms = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  for (int i = lane; i < n; i += 64) {
    const int p = slot_of(i);
    L = fmaf(fast_exp2(ml[2 * p] - ms), ml[2 * p + 1], L);
  }
  L = across_groups_sum<1>(L);

  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  constexpr int U = 4;
  int i = 0;
  for (; i + U <= n; i += U) {
    float f[U], x[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = slot_of(i + u);
      f[u] = ml[2 * p];
#pragma unroll
      for (int e = 0; e < E; ++e) x[u][e] = acc[static_cast<int64_t>(p) * D + 64 * e + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = fast_exp2(f[u] - ms);
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] = fmaf(w, x[u][e], O[e]);
    }
  }
  for (; i < n; ++i) {
    const int p = slot_of(i);
    const float w = fast_exp2(ml[2 * p] - ms);
#pragma unroll
    for (int e = 0; e < E; ++e) O[e] = fmaf(w, acc[static_cast<int64_t>(p) * D + 64 * e + lane], O[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) store_elem<QF>(a.out, sh * D + 64 * e + lane, L > 0.f ? O[e] / L : 0.f);
}

}  // namespace pkv_dev
