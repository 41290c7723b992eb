// Host side of pkv_paged_attention_decode: argument checks, the partition
// policy, the workspace contract and the two launches (decode, then the merge
// of partitions when the context is split).
#include <cmath>

#include "decode_dispatch.h"
#include "pkv_internal.h"

namespace pkv_dev {

template <int QF>
hipError_t launch_reduce(int head_dim, const DecodeArgs& a, unsigned grid, hipStream_t s) {
  if (head_dim == 64)
    hipLaunchKernelGGL((paged_decode_reduce_kernel<QF, 64>), dim3(grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((paged_decode_reduce_kernel<QF, 128>), dim3(grid), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv_dev

namespace {

// Automatic partitioning (measured on MI355X with the standard workloads at
// block size 16): a context of up to kWholeTokens tokens is handled by one
// workgroup per (sequence, kv head); longer ones are split into partitions of
// kSplitTokens tokens, so a few long sequences among short ones do not leave a
// tail of long-running workgroups.  Independently, the grid is split further
// until it has at least kMinItems workgroups (two per CU), so small batches
// still fill the chip.  Partitions are whole multiples of
// partition_align(block_size) tokens.
constexpr int64_t kWholeTokens = 2560;
constexpr int64_t kSplitTokens = 1024;
constexpr int64_t kMinItems = 512;

// Tokens a context can span from its partition origin: the whole table, or
// with a sliding window of W tokens at most W plus the rounding of the origin
// down to the partition alignment; rounded up to whole alignment units.
int64_t attended_tokens(int max_blocks, int block_size, int window) {
  const int64_t u = pkv_dev::partition_align(block_size);
  int64_t span = static_cast<int64_t>(max_blocks) * block_size;
  if (window > 0 && window + u - 1 < span) span = window + u - 1;
  return (span + u - 1) / u * u;
}

// Tokens per partition (equal to span when the context is not split), or -1
// for an invalid request.  partition_size = 0 picks automatically.
int64_t partition_tokens(int num_seqs, int num_kv_heads, int64_t span, int block_size,
                         int partition_size) {
  const int64_t u = pkv_dev::partition_align(block_size);
  if (span <= 0 || partition_size < 0) return -1;
  if (partition_size > 0) {
    if (partition_size % u) return -1;
    return partition_size >= span ? span : partition_size;
  }
  int64_t pt = span > kWholeTokens ? kSplitTokens : span;
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (pairs > 0 && pairs * ((span + pt - 1) / pt) < kMinItems) {
    const int64_t parts = (kMinItems + pairs - 1) / pairs;
    pt = ((span + parts - 1) / parts + u - 1) / u * u;
  }
  return pt < u ? u : (pt > span ? span : pt);
}

bool shapes_ok(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks) {
  return num_seqs >= 0 && num_heads > 0 && num_kv_heads > 0 && num_heads % num_kv_heads == 0 &&
         head_dim > 0 && block_size > 0 && max_blocks > 0;
}

}  // namespace

extern "C" {

int pkv_decode_partition_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int max_blocks_per_seq, int partition_size,
                              int sliding_window) {
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      sliding_window < 0 || !pkv_dev::supported_block_size(block_size) ||
      static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX / 2)
    return 0;
  const int64_t span = attended_tokens(max_blocks_per_seq, block_size, sliding_window);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size);
  if (pt <= 0 || pt >= span) return 0;
  return static_cast<int>(pt);
}

size_t pkv_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int partition_size,
                                 int sliding_window) {
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      sliding_window < 0 || !pkv_dev::supported_block_size(block_size) ||
      static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX / 2)
    return 0;
  const int64_t span = attended_tokens(max_blocks_per_seq, block_size, sliding_window);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size);
  if (pt <= 0 || pt >= span) return 0;
  const size_t parts = static_cast<size_t>((span + pt - 1) / pt);
  return static_cast<size_t>(num_seqs) * num_heads * parts * (head_dim + 2) * sizeof(float);
}

int pkv_paged_attention_decode(void* out, const void* q, const void* key_cache,
                               const void* value_cache, const float* k_scales,
                               const float* v_scales, const int32_t* block_tables,
                               const int32_t* context_lens, int num_seqs, int num_heads,
                               int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int num_blocks, float scale, int q_dtype,
                               int kv_dtype, int partition_size, int sliding_window,
                               void* workspace, size_t workspace_bytes, void* stream) {
  PKV_API_BEGIN
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "bad shape: seqs=%d heads=%d kv_heads=%d head_dim=%d block_size=%d "
                     "max_blocks=%d num_blocks=%d",
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  const bool float_pair = (kv_dtype == PKV_F32 && q_dtype == PKV_F32) ||
                          (kv_dtype == PKV_F16 && q_dtype == PKV_F16) ||
                          (kv_dtype == PKV_BF16 && q_dtype == PKV_BF16);
  const bool scaled_pair = (kv_dtype == PKV_I8 || kv_dtype == PKV_FP8) &&
                           (q_dtype == PKV_F16 || q_dtype == PKV_BF16);
  if (!float_pair && !scaled_pair)
    return pkv::fail(PKV_ERR_INVALID_ARG, "unsupported format pair q=%d kv=%d", q_dtype, kv_dtype);
  if (scaled_pair && (!k_scales || !v_scales))
    return pkv::fail(PKV_ERR_INVALID_ARG, "int8 and fp8 caches need k_scales and v_scales");
  if (head_dim != 64 && head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", head_dim);
  const int group = num_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "query heads per kv head %d (1, 2, 4, 8, 16)", group);
  if (!std::isfinite(scale)) return pkv::fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX / 2)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  if (sliding_window < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "sliding_window %d is negative", sliding_window);
  if (!pkv_dev::supported_block_size(block_size))
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d (8, 16 or 32)", block_size);
  const int64_t span = attended_tokens(max_blocks_per_seq, block_size, sliding_window);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size);
  if (pt <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "partition_size %d is not a multiple of %d tokens",
                     partition_size, pkv_dev::partition_align(block_size));
  const int parts = static_cast<int>((span + pt - 1) / pt);
  const size_t need =
      pkv_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, partition_size, sliding_window);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return pkv::fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                     workspace_bytes, workspace ? "" : ", NULL");
  // The kernels address one block's rows of a kv head with 32-bit offsets.
  if (static_cast<int64_t>(num_kv_heads) * head_dim * pkv::elem_bytes(kv_dtype) * block_size >
      INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "a cache block is larger than 2 GiB");
  const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * parts;
  if (items > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "grid too large");

  pkv_dev::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.key_cache = static_cast<const uint8_t*>(key_cache);
  a.value_cache = static_cast<const uint8_t*>(value_cache);
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  float* ws = static_cast<float*>(workspace);
  const size_t slots = static_cast<size_t>(num_seqs) * num_heads * parts;
  a.ws_ml = need ? ws : nullptr;
  a.ws_acc = need ? ws + 2 * slots : nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.align = pkv_dev::partition_align(block_size);
  a.part_tokens = static_cast<int>(pt);
  a.num_parts = parts;
  a.window = sliding_window;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok = false;
  hipError_t err = hipSuccess;
  const unsigned grid = static_cast<unsigned>(items);
  switch (kv_dtype) {
    case PKV_F32: err = pkv_dev::launch_decode_f32(q_dtype, head_dim, group, a, grid, s, ok); break;
    case PKV_F16: err = pkv_dev::launch_decode_f16(q_dtype, head_dim, group, a, grid, s, ok); break;
    case PKV_BF16: err = pkv_dev::launch_decode_bf16(q_dtype, head_dim, group, a, grid, s, ok); break;
    case PKV_I8: err = pkv_dev::launch_decode_i8(q_dtype, head_dim, group, a, grid, s, ok); break;
    case PKV_FP8: err = pkv_dev::launch_decode_fp8(q_dtype, head_dim, group, a, grid, s, ok); break;
    default: break;
  }
  if (!ok) return pkv::fail(PKV_ERR_UNSUPPORTED, "no kernel for this combination");
  if (err != hipSuccess)
    return pkv::fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
  if (parts > 1) {
    const unsigned rgrid = static_cast<unsigned>(static_cast<int64_t>(num_seqs) * num_heads);
    switch (q_dtype) {
      case PKV_F32: err = pkv_dev::launch_reduce<PKV_F32>(head_dim, a, rgrid, s); break;
      case PKV_F16: err = pkv_dev::launch_reduce<PKV_F16>(head_dim, a, rgrid, s); break;
      default: err = pkv_dev::launch_reduce<PKV_BF16>(head_dim, a, rgrid, s); break;
    }
    if (err != hipSuccess)
      return pkv::fail(PKV_ERR_HIP, "partition merge launch: %s", hipGetErrorString(err));
  }
  return PKV_OK;
  PKV_API_END
}

}  // extern "C"
