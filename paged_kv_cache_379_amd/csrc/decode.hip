// Host side of pkv_paged_attention_decode: argument checks, the partition
// policy, the workspace contract and the two launches (decode, then the merge
// of partitions when the context is split).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "decode_dispatch.h"
#include "pkv_internal.h"

namespace pkv_dev {

// rows: num_seqs * num_heads, kMergeRows per workgroup.
template <int QF>
hipError_t launch_reduce(int head_dim, const DecodeArgs& a, int64_t rows, hipStream_t s) {
  if ((rows + kMergeRows - 1) / kMergeRows > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>((rows + kMergeRows - 1) / kMergeRows));
  const dim3 block(kMergeRows * 64);
  if (head_dim == 64)
    hipLaunchKernelGGL((paged_decode_reduce_kernel<QF, 64>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((paged_decode_reduce_kernel<QF, 128>), grid, block, 0, s, a);
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
// still fill the chip, but not into partitions shorter than span / 32
// (clamped to kMinPartTokens .. kMaxFloorTokens): each partition adds a
// partial to write and merge and the merge is a second launch, so a few
// (sequence, kv head) pairs do best with a few dozen partitions of at least
// 128 tokens, and a table of at most 128 tokens stays whole.  Measured on
// MI355X with 8 pairs (HIP events, cold caches; automatic before this floor
// -> with it): 112 tokens 12.4 -> 8.2 us, 1024 tokens 17.2 -> 12.7, 2048
// 17.5 -> 13.5, 4096 18.6 -> 16.0, 16384 27.0 -> 23.4, 32768 37.3 -> 33.3.
// Partitions are whole multiples of partition_align(block_size) tokens.
constexpr int64_t kWholeTokens = 2560;
constexpr int64_t kSplitTokens = 1024;
constexpr int64_t kMinItems = 512;
constexpr int64_t kMinPartTokens = 128;
constexpr int64_t kMaxFloorTokens = 1024;
// With a sliding window every context longer than the window attends exactly
// the window, so whole windows give equal workgroups and no tail to split
// away; the grid is then split only below one workgroup per CU.  Measured on
// MI355X (32 sequences of 4096-16384 tokens, window 4096, 8 kv heads x 4
// query heads, bf16): 101.3 us with 1024-token partitions (about 1024 real
// workgroups against the 768 that fit at once), 93.8 with 2048, 89.1 with
// 4096 (plus a merge of the <= 15-token remainder).
constexpr int64_t kMinWindowItems = 256;

// kv heads per workgroup of the multi-head kernel (one query head per kv
// head): neighbouring heads read together stream faster, while fewer
// workgroups leave CUs idle once the grid drops below the 1024 slots (four
// per CU) the kernel fills.  Measured on MI355X (32 sequences x 64 heads,
// 2048 tokens): fp16 345.7 / 335.9 / 338.5 us and FP8 195.0 / 182.1 / 172.1
// us at 1 / 2 / 4 heads; 32 sequences x 32 heads (1024 workgroups), fp16:
// 98.2 / 107.1 / 113.7 us.  So: up to two heads for 16-bit caches and four
// for one-byte caches, as long as the grid keeps 1024 (16-bit) or 512
// (one-byte) workgroups.  fp32 rows already span 512 bytes per head.
int mha_heads_per_item(int num_seqs, int num_heads, int num_kv_heads, int parts, int kv_dtype) {
  if (num_heads != num_kv_heads) return 1;
  const int eb = pkv::elem_bytes(kv_dtype);
  if (eb > 2) return 1;
  const int64_t min_items = eb == 1 ? 512 : 1024;
  for (int h = eb == 1 ? 4 : 2; h > 1; h /= 2) {
    if (num_kv_heads % h == 0 &&
        static_cast<int64_t>(num_seqs) * (num_kv_heads / h) * parts >= min_items)
      return h;
  }
  return 1;
}

// Compute units of the current device (cached per device), 0 if unknown.
int device_cus() {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The multi-head kernel's plan: kv heads per workgroup and the run of the
// length-balanced sequence order (balanced_seq; 0 keeps the batch order).
// The order applies to batches of 2..64 sequences with whole contexts (one
// partition) of tables spanning at least kBalanceMinTokens tokens, whose grid
// is one round of workgroups (at least one and at most four per CU);
// its runs are the C / g sequence positions between the items one CU holds
// (C compute units, g workgroups per sequence).  With the order in place two
// heads per workgroup pay off down to one workgroup per CU.  Measured on
// MI355X with the 7B-like layer (32 sequences x 32 heads, fp16, uniform
// 128..2048-token contexts): one head per workgroup 100.9-101.3 us and two
// heads 108.6-109.1 us in batch order, two heads balanced 93.9 us (order
// from the host; computed in the kernel it also reads every length before
// the sequence's own loads); at uniform lengths two heads are faster as well
// (1088 tokens: 93.4-94.5 against 95.9-97.0 us; 2048: 167.6-168.3 against
// 173.5-174.4).  Short tables gain nothing: 32 x 32 heads of uniform 1..256 /
// 1..512 / 1..1024 tokens took 20.2-20.3 / 30.3-31.0 / 51.2-52.1 us with the
// order and two heads against 19.0-19.1 / 29.8-29.9 / 51.1-51.3 without.
constexpr int64_t kBalanceMinTokens = 1024;

struct MhaPlan {
  int hpi;
  int run;
};

MhaPlan mha_plan(int num_seqs, int num_heads, int num_kv_heads, int parts, int kv_dtype,
                 int64_t span) {
  MhaPlan p{mha_heads_per_item(num_seqs, num_heads, num_kv_heads, parts, kv_dtype), 0};
  if (parts != 1 || num_seqs < 2 || num_seqs > 64 || span < kBalanceMinTokens) return p;
  const int cus = device_cus();
  if (cus <= 0) return p;
  auto one_round = [&](int h) {
    const int64_t items = static_cast<int64_t>(num_seqs) * (num_kv_heads / h);
    return items >= cus && items <= 4 * static_cast<int64_t>(cus);
  };
  if (p.hpi == 1 && num_heads == num_kv_heads && pkv::elem_bytes(kv_dtype) == 2 &&
      num_kv_heads % 2 == 0 && static_cast<int64_t>(num_seqs) * (num_kv_heads / 2) >= cus &&
      one_round(2))
    p.hpi = 2;
  if (one_round(p.hpi)) p.run = std::max(1, cus / (num_kv_heads / p.hpi));
  return p;
}

// Tokens a context can span from its partition origin: the whole table, or
// with a sliding window of W tokens at most W plus the rounding of the origin
// down to the partition alignment; rounded up to whole alignment units.
int64_t attended_tokens(int max_blocks, int block_size, int window) {
  const int64_t u = pkv_dev::partition_align(block_size);
  int64_t span = static_cast<int64_t>(max_blocks) * block_size;
  if (window > 0 && window + u - 1 < span) span = window + u - 1;
  return (span + u - 1) / u * u;
}

// Whether a sliding window bounds what a context attends (the table holds
// more than the window).
bool window_binds(int max_blocks, int block_size, int window) {
  return window > 0 && static_cast<int64_t>(window) < static_cast<int64_t>(max_blocks) * block_size;
}

// Tokens per partition (equal to span when the context is not split), or -1
// for an invalid request.  partition_size = 0 picks automatically; windowed
// is window_binds() of the request.
int64_t partition_tokens(int num_seqs, int num_kv_heads, int64_t span, int block_size,
                         int partition_size, bool windowed) {
  const int64_t u = pkv_dev::partition_align(block_size);
  if (span <= 0 || partition_size < 0) return -1;
  if (partition_size > 0) {
    if (partition_size % u) return -1;
    return partition_size >= span ? span : partition_size;
  }
  int64_t pt = windowed || span <= kWholeTokens ? span : kSplitTokens;
  const int64_t min_items = windowed ? kMinWindowItems : kMinItems;
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (pairs > 0 && pairs * ((span + pt - 1) / pt) < min_items) {
    const int64_t parts = (min_items + pairs - 1) / pairs;
    const int64_t floor_tokens = std::min(std::max(span / 32, kMinPartTokens), kMaxFloorTokens);
    pt = std::max((span + parts - 1) / parts, floor_tokens);
    pt = (pt + u - 1) / u * u;
  }
  return pt < u ? u : (pt > span ? span : pt);
}

bool shapes_ok(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks) {
  return num_seqs >= 0 && num_heads > 0 && num_kv_heads > 0 && num_heads % num_kv_heads == 0 &&
         head_dim > 0 && block_size > 0 && max_blocks > 0;
}

// Checks shared by the decode entry points, for a non-empty batch whose
// shapes passed shapes_ok.
int check_decode(const void* out, const void* q, const void* key_cache, const void* value_cache,
                 const float* k_scales, const float* v_scales, const int32_t* block_tables,
                 const int32_t* context_lens, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int max_blocks_per_seq, int kv_dtype, int q_dtype, float scale,
                 int sliding_window) {
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
  // The kernels address one block's rows of a kv head with 32-bit offsets.
  if (static_cast<int64_t>(num_kv_heads) * head_dim * pkv::elem_bytes(kv_dtype) * block_size >
      INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "a cache block is larger than 2 GiB");
  return PKV_OK;
}

// Shared-prefix decode: prefix chunks of kMaxChunkTokens tokens, halved (down
// to kMinChunkTokens) until the prefix work has kMinPrefixItems workgroups.
// The decode items of the rest of each context share the launch and fill the
// chip as the prefix items drain, so the prefix needs fewer workgroups than a
// decode of its own; every chunk also adds a partial per (sequence, head) to
// write and merge.  Measured on MI355X (64 sequences, 8 kv heads x 8 query
// heads, 2000-token prefix): 43 us at 256 workgroups against 48.5 at 512 and
// 60 at 128; longer prefixes are not sensitive to it.
constexpr int kMaxChunkTokens = 1024;  // at most 64 tiles: one table entry per lane
constexpr int kMinChunkTokens = 128;
constexpr int64_t kMinPrefixItems = 256;

struct PrefixPlan {
  int chunk;        // tokens per prefix chunk
  int max_chunks;   // chunks of the longest prefix: the slots before the rest's partitions
  int parts;        // partitions of the rest of each context
  int part_tokens;  // tokens per partition of the rest
  int work_start[pkv_dev::kMaxPrefixGroups + 1];
};

int plan_prefix(int num_seqs, int num_heads, int num_kv_heads, int block_size, int max_blocks,
                const int32_t* groups, int num_groups, PrefixPlan* plan) {
  if (num_groups < 1 || num_groups > pkv_dev::kMaxPrefixGroups)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_groups %d (1 .. %d)", num_groups,
                     pkv_dev::kMaxPrefixGroups);
  if (!groups) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL groups");
  const int u = pkv_dev::partition_align(block_size);
  const int64_t cap = static_cast<int64_t>(max_blocks) * block_size;
  std::vector<char> taken(num_seqs, 0);
  for (int g = 0; g < num_groups; ++g) {
    const int first = groups[3 * g], n = groups[3 * g + 1], prefix = groups[3 * g + 2];
    if (first < 0 || n < 1 || static_cast<int64_t>(first) + n > num_seqs)
      return pkv::fail(PKV_ERR_INVALID_ARG, "group %d (%d, %d) outside the %d sequences", g, first,
                       n, num_seqs);
    for (int s = first; s < first + n; ++s) {
      if (taken[s]) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is in two groups", s);
      taken[s] = 1;
    }
    if (prefix <= 0 || prefix % u || prefix > cap)
      return pkv::fail(PKV_ERR_INVALID_ARG, "group %d prefix %d must be a positive multiple of %d "
                       "tokens, at most %lld", g, prefix, u, static_cast<long long>(cap));
  }
  const int G = num_heads / num_kv_heads;
  auto work = [&](int chunk, int* starts) {
    int64_t w = 0;
    for (int g = 0; g < num_groups; ++g) {
      if (starts) starts[g] = static_cast<int>(w);
      const int64_t rows = static_cast<int64_t>(groups[3 * g + 1]) * G;
      const int64_t tiles = (rows + 64 - 1) / 64;
      w += static_cast<int64_t>(num_kv_heads) * tiles * ((groups[3 * g + 2] + chunk - 1) / chunk);
    }
    if (starts) starts[num_groups] = static_cast<int>(w);
    return w;
  };
  int chunk = kMaxChunkTokens;
  while (work(chunk, nullptr) < kMinPrefixItems && chunk / 2 >= kMinChunkTokens &&
         (chunk / 2) % u == 0)
    chunk /= 2;
  if (chunk % u) chunk = u;  // 32-token blocks with 1024: stays a multiple
  const int64_t total = work(chunk, plan->work_start);
  if (total > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "prefix grid too large");
  int max_chunks = 0;
  for (int g = 0; g < num_groups; ++g)
    max_chunks = std::max(max_chunks, (groups[3 * g + 2] + chunk - 1) / chunk);
  const int64_t span = attended_tokens(max_blocks, block_size, 0);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, 0, false);
  plan->chunk = chunk;
  plan->max_chunks = max_chunks;
  plan->part_tokens = static_cast<int>(pt);
  plan->parts = static_cast<int>((span + pt - 1) / pt);
  return PKV_OK;
}

// Scratch of pkv_paged_attention_decode_noalloc: the split-context partials
// for callers that cannot allocate device memory.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddress {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddress g_scratch[kMaxDevices];

// Device address of the current device's scratch, or NULL (with *err set).
void* scratch_address(int* device, hipError_t* err) {
  *err = hipGetDevice(device);
  if (*err != hipSuccess) return nullptr;
  if (*device < 0 || *device >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchAddress& slot = g_scratch[*device];
  std::call_once(slot.once, [&slot] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    slot.ptr = slot.err == hipSuccess ? p : nullptr;
  });
  *err = slot.err;
  return slot.ptr;
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
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size,
                                      window_binds(max_blocks_per_seq, block_size, sliding_window));
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
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size,
                                      window_binds(max_blocks_per_seq, block_size, sliding_window));
  if (pt <= 0 || pt >= span) return 0;
  const size_t parts = static_cast<size_t>((span + pt - 1) / pt);
  return static_cast<size_t>(num_seqs) * num_heads * parts * (head_dim + 2) * sizeof(float);
}

int pkv_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int partition_size, int sliding_window, int kv_dtype,
                    int* plan) {
  PKV_API_BEGIN
  if (!plan) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL plan");
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      num_seqs == 0 || sliding_window < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad shape");
  if (!pkv_dev::supported_block_size(block_size))
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d (8, 16 or 32)", block_size);
  if (kv_dtype < PKV_F32 || kv_dtype > PKV_FP8)
    return pkv::fail(PKV_ERR_INVALID_ARG, "kv_dtype %d", kv_dtype);
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX / 2)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  const int64_t span = attended_tokens(max_blocks_per_seq, block_size, sliding_window);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size,
                                      window_binds(max_blocks_per_seq, block_size, sliding_window));
  if (pt <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "partition_size %d is not a multiple of %d tokens",
                     partition_size, pkv_dev::partition_align(block_size));
  const int parts = static_cast<int>((span + pt - 1) / pt);
  const int group = num_heads / num_kv_heads;
  const bool vector = kv_dtype == PKV_F32 || group == 1;
  const int hpi = vector ? mha_plan(num_seqs, num_heads, num_kv_heads, parts, kv_dtype, span).hpi : 1;
  const int64_t items = static_cast<int64_t>(num_seqs) * (num_kv_heads / hpi) * parts;
  if (items > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "grid too large");
  plan[0] = parts > 1 ? static_cast<int>(pt) : 0;
  plan[1] = parts;
  plan[2] = hpi;
  plan[3] = vector ? 0 : 1;
  plan[4] = static_cast<int>(items);
  return PKV_OK;
  PKV_API_END
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
  if (int rc = check_decode(out, q, key_cache, value_cache, k_scales, v_scales, block_tables,
                            context_lens, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, kv_dtype, q_dtype, scale, sliding_window))
    return rc;
  const int group = num_heads / num_kv_heads;
  const int64_t span = attended_tokens(max_blocks_per_seq, block_size, sliding_window);
  const int64_t pt = partition_tokens(num_seqs, num_kv_heads, span, block_size, partition_size,
                                      window_binds(max_blocks_per_seq, block_size, sliding_window));
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
  const bool vector = kv_dtype == PKV_F32 || group == 1;
  const MhaPlan mp = vector ? mha_plan(num_seqs, num_heads, num_kv_heads, parts, kv_dtype, span)
                            : MhaPlan{1, 0};
  const int hpi = mp.hpi;
  const int64_t items = static_cast<int64_t>(num_seqs) * (num_kv_heads / hpi) * parts;
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
  a.heads_per_item = hpi;
  a.balance_run = mp.run;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.prefix_lens = nullptr;
  a.part_base = 0;
  a.prefix_chunk = 1;
  a.merge_prefix = 0;

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
    const int64_t rgrid = static_cast<int64_t>(num_seqs) * num_heads;
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

size_t pkv_decode_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int max_blocks_per_seq,
                                        const int32_t* groups, int num_groups) {
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      !pkv_dev::supported_block_size(block_size) ||
      static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX / 2)
    return 0;
  PrefixPlan plan;
  if (plan_prefix(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq, groups,
                  num_groups, &plan) != PKV_OK) {
    pkv::clear_error();
    return 0;
  }
  const size_t parts = static_cast<size_t>(plan.max_chunks) + plan.parts;
  return static_cast<size_t>(num_seqs) * num_heads * parts * (head_dim + 2) * sizeof(float);
}

int pkv_paged_attention_decode_prefix(void* out, const void* q, const void* key_cache,
                                      const void* value_cache, const float* k_scales,
                                      const float* v_scales, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* prefix_lens,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      float scale, int q_dtype, int kv_dtype,
                                      const int32_t* groups, int num_groups, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  PKV_API_BEGIN
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) ||
      num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "bad shape: seqs=%d heads=%d kv_heads=%d head_dim=%d block_size=%d "
                     "max_blocks=%d num_blocks=%d",
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks);
  if (num_seqs == 0) return PKV_OK;
  if (int rc = check_decode(out, q, key_cache, value_cache, k_scales, v_scales, block_tables,
                            context_lens, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, kv_dtype, q_dtype, scale, 0))
    return rc;
  if (!prefix_lens) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL prefix_lens");
  PrefixPlan plan;
  if (int rc = plan_prefix(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                           groups, num_groups, &plan))
    return rc;
  // fp32 caches have no matrix-core path: the plain decode gives the same
  // result (and needs no more workspace than the shared-prefix one).
  if (kv_dtype == PKV_F32)
    return pkv_paged_attention_decode(out, q, key_cache, value_cache, k_scales, v_scales,
                                      block_tables, context_lens, num_seqs, num_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, scale, q_dtype, kv_dtype, 0, 0, workspace,
                                      workspace_bytes, stream);
  const int parts = plan.max_chunks + plan.parts;
  const size_t need = static_cast<size_t>(num_seqs) * num_heads * parts * (head_dim + 2) *
                      sizeof(float);
  if (!workspace || workspace_bytes < need)
    return pkv::fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                     workspace_bytes, workspace ? "" : ", NULL");
  const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * plan.parts;
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
  a.ws_ml = ws;
  a.ws_acc = ws + 2 * slots;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.align = pkv_dev::partition_align(block_size);
  a.part_tokens = plan.part_tokens;
  a.num_parts = parts;
  a.window = 0;
  a.heads_per_item = 1;
  a.balance_run = 0;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.prefix_lens = prefix_lens;
  a.part_base = plan.max_chunks;
  a.prefix_chunk = plan.chunk;
  // Grouped-query heads: the prefix items and the decode of the rest of each
  // context share one launch (the rest writes partials, and the merge kernel
  // combines them with the prefix chunks).  One query head per kv head: the
  // prefix kernel, then the multi-head decode of the rest, which merges the
  // prefix chunks into its own result when the rest is one partition.
  const int group = num_heads / num_kv_heads;
  const bool fused = group >= 2 && group <= 16;
  a.merge_prefix = (!fused && plan.parts == 1) ? 1 : 0;

  pkv_dev::PrefixArgs pa;
  pa.d = a;
  pa.num_groups = num_groups;
  for (int g = 0; g < num_groups; ++g) {
    pa.group_first[g] = groups[3 * g];
    pa.group_count[g] = groups[3 * g + 1];
    pa.group_prefix[g] = groups[3 * g + 2];
  }
  for (int g = 0; g <= num_groups; ++g) pa.work_start[g] = plan.work_start[g];

  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok = false;
  hipError_t err = hipSuccess;
  const unsigned n_prefix = static_cast<unsigned>(plan.work_start[num_groups]);
  const unsigned grid = static_cast<unsigned>(items);
  if (static_cast<int64_t>(n_prefix) + (fused ? items : 0) > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "grid too large");
  const unsigned n_rest = fused ? grid : 0;
  switch (kv_dtype) {
    case PKV_F16:
      err = pkv_dev::launch_prefix_f16(q_dtype, head_dim, group, pa, n_prefix, n_rest, s, ok);
      break;
    case PKV_BF16:
      err = pkv_dev::launch_prefix_bf16(q_dtype, head_dim, group, pa, n_prefix, n_rest, s, ok);
      break;
    case PKV_I8:
      err = pkv_dev::launch_prefix_i8(q_dtype, head_dim, group, pa, n_prefix, n_rest, s, ok);
      break;
    case PKV_FP8:
      err = pkv_dev::launch_prefix_fp8(q_dtype, head_dim, group, pa, n_prefix, n_rest, s, ok);
      break;
    default: break;
  }
  if (!ok) return pkv::fail(PKV_ERR_UNSUPPORTED, "no prefix kernel for this combination");
  if (err != hipSuccess)
    return pkv::fail(PKV_ERR_HIP, "prefix launch: %s", hipGetErrorString(err));
  if (!fused) {
    switch (kv_dtype) {
      case PKV_F16: err = pkv_dev::launch_decode_f16(q_dtype, head_dim, group, a, grid, s, ok); break;
      case PKV_BF16: err = pkv_dev::launch_decode_bf16(q_dtype, head_dim, group, a, grid, s, ok); break;
      case PKV_I8: err = pkv_dev::launch_decode_i8(q_dtype, head_dim, group, a, grid, s, ok); break;
      case PKV_FP8: err = pkv_dev::launch_decode_fp8(q_dtype, head_dim, group, a, grid, s, ok); break;
      default: break;
    }
    if (!ok) return pkv::fail(PKV_ERR_UNSUPPORTED, "no kernel for this combination");
    if (err != hipSuccess)
      return pkv::fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
  }
  if (!a.merge_prefix) {
    const int64_t rgrid = static_cast<int64_t>(num_seqs) * num_heads;
    switch (q_dtype) {
      case PKV_F16: err = pkv_dev::launch_reduce<PKV_F16>(head_dim, a, rgrid, s); break;
      default: err = pkv_dev::launch_reduce<PKV_BF16>(head_dim, a, rgrid, s); break;
    }
    if (err != hipSuccess)
      return pkv::fail(PKV_ERR_HIP, "partition merge launch: %s", hipGetErrorString(err));
  }
  return PKV_OK;
  PKV_API_END
}

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* key_cache,
                                       const void* value_cache, const float* k_scales,
                                       const float* v_scales, const int32_t* block_tables,
                                       const int32_t* context_lens, int num_seqs, int num_heads,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int max_blocks_per_seq, int num_blocks, float scale,
                                       int q_dtype, int kv_dtype, int partition_size,
                                       int sliding_window, void* stream) {
  PKV_API_BEGIN
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq))
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad shape");
  const size_t need =
      pkv_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, partition_size, sliding_window);
  if (need > kScratchBytes)
    return pkv::fail(PKV_ERR_WORKSPACE,
                     "these shapes need %zu bytes of partials; the static scratch holds %zu "
                     "(use pkv_paged_attention_decode with a workspace)",
                     need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int device = -1;
    hipError_t err = hipSuccess;
    ws = scratch_address(&device, &err);
    if (!ws)
      return pkv::fail(PKV_ERR_HIP, "scratch address on device %d: %s", device,
                       hipGetErrorString(err));
  }
  return pkv_paged_attention_decode(out, q, key_cache, value_cache, k_scales, v_scales,
                                    block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                    head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                                    q_dtype, kv_dtype, partition_size, sliding_window, ws,
                                    need > 0 ? kScratchBytes : 0, stream);
  PKV_API_END
}

}  // extern "C"
