/*
 * pkv.h -- C ABI of libpkv.so: paged-attention decode on AMD MI355X (gfx950).
 *
 * Page keys used in the citations below:
 *   [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com)
 *   [P2] "大模型部署中KV Cache优化策略与显存管理实践教程" (yunthe.com)
 *   [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn)
 *
 * Conventions shared by every entry point:
 *   - Every function returns an int status (PKV_OK = 0) and never lets a C++
 *     exception cross the ABI.  On failure pkv_last_error() returns a message
 *     for the calling thread, valid until that thread's next pkv_* call.
 *   - Device buffers are owned by the caller (the library never allocates,
 *     frees or synchronises device memory, except that pkv_copy_blocks takes
 *     its pairs from host memory).  Host buffers are only read or written during
 *     the call, except the pinned host pools of pkv_swap_blocks, which its
 *     kernel reads and writes on the stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Kernels are enqueued on it; functions return before they finish.
 *   - Shapes and sizes are validated on the host.  Values that live in device
 *     memory (block tables, context lengths, slots) cannot be checked without a
 *     device sync: kernels clamp them so that no access leaves its buffer, and
 *     pkv_validate_tables checks host copies when the caller wants an error.
 *
 * Data layout (device, row-major, from the address formula in the kernel
 * sketch of [P1] "PagedAttention注意力计算流程"):
 *   key_cache, value_cache  [num_blocks][block_size][num_kv_heads][head_dim]
 *                           element (b, o, h, d) at ((b*bs + o)*Hkv + h)*D + d
 *   q, out                  [num_seqs][num_heads][head_dim]
 *   block_tables            int32 [num_seqs][max_blocks_per_seq]
 *   context_lens            int32 [num_seqs]
 *   k_scales, v_scales      fp32 [num_blocks][num_kv_heads]   (int8 and fp8 caches)
 *                           value of a stored code = decode(code) * scale
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,  /* null pointer, bad shape, bad enum value        */
  PKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, format)   */
  PKV_ERR_OOM = 3,          /* allocator: not enough free blocks              */
  PKV_ERR_DOUBLE_FREE = 4,  /* allocator: a reference dropped twice           */
  PKV_ERR_INDEX = 5,        /* allocator: token past the allocated blocks     */
  PKV_ERR_HIP = 6,          /* a HIP runtime call failed                      */
  PKV_ERR_WORKSPACE = 7     /* decode: workspace missing or too small         */
};

/* Storage formats.  PKV_FP8 is the OCP FP8 E4M3 format (sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; no infinities, 0x7F / 0xFF are NaN, largest
 * finite 448): the [P2] "量化压缩KV Cache的INT8与FP8方案" FP8 cache option,
 * whose printed "E4M1" is read as E4M3. */
enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_I8 = 3, PKV_FP8 = 4 };

/* Message describing the calling thread's last failure ("" if none). */
const char* pkv_last_error(void);

/* ABI version (bumped when a signature changes). */
int pkv_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Decode                                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Tokens per context partition that pkv_paged_attention_decode will use for
 * these shapes when called with the same `partition_size` (0 = automatic).
 * The result is a multiple of U = max(block_size, 16), or 0 if the context is
 * not split.  Returns 0 for invalid shapes or an unsupported block size.  The
 * automatic choice depends on shapes only (never on device data): with
 * span = max_blocks_per_seq * block_size rounded up to U, a span of up to 2560
 * tokens is not split, a longer one is split into 1024-token partitions, and
 * the partitions are made smaller towards
 * num_seqs * num_kv_heads * partitions >= 512, but not below span / 32
 * tokens clamped to 128 .. 1024 (so a span of at most 128 tokens stays
 * whole).  With a sliding window W that is shorter than the table, the span
 * is W + U - 1 rounded up to U, it is not split by length (every context
 * longer than W attends exactly W tokens), and it is split into equal
 * partitions only towards num_seqs * num_kv_heads * partitions >= 256, with
 * the same floor.  Partitions are rounded up to U.  The partitions of a
 * sequence start at its first attended token rounded down to U.
 */
int pkv_decode_partition_size(int num_seqs, int num_heads, int num_kv_heads,
                              int head_dim, int block_size,
                              int max_blocks_per_seq, int partition_size,
                              int sliding_window);

/*
 * Workspace bytes the decode needs for these shapes (0 when the context is
 * not split, in which case `workspace` may be NULL): fp32 (max, sum) and
 * head_dim accumulators per (sequence, query head, partition), the partial
 * softmax results that the merge kernel combines.  The pages' kernel sketch
 * ([P1] "PagedAttention注意力计算流程") has no split; the partials are this
 * library's way to spread one long context over many workgroups.  Same
 * arguments as pkv_decode_partition_size.
 */
size_t pkv_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                 int head_dim, int block_size,
                                 int max_blocks_per_seq, int partition_size,
                                 int sliding_window);

/*
 * How pkv_paged_attention_decode will run for these shapes and this cache
 * format (the same arguments, plus kv_dtype): the grid that splits the work
 * of [P1] "PagedAttention注意力计算流程" into workgroups.  plan: host int[5]
 * receiving
 *   [0] tokens per partition (0 when contexts are not split),
 *   [1] partitions per (sequence, kv head),
 *   [2] kv heads per workgroup (multi-head kernel: 1, 2 or 4; else 1),
 *   [3] kernel: 0 = multi-head kernel on the vector ALUs (one query head per
 *       kv head, or an fp32 cache), 1 = grouped-query kernel on the matrix
 *       cores,
 *   [4] workgroups of the decode launch.
 * Depends on shapes and on the current device's compute-unit count (see the
 * length-balanced order under pkv_paged_attention_decode; without a device
 * the plan is the one without that order), never on device data.  Errors:
 * INVALID_ARG (bad shape, partition size or format), UNSUPPORTED (block
 * size).
 */
int pkv_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int partition_size, int sliding_window, int kv_dtype,
                    int* plan);

/*
 * Paged-attention decode ([P1] "PagedAttention注意力计算流程" and its kernel
 * sketch; [P3] section 三): for each sequence s and query head h, with
 * n = context_lens[s] and kv head kvh = h / (num_heads / num_kv_heads),
 *
 *   token i < n  ->  physical block block_tables[s][i / bs], offset i % bs
 *   score_i      =   scale * dot(q[s][h], K[i][kvh])
 *   out[s][h]    =   sum_i softmax(score)_i * V[i][kvh]
 *
 * with K/V of an int8 or fp8 cache dequantised as code * scale[block][kvh]
 * ([P2] "量化压缩KV Cache的INT8与FP8方案"; one scale per (block, kv head)).
 * The softmax is computed stably (scores shifted by their maximum), in fp32;
 * long contexts are split into partitions whose partial results are merged
 * exactly.  n = 0 gives an all-zero output.  Table entries past
 * ceil(n / bs) and slots past n are never read.
 *
 * With sliding_window = W > 0 only tokens max(0, n - W) .. n - 1 are attended
 * (the window of [P2] "Sliding Window Attention控制长序列显存"); table entries
 * of blocks before the window are never read (they may be -1 after
 * pkv_seq_trim_window).
 *
 *   out          device, [B][H][D] in q_dtype (written)
 *   q            device, [B][H][D] in q_dtype: F32, F16 or BF16
 *   key_cache    device, see layout above, kv_dtype
 *   value_cache  device, same shape and format as key_cache
 *   k_scales     device fp32 [NB][Hkv], required iff kv_dtype is I8 or FP8
 *   v_scales     device fp32 [NB][Hkv], required iff kv_dtype is I8 or FP8.
 *                Bound: with an F16 query and several query heads per kv head
 *                (the matrix-core kernel, here and in the shared-prefix
 *                decode) each softmax weight, up to 2^8, is multiplied by its
 *                block's v_scale and fed to the matrix cores as two f16 parts;
 *                v_scale <= 256 keeps that product within about 22 bits of
 *                precision.  Larger values lose precision, and above 511 the
 *                parts saturate (wrong outputs).  Scales are device data and
 *                are not checked.  BF16 queries have no such bound.
 *   block_tables device int32 [B][max_blocks_per_seq]
 *   context_lens device int32 [B]; values are clamped to
 *                [0, max_blocks_per_seq * block_size]
 *   kv_dtype     F32 (q F32), F16 (q F16), BF16 (q BF16), I8 or FP8 (q F16
 *                or BF16)
 *   head_dim     64 or 128; block_size 8, 16 or 32 ([P1] deployment section:
 *                16 by default);
 *                num_heads / num_kv_heads in {1, 2, 4, 8, 16}
 *   partition_size  tokens per partition, a multiple of max(block_size, 16), or 0 for
 *                the library's choice; a value >= the longest possible context
 *                disables splitting
 *   sliding_window  0 (attend to the whole context) or W > 0 tokens
 *   workspace    device scratch of >= pkv_decode_workspace_size(...) bytes
 *                (may be NULL when that is 0); fully rewritten by each call,
 *                so calls that share a workspace must be stream-ordered
 *
 * Scheduling (not part of the result): batches of 2..64 sequences decoded
 * by the multi-head kernel with whole contexts, tables of at least 1024
 * tokens and a grid that fills the GPU's compute units once to four times,
 * are dealt to the workgroups by context length (each workgroup reads all
 * lengths), so that every compute unit gets long and short contexts alike;
 * equal lengths keep the batch order.
 *
 * A block id outside [0, num_blocks) in a position that is read makes that
 * block's tokens count as masked (output unspecified but finite, no
 * out-of-bounds access).  Errors: INVALID_ARG (null pointer, bad shape or
 * format pair), UNSUPPORTED (head_dim, block_size, group size), WORKSPACE,
 * HIP (launch failure).
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* key_cache,
                               const void* value_cache, const float* k_scales,
                               const float* v_scales, const int32_t* block_tables,
                               const int32_t* context_lens, int num_seqs,
                               int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq,
                               int num_blocks, float scale, int q_dtype,
                               int kv_dtype, int partition_size, int sliding_window,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and result, without `workspace` and
 * `workspace_bytes`.  When the contexts are split, the partials go to a
 * scratch array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds
 * in each GPU's memory from its first call on that GPU until the process
 * ends; the call itself allocates nothing.  Shapes whose
 * pkv_decode_workspace_size exceeds that are rejected with WORKSPACE (nothing
 * is launched).  Every call on one GPU shares that GPU's scratch: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.  Nothing in the scratch has to start at zero (each
 * call writes every partial it reads).  Errors: those of
 * pkv_paged_attention_decode, plus HIP if the scratch's device address cannot
 * be obtained.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* key_cache,
                                       const void* value_cache, const float* k_scales,
                                       const float* v_scales, const int32_t* block_tables,
                                       const int32_t* context_lens, int num_seqs, int num_heads,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int max_blocks_per_seq, int num_blocks, float scale,
                                       int q_dtype, int kv_dtype, int partition_size,
                                       int sliding_window, void* stream);

/*
 * Shared-prefix decode ([P1] "vLLM调度器与PagedAttention协同工作" item 2:
 * requests that share a system prompt share its blocks; [P2] "Prefix Cache
 * 复用共享前缀的KV Cache"): the same result as pkv_paged_attention_decode,
 * computed so that a prefix shared by a group of sequences is attended once
 * for all of the group's query heads instead of once per sequence.  A prefix
 * kernel handles each group's shared tokens (many query rows per K/V tile, on
 * the matrix cores), the decode kernels the rest of every context (for
 * grouped-query heads in the same launch, after the prefix work), and the two
 * parts are combined exactly.  No host synchronisation or allocation: the
 * call can be captured in a HIP graph.
 *
 * Groups are ranges of the batch:
 *   groups        HOST int32 [3 * num_groups]: (first sequence, number of
 *                 sequences, shared tokens) per group; the ranges lie within
 *                 [0, num_seqs) and do not overlap (sequences outside every
 *                 group have no shared prefix); shared tokens are a positive
 *                 multiple of max(block_size, 16), at most
 *                 max_blocks_per_seq * block_size
 *   num_groups    1 .. 32
 *   prefix_lens   device int32 [num_seqs]: the shared tokens of the
 *                 sequence's group, 0 for a sequence outside every group
 * Preconditions (not checked on the device): the sequences of a group have
 * the same table entries for their shared tokens (as forks of a common
 * prompt have) and context lengths >= the shared tokens.  Violations
 * give wrong outputs but no out-of-bounds access.  No sliding window.
 * workspace: >= pkv_decode_prefix_workspace_size(...) bytes (always needed).
 * fp32 caches run the plain decode (no matrix-core path).
 * Other arguments and errors as pkv_paged_attention_decode, plus INVALID_ARG
 * for bad groups.
 */
int pkv_paged_attention_decode_prefix(void* out, const void* q, const void* key_cache,
                                      const void* value_cache, const float* k_scales,
                                      const float* v_scales, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* prefix_lens,
                                      int num_seqs, int num_heads, int num_kv_heads,
                                      int head_dim, int block_size, int max_blocks_per_seq,
                                      int num_blocks, float scale, int q_dtype, int kv_dtype,
                                      const int32_t* groups, int num_groups, void* workspace,
                                      size_t workspace_bytes, void* stream);
/* Workspace bytes of pkv_paged_attention_decode_prefix (0 for invalid shapes
 * or groups). */
size_t pkv_decode_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int max_blocks_per_seq,
                                        const int32_t* groups, int num_groups);

/* ------------------------------------------------------------------------ */
/* Cache write                                                               */
/* ------------------------------------------------------------------------ */

/*
 * reshape_and_cache: scatter each new token's K and V rows into its cache
 * slot.  Token t goes to block slot_mapping[t] / bs, offset slot_mapping[t] % bs
 * (the inverse of the physical offset phys * bs + offset of the [P1] kernel
 * sketch).  A slot < 0, or one at or past num_blocks * bs, is skipped.
 *
 *   k, v         device, [num_tokens][num_kv_heads][head_dim] in src_dtype
 *   key_cache, value_cache  device, layout above, kv_dtype (written)
 *   k_scales, v_scales      device fp32 [NB][Hkv], required iff kv_dtype == I8:
 *                the existing scale of each (block, kv head); the int8 code is
 *                clamp(rint(x / scale), -127, 127) with the division and the
 *                round-half-to-even done in fp32
 *   slot_mapping device int32 [num_tokens]
 *   src_dtype    equal to kv_dtype for float caches; F32, F16 or BF16 for I8
 *
 * Slots must be distinct among the tokens of one call (else which write wins
 * is unspecified).  Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
int pkv_reshape_and_cache(const void* k, const void* v, void* key_cache,
                          void* value_cache, const float* k_scales,
                          const float* v_scales, const int32_t* slot_mapping,
                          int num_tokens, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int src_dtype,
                          int kv_dtype, void* stream);

/*
 * Copy whole physical blocks (K and V, and for int8 caches their scales) from
 * src to dst: the data copy that copy-on-write leaves to the caller ([P3]
 * section 二, copy_on_write).  `pairs` is HOST memory: n_pairs (src, dst)
 * int32 pairs; ids must be in [0, num_blocks) and dst ids distinct and not
 * used as a src in the same call.  block_bytes = bs * Hkv * D * element size.
 * k_scales / v_scales may be NULL (float caches); scale_stride = Hkv.
 * Errors: INVALID_ARG, HIP.
 */
int pkv_copy_blocks(void* key_cache, void* value_cache, float* k_scales,
                    float* v_scales, const int32_t* pairs, int n_pairs,
                    size_t block_bytes, int num_blocks, int scale_stride,
                    void* stream);

/*
 * Swap whole blocks between the device pool and a pool of host blocks
 * ([P1] "vLLM调度器与PagedAttention协同工作", preemption and recovery: when
 * device memory runs short a low-priority request's KV moves to CPU memory,
 * freeing its device blocks, and is copied back once blocks are free again;
 * [P1] deployment section, swap_space).
 *
 *   key_cache, value_cache, k_scales, v_scales  the device pool (layout above;
 *                scales NULL for float caches, else fp32 [num_blocks][scale_stride])
 *   host_key, host_value  PINNED host memory allocated with hipHostMalloc (or a
 *                pinned torch tensor), [num_host_blocks][block_bytes]: block h
 *                at byte h * block_bytes, the same bytes a device block holds
 *   host_k_scales, host_v_scales  pinned host fp32 [num_host_blocks][scale_stride],
 *                NULL exactly when k_scales is
 *   pairs        HOST int32 pairs, n_pairs of them, as pkv_seq_swap_out and
 *                pkv_seq_swap_in return them:
 *                  direction PKV_SWAP_OUT: (device block, host block), device -> host
 *                  direction PKV_SWAP_IN:  (host block, device block), host -> device
 *                destination ids distinct; a source may repeat
 *
 * The copy is one kernel that reads and writes the pinned memory through its
 * device mapping (no per-block DMA requests).  It is enqueued on `stream`;
 * synchronise before the host reads host blocks written by a swap-out, and
 * keep the source blocks unchanged until the copy has finished.
 * Errors: INVALID_ARG (ids out of range, repeated destinations, host memory
 * that is not pinned), HIP.
 */
enum { PKV_SWAP_OUT = 0, PKV_SWAP_IN = 1 };
int pkv_swap_blocks(void* key_cache, void* value_cache, float* k_scales, float* v_scales,
                    void* host_key, void* host_value, float* host_k_scales,
                    float* host_v_scales, const int32_t* pairs, int n_pairs,
                    size_t block_bytes, int num_blocks, int num_host_blocks,
                    int scale_stride, int direction, void* stream);

/*
 * Plain device-to-device streaming copy of `bytes` bytes (a multiple of 16,
 * 16-byte aligned pointers) with the library's own kernel: the reference
 * point for achievable HBM bandwidth and for scaling hardware byte counters.
 */
int pkv_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Read-only streaming probe over `bytes` bytes of device memory at `src` (a
 * multiple of 16, 16-byte aligned) with the decode's loads (16-byte,
 * non-temporal), each workgroup reading one contiguous stretch: the reference
 * point for the read bandwidth of a plain stream.  Each thread folds the words it read with XOR and writes the fold to
 * the device word `sink` only when it equals `sentinel`, so that no load can
 * be optimised away; `sink` must be a writable device word (its content
 * after the call is unspecified unless some fold equals the sentinel).
 * Errors: INVALID_ARG (NULL, misaligned, size), HIP.
 */
int pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t sentinel,
                    void* stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator ([P3] section 二: BlockManager / BlockTable; [P1]     */
/* "PagedAttention分页内存管理原理" and "vLLM调度器与PagedAttention协同工作"). */
/* Host memory only, no device calls.  Not thread safe: one allocator must   */
/* not be used from two threads at once.                                    */
/* ------------------------------------------------------------------------ */

typedef struct pkv_allocator pkv_allocator;

/* A pool of num_blocks blocks of block_size tokens; free list = 0..N-1, and
 * blocks leave from its END (the first allocation returns N-1).  INVALID_ARG
 * when num_blocks * block_size exceeds INT32_MAX (slots are int32). */
int pkv_allocator_create(int num_blocks, int block_size, pkv_allocator** out);
int pkv_allocator_destroy(pkv_allocator* a);

/* Replace the free list by `order` (n == num_blocks, a permutation); legal
 * only while every block is free.  Blocks then leave from order[n-1] down. */
int pkv_allocator_set_free_order(pkv_allocator* a, const int32_t* order, int n);

/* Allocate n blocks (all or nothing; OOM leaves the state unchanged); each
 * gets reference count 1.  out_ids: host int32[n]. */
int pkv_allocate(pkv_allocator* a, int n, int32_t* out_ids);

/* Drop one reference per listed id; a block reaching 0 goes back on the free
 * list (reused first).  A drop below 0 is DOUBLE_FREE, detected before any
 * change. */
int pkv_free(pkv_allocator* a, const int32_t* ids, int n);

/* Add one reference per listed id (ids must be allocated): sharing of prompt
 * blocks ([P1] shared prefixes through reference counts). */
int pkv_incref(pkv_allocator* a, const int32_t* ids, int n);

/* Copy-on-write of one block ([P3] section 二): a sole owner keeps the block
 * (*copied = 0); a shared block gives the writer a new block (*copied = 1,
 * the caller copies the data) and drops one reference of the old one.
 * INVALID_ARG if the block is not allocated; OOM if no block is free. */
int pkv_copy_on_write(pkv_allocator* a, int32_t id, int32_t* new_id, int* copied);

/* Reference count of a block, and the number of free blocks ([P3] section 二:
 * the block manager's per-block counts and its free list). */
int pkv_ref_count(const pkv_allocator* a, int32_t id, int* out);
int pkv_num_free(const pkv_allocator* a, int* out);
/* 1 - free / num_blocks ([P3] section 二, usage_ratio). */
int pkv_usage_ratio(const pkv_allocator* a, double* out);
/* Copy of the free list ([P3] section 二), bottom to top (the next block to
 * leave is last). */
int pkv_free_list(const pkv_allocator* a, int32_t* out, int cap, int* n);
/* Number of copy-on-write copies handed out so far ([P3] section 二,
 * copy_on_write). */
int pkv_cow_count(const pkv_allocator* a, int64_t* out);

/* Sequences: a logical block table plus a token count ([P3] BlockTable). */
int pkv_seq_create(pkv_allocator* a, int32_t* seq);
/* A child sequence sharing all of the parent's blocks (one more reference
 * each) and its token count: parallel sampling / shared prompts. */
int pkv_seq_fork(pkv_allocator* a, int32_t seq, int32_t* child);
/*
 * Append n tokens with on-demand allocation ([P1] scheduler section): a token
 * that starts a logical block takes a new block; a token that lands in a
 * partly filled last block shared with other sequences first triggers
 * copy-on-write of that block.  All or nothing (OOM leaves the state
 * unchanged).  slots_out: host int32[n], slot = block * bs + offset of each
 * token.  cow_pairs_out: host int32[2 * cow_cap] receiving (src, dst) block
 * pairs to copy before writing (at most 1 per call); *n_cow their number.
 */
int pkv_seq_append_tokens(pkv_allocator* a, int32_t seq, int n, int32_t* slots_out,
                          int32_t* cow_pairs_out, int cow_cap, int* n_cow);
/*
 * Sliding window ([P2] "Sliding Window Attention控制长序列显存": a sequence
 * keeps the KV of its last W tokens only, so its cache stays bounded in size):
 * drop this sequence's reference to every block that holds no token of its
 * last `window` tokens (blocks before the one holding token
 * max(0, tokens - window)).  Their table entries become -1 (exported as the
 * pad value; a lookup of their tokens is INDEX).  *n_released receives the
 * number of blocks released; `released` (host int32[cap], may be NULL) their
 * ids, in logical order.  INVALID_ARG (state unchanged) if window <= 0 or cap
 * is too small for a non-NULL `released`.
 */
int pkv_seq_trim_window(pkv_allocator* a, int32_t seq, int window, int32_t* released,
                        int cap, int* n_released);
/*
 * Swap pool ([P1] "vLLM调度器与PagedAttention协同工作", preemption and
 * recovery; [P1] deployment section, swap_space in GB).  The allocator also
 * tracks num_host_blocks host blocks (ids 0..num_host_blocks-1, a LIFO free
 * list like the device pool's, the first taken is num_host_blocks-1).  Legal
 * only while no sequence is swapped out; a new size resets the host free list.
 */
int pkv_allocator_set_host_pool(pkv_allocator* a, int num_host_blocks);
int pkv_host_num_free(const pkv_allocator* a, int* out);
/*
 * Preempt a sequence: each of its blocks (entries -1 after a trim stay -1)
 * takes a host block, and the sequence drops its device reference (a block
 * it shared stays with the other sequences; a block it alone held returns to
 * the free list).  Its table then holds host ids and the sequence is
 * "swapped out": append, fork, trim, lookup and export of it fail with
 * INVALID_ARG until pkv_seq_swap_in.  pairs: host int32[2 * cap] receiving
 * (device block, host block) in logical order, for pkv_swap_blocks with
 * PKV_SWAP_OUT, to be enqueued BEFORE any write into the released device
 * blocks.  *n_pairs = the number of pairs needed, set also on failure.
 * All or nothing: OOM if the host pool is short, INVALID_ARG if cap is too
 * small or the sequence is already swapped out.
 */
int pkv_seq_swap_out(pkv_allocator* a, int32_t seq, int32_t* pairs, int cap, int* n_pairs);
/*
 * Bring a swapped-out sequence back: each host block takes a fresh device
 * block (reference count 1; sharing from before the swap-out is not restored)
 * and returns to the host free list.  pairs receives (host block, device
 * block) for pkv_swap_blocks with PKV_SWAP_IN.  All or nothing: OOM if too
 * few device blocks are free; INVALID_ARG if cap is too small or the sequence
 * is not swapped out.
 */
int pkv_seq_swap_in(pkv_allocator* a, int32_t seq, int32_t* pairs, int cap, int* n_pairs);
int pkv_seq_is_swapped(const pkv_allocator* a, int32_t seq, int* out);
/* Release all of the sequence's block references (host blocks if it is
 * swapped out) and forget it. */
int pkv_seq_free(pkv_allocator* a, int32_t seq);
int pkv_seq_num_tokens(const pkv_allocator* a, int32_t seq, int* out);
/* The sequence's logical block table (-1 for blocks released by a trim; host
 * block ids while it is swapped out). */
int pkv_seq_block_ids(const pkv_allocator* a, int32_t seq, int32_t* out, int cap, int* n);
/* Physical block of a logical token ([P3] BlockTable lookup): INDEX if the
 * token's logical block has not been allocated; INVALID_ARG if swapped out. */
int pkv_seq_physical_block(const pkv_allocator* a, int32_t seq, int token, int32_t* out);
/*
 * Export host block tables for a batch, in the layout the decode reads: one
 * row of max_blocks entries per sequence (the row stride max_blocks of the
 * table lookup in the kernel sketch of [P1] "PagedAttention注意力计算流程"),
 * filled from the sequences' logical tables ([P3] section 二, BlockTable).
 * out_tables int32[n][max_blocks]
 * padded with `pad`, out_lens int32[n] token counts.  INVALID_ARG if a
 * sequence holds more than max_blocks blocks.
 */
int pkv_export_block_tables(const pkv_allocator* a, const int32_t* seqs, int n,
                            int max_blocks, int32_t pad, int32_t* out_tables,
                            int32_t* out_lens);

/*
 * Debug check of HOST copies of decode inputs: every table entry a context
 * reads (only the window's blocks when sliding_window > 0) lies in
 * [0, num_blocks), and 0 <= len <= max_blocks * block_size.
 * On INVALID_ARG, *bad_seq / *bad_block name the first offending entry
 * (bad_block = -1 for a bad length).
 */
int pkv_validate_tables(const int32_t* tables, const int32_t* lens, int num_seqs,
                        int max_blocks, int block_size, int num_blocks,
                        int sliding_window, int* bad_seq, int* bad_block);

/*
 * Host helper for pkv_paged_attention_decode_prefix ([P1] scheduler section,
 * item 2: forks of one prompt share its blocks): scans HOST copies of the
 * tables in batch order and returns groups of consecutive sequences (at least
 * max(min_group, 2) of them) whose tables hold the same block ids for their
 * leading blocks.  A group's shared tokens are the whole blocks that every
 * member's context covers and all members agree on, rounded down to
 * max(block_size, 16), and at least min_tokens.  Greedy: a group grows while
 * the next sequence keeps at least min_tokens shared.  At most 32 groups
 * (the rest of the batch is then left ungrouped).  groups_out: host int32
 * [3 * cap] receiving (first sequence, count, shared tokens); *n_groups their
 * number (set also when cap is too small: INVALID_ARG).
 */
int pkv_find_shared_prefixes(const int32_t* tables, const int32_t* lens, int num_seqs,
                             int max_blocks, int block_size, int min_tokens, int min_group,
                             int32_t* groups_out, int cap, int* n_groups);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PKV_H_ */
