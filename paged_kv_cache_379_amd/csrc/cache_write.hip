// The cache write (reshape_and_cache), the block copies behind copy-on-write
// and swapping, and a plain streaming copy used as the bandwidth reference.
//
// Page keys:
//   [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com)
//   [P2] "大模型部署中KV Cache优化策略与显存管理实践教程" (yunthe.com)
//   [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn)
//
// A new token's K and V rows ([Hkv][D], contiguous in the source and in the
// cache slot, by the layout of the [P1] kernel sketch) are written to
// block slot / bs, offset slot % bs.  Workgroups per (token, K or V, slice of
// kWriteThreads 16-byte vectors of the row) move the row with one 16-byte load
// and store per thread, so a write costs one memory round trip; an int8 cache
// quantises on the way with the (block, kv head) scale ([P2] INT8 KV cache
// section; scale granularity is this library's reading).
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "decode_kernel.h"
#include "pkv_internal.h"

namespace {

using pkv_dev::Format;
using pkv_dev::unpack16;

struct CacheWriteArgs {
  const uint8_t* k;
  const uint8_t* v;
  uint8_t* key_cache;
  uint8_t* value_cache;
  const float* k_scales;
  const float* v_scales;
  const int32_t* slots;
  int64_t num_slots;  // num_blocks * block_size
  int num_kv_heads;
  int head_dim;
  int block_size;
};

constexpr int kWriteThreads = 256;

// fp32 -> OCP FP8 E4M3 code: the nearest representable value, ties to the
// even mantissa; magnitudes of 448 and above (infinities included) saturate
// to 448 and NaN gives 0x7F.  Below 2^-6 the values are the multiples of
// 2^-9 (subnormals); above, 8 steps per binade: q = a * 2^(3 - e) lies in
// [8, 16], and q = 16 carries into the next exponent by itself.
__device__ __forceinline__ uint32_t encode_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | static_cast<uint32_t>(rintf(a * 512.f));
  const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  const uint32_t q = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));
  return sign | ((static_cast<uint32_t>(e + 7) << 3) + q - 8u);
}

// The stored byte of x / scale for a one-byte cache format (IEEE division).
template <int KF>
__device__ __forceinline__ uint32_t quantise_byte(float x, float sc) {
  if constexpr (KF == PKV_I8) {
    float qv = rintf(x / sc);  // round half to even
    qv = fminf(fmaxf(qv, -127.f), 127.f);
    return static_cast<uint32_t>(static_cast<int32_t>(qv)) & 0xFFu;
  } else {
    return encode_e4m3(x / sc);
  }
}

template <int SF, int KF>
__global__ void __launch_bounds__(kWriteThreads) cache_write_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const uint8_t* src = is_v ? a.v : a.k;
  uint8_t* dst = is_v ? a.value_cache : a.key_cache;
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * a.head_dim;
  // this thread's 16-byte vector (float caches) or 16-element chunk (one-byte
  // caches) of the row
  const int64_t c = static_cast<int64_t>(blockIdx.z) * kWriteThreads + threadIdx.x;
  if constexpr (!pkv_dev::scaled_format(KF)) {
    static_assert(SF == KF, "float caches take rows of their own format");
    const int64_t vecs = row_elems * Format<KF>::kBytes / 16;
    const uint4* s4 = reinterpret_cast<const uint4*>(src) + t * vecs;
    uint4* d4 = reinterpret_cast<uint4*>(dst) + static_cast<int64_t>(slot) * vecs;
    if (c < vecs) d4[c] = s4[c];
  } else {
    const float* scales = is_v ? a.v_scales : a.k_scales;
    const int blk = slot / a.block_size;
    constexpr int kSrcVecs = 16 * Format<SF>::kBytes / 16;  // uint4s per 16 elements
    const int64_t chunks = row_elems / 16;
    const uint4* s4 = reinterpret_cast<const uint4*>(src) + t * chunks * kSrcVecs;
    uint4* d4 = reinterpret_cast<uint4*>(dst) + static_cast<int64_t>(slot) * chunks;
    if (c < chunks) {
      const int kvh = static_cast<int>(c * 16 / a.head_dim);
      const float sc = scales[static_cast<int64_t>(blk) * a.num_kv_heads + kvh];
      float x[16];
#pragma unroll
      for (int v = 0; v < kSrcVecs; ++v) unpack16<SF>(s4[c * kSrcVecs + v], x + v * (16 / kSrcVecs));
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e / 4] |= quantise_byte<KF>(x[e], sc) << (8 * (e % 4));
      d4[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Row slices per (token, K or V): one thread per 16-byte vector of a float
// row, or per 16 elements of a one-byte row.
template <int SF, int KF>
int64_t write_slices(const CacheWriteArgs& a) {
  const int64_t row_elems = static_cast<int64_t>(a.num_kv_heads) * a.head_dim;
  const int64_t per_row = pkv_dev::scaled_format(KF) ? row_elems / 16
                                                     : row_elems * Format<KF>::kBytes / 16;
  return (per_row + kWriteThreads - 1) / kWriteThreads;
}

template <int SF, int KF>
hipError_t launch_write(const CacheWriteArgs& a, int num_tokens, hipStream_t s) {
  const int64_t slices = write_slices<SF, KF>(a);
  if (slices > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((cache_write_kernel<SF, KF>), dim3(num_tokens, 2, static_cast<unsigned>(slices)),
                     dim3(kWriteThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Whole-block copies: copy-on-write (device to device) and swapping (device
// to pinned host and back, through the host memory's device mapping).  Pairs
// travel by value in the kernel arguments, so no host-to-device transfer of
// the pair list is needed.
constexpr int kPairsPerLaunch = 192;
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyChunk = kCopyThreads * 16 * kCopyUnroll;  // bytes per workgroup

struct CopyBlocksArgs {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  const float* src_ks;  // scales, NULL for float caches
  const float* src_vs;
  float* dst_ks;
  float* dst_vs;
  int64_t block_bytes;
  int scale_stride;
  int n;
  int32_t src[kPairsPerLaunch];
  int32_t dst[kPairsPerLaunch];
};

// 16-byte store with the non-temporal hint.  Measured on the block copies:
// 32 blocks of 512 KiB took 17.8 us with ordinary stores and 4.4 us with
// these; 192 blocks 35.4 us and 29.8 us.
__device__ __forceinline__ void store_stream16(uint4* p, const uint4& v) {
  const pkv_dev::u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<pkv_dev::u32x4_t*>(p));
}

// Grid (pair, chunk of the block, K or V).  Every thread issues its loads
// before its stores, so a workgroup keeps kCopyUnroll 16-byte requests per
// lane in flight (this matters when the source sits across PCIe).
template <bool kStreamStore>
__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(CopyBlocksArgs a) {
  const int p = blockIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * kCopyChunk;
  const bool is_v = blockIdx.z != 0;
  const uint4* s = reinterpret_cast<const uint4*>((is_v ? a.src_v : a.src_k) +
                                                  a.src[p] * a.block_bytes + c0);
  uint4* d = reinterpret_cast<uint4*>((is_v ? a.dst_v : a.dst_k) + a.dst[p] * a.block_bytes + c0);
  int64_t nvec = (a.block_bytes - c0) / 16;
  if (nvec > kCopyChunk / 16) nvec = kCopyChunk / 16;
  const int i0 = threadIdx.x;
  if (nvec == kCopyChunk / 16) {
    uint4 r[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) r[u] = s[i0 + u * kCopyThreads];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      if (kStreamStore)
        store_stream16(&d[i0 + u * kCopyThreads], r[u]);
      else
        d[i0 + u * kCopyThreads] = r[u];
    }
  } else {
    for (int64_t i = i0; i < nvec; i += kCopyThreads) {
      if (kStreamStore)
        store_stream16(&d[i], s[i]);
      else
        d[i] = s[i];
    }
  }
  const float* ss = is_v ? a.src_vs : a.src_ks;
  float* ds = is_v ? a.dst_vs : a.dst_ks;
  if (ss && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < a.scale_stride; i += kCopyThreads)
      ds[static_cast<int64_t>(a.dst[p]) * a.scale_stride + i] =
          ss[static_cast<int64_t>(a.src[p]) * a.scale_stride + i];
  }
}

// Checks shared by the block copies: ids in range, destinations distinct.
int check_pairs(const int32_t* pairs, int n_pairs, int num_src, int num_dst,
                std::vector<char>* is_dst_out) {
  std::vector<char> is_dst(num_dst, 0);
  for (int i = 0; i < n_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_src || d < 0 || d >= num_dst)
      return pkv::fail(PKV_ERR_INVALID_ARG, "pair %d (%d, %d) outside [0, %d) x [0, %d)", i, s, d,
                       num_src, num_dst);
    if (is_dst[d]) return pkv::fail(PKV_ERR_INVALID_ARG, "block %d is a destination twice", d);
    is_dst[d] = 1;
  }
  if (is_dst_out) is_dst_out->swap(is_dst);
  return PKV_OK;
}

int launch_block_copies(CopyBlocksArgs a, const int32_t* pairs, int n_pairs, bool stream_store,
                        hipStream_t st) {
  const int64_t chunks = (a.block_bytes + kCopyChunk - 1) / kCopyChunk;
  if (chunks > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "block_bytes too large");
  for (int base = 0; base < n_pairs; base += kPairsPerLaunch) {
    a.n = n_pairs - base < kPairsPerLaunch ? n_pairs - base : kPairsPerLaunch;
    for (int i = 0; i < a.n; ++i) {
      a.src[i] = pairs[2 * (base + i)];
      a.dst[i] = pairs[2 * (base + i) + 1];
    }
    const dim3 grid(a.n, static_cast<unsigned>(chunks), 2);
    if (stream_store)
      hipLaunchKernelGGL(copy_blocks_kernel<true>, grid, dim3(kCopyThreads), 0, st, a);
    else
      hipLaunchKernelGGL(copy_blocks_kernel<false>, grid, dim3(kCopyThreads), 0, st, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return pkv::fail(PKV_ERR_HIP, "copy launch: %s", hipGetErrorString(err));
  }
  return PKV_OK;
}

// Device address of pinned host memory (NULL stays NULL).
int host_mapping(void* host, const char* what, void** dev) {
  *dev = nullptr;
  if (!host) return PKV_OK;
  const hipError_t err = hipHostGetDevicePointer(dev, host, 0);
  if (err != hipSuccess || !*dev) {
    (void)hipGetLastError();  // clear the sticky error left by the failed query
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s is not pinned host memory (hipHostMalloc): %s", what,
                     hipGetErrorString(err));
  }
  return PKV_OK;
}

// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ void __launch_bounds__(kStreamThreads) stream_copy_kernel(uint4* __restrict__ dst,
                                                                     const uint4* __restrict__ src,
                                                                     int64_t nvec) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kStreamThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kStreamThreads + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * stride < nvec; i += kStreamUnroll * stride) {
    uint4 r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) r[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) dst[i + u * stride] = r[u];
  }
  for (; i < nvec; i += stride) dst[i] = src[i];
}

// Read-only streaming probe with the decode's loads (16-byte, non-temporal).
// Each workgroup reads one contiguous stretch of the buffer, kReadUnroll
// 4 KiB pieces in flight: measured on MI355X over 2 GiB, 7.0-7.1 TB/s, against
// 6.2-6.3 TB/s when the whole grid sweeps the buffer together (each
// workgroup's pieces a grid's width apart).  Each thread folds what it read
// with XOR and stores the fold to the sink only if it equals the sentinel, a
// run-time value, so no load can be dropped.
constexpr int kReadUnroll = 16;

__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint4* __restrict__ src,
                                                                     int64_t nvec, uint32_t* sink,
                                                                     uint32_t sentinel) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < nvec ? b0 + per : nvec;
  int64_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * kStreamThreads < b1; i += kReadUnroll * kStreamThreads) {
    u32x4 r[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + u * kStreamThreads));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (; i < b1; i += kStreamThreads) {
    const uint4 r = src[i];
    acc ^= r.x ^ r.y ^ r.z ^ r.w;
  }
  if (acc == sentinel) *sink = acc;
}

}  // namespace

extern "C" {

int pkv_reshape_and_cache(const void* k, const void* v, void* key_cache, void* value_cache,
                          const float* k_scales, const float* v_scales,
                          const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, int src_dtype,
                          int kv_dtype, void* stream) {
  PKV_API_BEGIN
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad shape: tokens=%d kv_heads=%d head_dim=%d "
                     "block_size=%d num_blocks=%d", num_tokens, num_kv_heads, head_dim,
                     block_size, num_blocks);
  if (num_tokens == 0) return PKV_OK;
  if (num_tokens > 65535 * 1024) return pkv::fail(PKV_ERR_INVALID_ARG, "too many tokens");
  if (!k || !v || !key_cache || !value_cache || !slot_mapping)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (head_dim % 16) return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d not a multiple of 16", head_dim);
  CacheWriteArgs a;
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.key_cache = static_cast<uint8_t*>(key_cache);
  a.value_cache = static_cast<uint8_t*>(value_cache);
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.slots = slot_mapping;
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (kv_dtype == PKV_I8) {
    if (!k_scales || !v_scales) return pkv::fail(PKV_ERR_INVALID_ARG, "int8 cache needs scales");
    switch (src_dtype) {
      case PKV_F32: err = launch_write<PKV_F32, PKV_I8>(a, num_tokens, s); break;
      case PKV_F16: err = launch_write<PKV_F16, PKV_I8>(a, num_tokens, s); break;
      case PKV_BF16: err = launch_write<PKV_BF16, PKV_I8>(a, num_tokens, s); break;
      default: return pkv::fail(PKV_ERR_INVALID_ARG, "int8 cache takes F32/F16/BF16 rows");
    }
  } else if (kv_dtype == PKV_FP8) {
    if (!k_scales || !v_scales) return pkv::fail(PKV_ERR_INVALID_ARG, "fp8 cache needs scales");
    switch (src_dtype) {
      case PKV_F32: err = launch_write<PKV_F32, PKV_FP8>(a, num_tokens, s); break;
      case PKV_F16: err = launch_write<PKV_F16, PKV_FP8>(a, num_tokens, s); break;
      case PKV_BF16: err = launch_write<PKV_BF16, PKV_FP8>(a, num_tokens, s); break;
      default: return pkv::fail(PKV_ERR_INVALID_ARG, "fp8 cache takes F32/F16/BF16 rows");
    }
  } else {
    if (src_dtype != kv_dtype)
      return pkv::fail(PKV_ERR_INVALID_ARG, "float cache format %d takes rows of the same "
                       "format (got %d)", kv_dtype, src_dtype);
    switch (kv_dtype) {
      case PKV_F32: err = launch_write<PKV_F32, PKV_F32>(a, num_tokens, s); break;
      case PKV_F16: err = launch_write<PKV_F16, PKV_F16>(a, num_tokens, s); break;
      case PKV_BF16: err = launch_write<PKV_BF16, PKV_BF16>(a, num_tokens, s); break;
      default: return pkv::fail(PKV_ERR_INVALID_ARG, "unknown cache format %d", kv_dtype);
    }
  }
  if (err != hipSuccess) return pkv::fail(PKV_ERR_HIP, "cache write launch: %s", hipGetErrorString(err));
  return PKV_OK;
  PKV_API_END
}

int pkv_copy_blocks(void* key_cache, void* value_cache, float* k_scales, float* v_scales,
                    const int32_t* pairs, int n_pairs, size_t block_bytes, int num_blocks,
                    int scale_stride, void* stream) {
  PKV_API_BEGIN
  if (n_pairs < 0 || num_blocks <= 0 || block_bytes == 0 || block_bytes % 16)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or block_bytes (%zu, multiple of 16)", block_bytes);
  if (n_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !pairs) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if ((k_scales != nullptr) != (v_scales != nullptr) || (k_scales && scale_stride <= 0))
    return pkv::fail(PKV_ERR_INVALID_ARG, "scales must be given together with scale_stride > 0");
  std::vector<char> is_dst;
  if (int rc = check_pairs(pairs, n_pairs, num_blocks, num_blocks, &is_dst)) return rc;
  for (int i = 0; i < n_pairs; ++i)
    if (is_dst[pairs[2 * i]])
      return pkv::fail(PKV_ERR_INVALID_ARG, "block %d is both source and destination", pairs[2 * i]);
  CopyBlocksArgs a;
  a.src_k = a.dst_k = static_cast<uint8_t*>(key_cache);
  a.src_v = a.dst_v = static_cast<uint8_t*>(value_cache);
  a.src_ks = a.dst_ks = k_scales;
  a.src_vs = a.dst_vs = v_scales;
  a.block_bytes = static_cast<int64_t>(block_bytes);
  a.scale_stride = scale_stride;
  return launch_block_copies(a, pairs, n_pairs, true, static_cast<hipStream_t>(stream));
  PKV_API_END
}

int pkv_swap_blocks(void* key_cache, void* value_cache, float* k_scales, float* v_scales,
                    void* host_key, void* host_value, float* host_k_scales, float* host_v_scales,
                    const int32_t* pairs, int n_pairs, size_t block_bytes, int num_blocks,
                    int num_host_blocks, int scale_stride, int direction, void* stream) {
  PKV_API_BEGIN
  if (n_pairs < 0 || num_blocks <= 0 || num_host_blocks <= 0 || block_bytes == 0 ||
      block_bytes % 16)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad count, pool size or block_bytes (%zu, multiple "
                     "of 16)", block_bytes);
  if (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN)
    return pkv::fail(PKV_ERR_INVALID_ARG, "direction %d is neither PKV_SWAP_OUT nor PKV_SWAP_IN",
                     direction);
  if (n_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !host_key || !host_value || !pairs)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if ((k_scales != nullptr) != (v_scales != nullptr) ||
      (k_scales != nullptr) != (host_k_scales != nullptr) ||
      (k_scales != nullptr) != (host_v_scales != nullptr) || (k_scales && scale_stride <= 0))
    return pkv::fail(PKV_ERR_INVALID_ARG, "device and host scales must be given together, "
                     "with scale_stride > 0");
  if (reinterpret_cast<uintptr_t>(host_key) % 16 || reinterpret_cast<uintptr_t>(host_value) % 16)
    return pkv::fail(PKV_ERR_INVALID_ARG, "host pools must be 16-byte aligned");
  const bool out = direction == PKV_SWAP_OUT;
  if (int rc = check_pairs(pairs, n_pairs, out ? num_blocks : num_host_blocks,
                           out ? num_host_blocks : num_blocks, nullptr))
    return rc;
  void *hk, *hv, *hks, *hvs;
  if (int rc = host_mapping(host_key, "host_key", &hk)) return rc;
  if (int rc = host_mapping(host_value, "host_value", &hv)) return rc;
  if (int rc = host_mapping(host_k_scales, "host_k_scales", &hks)) return rc;
  if (int rc = host_mapping(host_v_scales, "host_v_scales", &hvs)) return rc;
  CopyBlocksArgs a;
  uint8_t* dk = static_cast<uint8_t*>(key_cache);
  uint8_t* dv = static_cast<uint8_t*>(value_cache);
  uint8_t* mk = static_cast<uint8_t*>(hk);
  uint8_t* mv = static_cast<uint8_t*>(hv);
  a.src_k = out ? dk : mk;
  a.src_v = out ? dv : mv;
  a.dst_k = out ? mk : dk;
  a.dst_v = out ? mv : dv;
  a.src_ks = out ? k_scales : static_cast<float*>(hks);
  a.src_vs = out ? v_scales : static_cast<float*>(hvs);
  a.dst_ks = out ? static_cast<float*>(hks) : k_scales;
  a.dst_vs = out ? static_cast<float*>(hvs) : v_scales;
  a.block_bytes = static_cast<int64_t>(block_bytes);
  a.scale_stride = scale_stride;
#ifndef PKV_SWAP_OUT_STREAM_STORE
#define PKV_SWAP_OUT_STREAM_STORE 0
#endif
  const bool stream_store = !out || PKV_SWAP_OUT_STREAM_STORE;
  return launch_block_copies(a, pairs, n_pairs, stream_store, static_cast<hipStream_t>(stream));
  PKV_API_END
}

int pkv_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  PKV_API_BEGIN
  if (bytes == 0) return PKV_OK;
  if (!dst || !src || bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16 ||
      reinterpret_cast<uintptr_t>(src) % 16)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL or misaligned pointer, or size not a multiple of 16");
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  int64_t blocks = (nvec + kStreamThreads * kStreamUnroll - 1) / (kStreamThreads * kStreamUnroll);
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), nvec);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return pkv::fail(PKV_ERR_HIP, "copy launch: %s", hipGetErrorString(err));
  return PKV_OK;
  PKV_API_END
}

int pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t sentinel,
                    void* stream) {
  PKV_API_BEGIN
  if (bytes == 0) return PKV_OK;
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL or misaligned pointer, or size not a multiple of 16");
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  // 8192 workgroups (32 per CU): stretches of 256 KiB over 2 GiB
  int64_t blocks = (nvec + kStreamThreads * kReadUnroll - 1) / (kStreamThreads * kReadUnroll);
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), nvec, sink,
                     sentinel);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return pkv::fail(PKV_ERR_HIP, "read launch: %s", hipGetErrorString(err));
  return PKV_OK;
  PKV_API_END
}

}  // extern "C"
