// Launch helpers for the decode kernels: one instantiation per (cache format,
// query format, head_dim, group size).  Each decode_<format>.hip file
// instantiates the kernels of one cache format so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "decode_gqa_kernel.h"
#include "decode_kernel.h"
#include "decode_prefix_kernel.h"

namespace pkv_dev {

constexpr int kDecodeWaves = 4;
constexpr int kMaxGroup = 16;  // query heads per kv head, padded to one 16-wide MFMA tile

// Returns hipSuccess and sets ok = false when the combination is not built.
// Multi-head attention (group 1) and fp32 caches run on the vector ALUs;
// grouped-query attention with 16-bit, int8 or fp8 caches runs on the matrix
// cores.
template <int KF, int QF, int D, int G, int BS>
hipError_t launch_vector(const DecodeArgs& a, unsigned grid, hipStream_t s, bool& ok) {
  // One-byte rows of head_dim 64 are half a 128-byte line: with an even
  // number of kv heads per workgroup, each load row covers two neighbouring
  // heads (HR = 2).
  if constexpr (G == 1 && Format<KF>::kBytes == 1 && D == 64) {
    if (a.heads_per_item % 2 == 0) {
      ok = true;
      hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, G, kDecodeWaves, BS, 2>), dim3(grid),
                         dim3(kDecodeWaves * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (DecodeTile<KF, QF, D, G, kDecodeWaves, BS>::kBuilt) {
    ok = true;
    hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, G, kDecodeWaves, BS>), dim3(grid),
                       dim3(kDecodeWaves * 64), 0, s, a);
    return hipGetLastError();
  } else {
    ok = false;
    return hipSuccess;
  }
}

template <int KF, int QF, int D, int BS>
hipError_t launch_decode_groups(int group, const DecodeArgs& a, unsigned grid, hipStream_t s,
                                bool& ok) {
  ok = true;
  const dim3 g(grid), b(kDecodeWaves * 64);
  if constexpr (KF == PKV_F32) {
    switch (group) {
      case 1: return launch_vector<KF, QF, D, 1, BS>(a, grid, s, ok);
      case 2: return launch_vector<KF, QF, D, 2, BS>(a, grid, s, ok);
      case 4: return launch_vector<KF, QF, D, 4, BS>(a, grid, s, ok);
      case 8: return launch_vector<KF, QF, D, 8, BS>(a, grid, s, ok);
      case 16: return launch_vector<KF, QF, D, 16, BS>(a, grid, s, ok);
      default: ok = false; return hipSuccess;
    }
  } else {
    if (group == 1) return launch_vector<KF, QF, D, 1, BS>(a, grid, s, ok);
    if (group >= 2 && group <= 8) {
      hipLaunchKernelGGL((paged_decode_gqa_kernel<KF, QF, D, kDecodeWaves, true, BS>), g, b, 0, s, a);
    } else if (group > 8 && group <= kMaxGroup) {
      hipLaunchKernelGGL((paged_decode_gqa_kernel<KF, QF, D, kDecodeWaves, false, BS>), g, b, 0, s, a);
    } else {
      ok = false;
      return hipSuccess;
    }
  }
  return hipGetLastError();
}

template <int KF, int QF, int D>
hipError_t launch_decode_block(int group, int block_size, const DecodeArgs& a, unsigned grid,
                               hipStream_t s, bool& ok) {
  switch (block_size) {
    case 8: return launch_decode_groups<KF, QF, D, 8>(group, a, grid, s, ok);
    case 16: return launch_decode_groups<KF, QF, D, 16>(group, a, grid, s, ok);
    case 32: return launch_decode_groups<KF, QF, D, 32>(group, a, grid, s, ok);
    default: ok = false; return hipSuccess;
  }
}

template <int KF, int QF>
hipError_t launch_decode_dims(int head_dim, int group, const DecodeArgs& a, unsigned grid,
                              hipStream_t s, bool& ok) {
  if (head_dim == 64) return launch_decode_block<KF, QF, 64>(group, a.block_size, a, grid, s, ok);
  if (head_dim == 128) return launch_decode_block<KF, QF, 128>(group, a.block_size, a, grid, s, ok);
  ok = false;
  return hipSuccess;
}

// The shared-prefix kernel (16-bit, int8 and fp8 caches; matrix cores):
// n_prefix prefix work items alone (n_rest = 0), or together with the n_rest
// grouped-query decode items of the rest of each context in one launch.
template <int KF, int QF, int D, int BS>
hipError_t launch_prefix_bs(int group, const PrefixArgs& pa, unsigned n_prefix, unsigned n_rest,
                            hipStream_t s, bool& ok) {
  ok = true;
  const dim3 b(kPrefixWaves * 64);
  if (n_rest == 0) {
    hipLaunchKernelGGL((paged_prefix_kernel<KF, QF, D, BS>), dim3(n_prefix), b, 0, s, pa);
  } else if (group >= 2 && group <= 8) {
    hipLaunchKernelGGL((paged_prefix_fused_kernel<KF, QF, D, true, BS>), dim3(n_prefix + n_rest), b,
                       0, s, pa, static_cast<int>(n_prefix));
  } else if (group > 8 && group <= kMaxGroup) {
    hipLaunchKernelGGL((paged_prefix_fused_kernel<KF, QF, D, false, BS>), dim3(n_prefix + n_rest),
                       b, 0, s, pa, static_cast<int>(n_prefix));
  } else {
    ok = false;
    return hipSuccess;
  }
  return hipGetLastError();
}

template <int KF, int QF, int D>
hipError_t launch_prefix_block(int group, const PrefixArgs& pa, unsigned n_prefix,
                               unsigned n_rest, hipStream_t s, bool& ok) {
  switch (pa.d.block_size) {
    case 8: return launch_prefix_bs<KF, QF, D, 8>(group, pa, n_prefix, n_rest, s, ok);
    case 16: return launch_prefix_bs<KF, QF, D, 16>(group, pa, n_prefix, n_rest, s, ok);
    case 32: return launch_prefix_bs<KF, QF, D, 32>(group, pa, n_prefix, n_rest, s, ok);
    default: ok = false; return hipSuccess;
  }
}

template <int KF, int QF>
hipError_t launch_prefix_dims(int head_dim, int group, const PrefixArgs& pa, unsigned n_prefix,
                              unsigned n_rest, hipStream_t s, bool& ok) {
  if (head_dim == 64) return launch_prefix_block<KF, QF, 64>(group, pa, n_prefix, n_rest, s, ok);
  if (head_dim == 128) return launch_prefix_block<KF, QF, 128>(group, pa, n_prefix, n_rest, s, ok);
  ok = false;
  return hipSuccess;
}

// Defined in decode_f16.hip, decode_bf16.hip, decode_i8.hip, decode_fp8.hip.
hipError_t launch_prefix_f16(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                             unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok);
hipError_t launch_prefix_bf16(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                              unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok);
hipError_t launch_prefix_i8(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                            unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok);
hipError_t launch_prefix_fp8(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                             unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok);

// Defined in decode_f32.hip, decode_f16.hip, decode_bf16.hip, decode_i8.hip,
// decode_fp8.hip.
hipError_t launch_decode_f32(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok);
hipError_t launch_decode_f16(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok);
hipError_t launch_decode_bf16(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                              unsigned grid, hipStream_t s, bool& ok);
hipError_t launch_decode_i8(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                            unsigned grid, hipStream_t s, bool& ok);
hipError_t launch_decode_fp8(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok);

}  // namespace pkv_dev
