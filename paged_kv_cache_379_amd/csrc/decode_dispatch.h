// Launch helpers for the decode kernels: one instantiation per (cache format,
// query format, head_dim, group size).  Each decode_<format>.hip file
// instantiates the kernels of one cache format so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "decode_gqa_kernel.h"
#include "decode_kernel.h"

namespace pkv_dev {

constexpr int kDecodeWaves = 4;
constexpr int kMaxGroup = 16;  // query heads per kv head, padded to one 16-wide MFMA tile

// Returns hipSuccess and sets ok = false when the combination is not built.
// Multi-head attention (group 1) and fp32 caches run on the vector ALUs;
// grouped-query attention with 16-bit, int8 or fp8 caches runs on the matrix
// cores.
template <int KF, int QF, int D>
hipError_t launch_decode_groups(int group, const DecodeArgs& a, unsigned grid, hipStream_t s,
                                bool& ok) {
  ok = true;
  const dim3 g(grid), b(kDecodeWaves * 64);
  if constexpr (KF == PKV_F32) {
    switch (group) {
      case 1: hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 1, kDecodeWaves>), g, b, 0, s, a); break;
      case 2: hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 2, kDecodeWaves>), g, b, 0, s, a); break;
      case 4: hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 4, kDecodeWaves>), g, b, 0, s, a); break;
      case 8: hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 8, kDecodeWaves>), g, b, 0, s, a); break;
      case 16: hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 16, kDecodeWaves>), g, b, 0, s, a); break;
      default: ok = false; return hipSuccess;
    }
  } else {
    if (group == 1) {
      hipLaunchKernelGGL((paged_decode_kernel<KF, QF, D, 1, kDecodeWaves>), g, b, 0, s, a);
    } else if (group >= 2 && group <= 8) {
      hipLaunchKernelGGL((paged_decode_gqa_kernel<KF, QF, D, kDecodeWaves, true>),
                         g, b, 0, s, a);
    } else if (group > 8 && group <= kMaxGroup) {
      hipLaunchKernelGGL((paged_decode_gqa_kernel<KF, QF, D, kDecodeWaves, false>),
                         g, b, 0, s, a);
    } else {
      ok = false;
      return hipSuccess;
    }
  }
  return hipGetLastError();
}

template <int KF, int QF>
hipError_t launch_decode_dims(int head_dim, int group, const DecodeArgs& a, unsigned grid,
                              hipStream_t s, bool& ok) {
  if (head_dim == 64) return launch_decode_groups<KF, QF, 64>(group, a, grid, s, ok);
  if (head_dim == 128) return launch_decode_groups<KF, QF, 128>(group, a, grid, s, ok);
  ok = false;
  return hipSuccess;
}

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
