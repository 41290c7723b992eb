// Decode kernels for FP8 (E4M3) caches with per-(block, kv head) scales
// (queries in F16 or BF16).
#include "decode_dispatch.h"

namespace pkv_dev {

hipError_t launch_decode_fp8(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok) {
  if (q_dtype == PKV_F16) return launch_decode_dims<PKV_FP8, PKV_F16>(head_dim, group, a, grid, s, ok);
  if (q_dtype == PKV_BF16) return launch_decode_dims<PKV_FP8, PKV_BF16>(head_dim, group, a, grid, s, ok);
  ok = false;
  return hipSuccess;
}

hipError_t launch_prefix_fp8(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                             unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok) {
  if (q_dtype == PKV_F16)
    return launch_prefix_dims<PKV_FP8, PKV_F16>(head_dim, group, pa, n_prefix, n_rest, s, ok);
  if (q_dtype == PKV_BF16)
    return launch_prefix_dims<PKV_FP8, PKV_BF16>(head_dim, group, pa, n_prefix, n_rest, s, ok);
  ok = false;
  return hipSuccess;
}

}  // namespace pkv_dev
