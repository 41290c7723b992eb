// Decode kernels for BF16-format caches (queries in BF16).
#include "decode_dispatch.h"

namespace pkv_dev {

hipError_t launch_decode_bf16(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok) {
  if (q_dtype == PKV_BF16) return launch_decode_dims<PKV_BF16, PKV_BF16>(head_dim, group, a, grid, s, ok);
  ok = false;
  return hipSuccess;
}

hipError_t launch_prefix_bf16(int q_dtype, int head_dim, int group, const PrefixArgs& pa,
                              unsigned n_prefix, unsigned n_rest, hipStream_t s, bool& ok) {
  if (q_dtype == PKV_BF16)
    return launch_prefix_dims<PKV_BF16, PKV_BF16>(head_dim, group, pa, n_prefix, n_rest, s, ok);
  ok = false;
  return hipSuccess;
}

}  // namespace pkv_dev
