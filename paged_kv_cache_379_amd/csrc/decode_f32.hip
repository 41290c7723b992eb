// Decode kernels for F32-format caches (queries in F32).
#include "decode_dispatch.h"

namespace pkv_dev {

hipError_t launch_decode_f32(int q_dtype, int head_dim, int group, const DecodeArgs& a,
                             unsigned grid, hipStream_t s, bool& ok) {
  if (q_dtype == PKV_F32) return launch_decode_dims<PKV_F32, PKV_F32>(head_dim, group, a, grid, s, ok);
  ok = false;
  return hipSuccess;
}

}  // namespace pkv_dev
