// Internal declarations shared by the host-side sources of libpkv.so.
#pragma once

#include <cstddef>
#include <cstdint>
#include <new>

#include "pkv.h"

namespace pkv {

// Record a failure for pkv_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Bytes per stored element of a PKV_* format, 0 if unknown.
inline int elem_bytes(int fmt) {
  switch (fmt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_I8: return 1;
    case PKV_FP8: return 1;
    default: return 0;
  }
}

}  // namespace pkv

// Every exported function body runs inside these: the thread's error message
// is cleared on entry and no C++ exception escapes through the C ABI.
#define PKV_API_BEGIN \
  pkv::clear_error(); \
  try {
#define PKV_API_END                                                   \
  }                                                                   \
  catch (const std::bad_alloc&) {                                     \
    return pkv::fail(PKV_ERR_INVALID_ARG, "host allocation failed");  \
  }                                                                   \
  catch (...) {                                                       \
    return pkv::fail(PKV_ERR_INVALID_ARG, "unexpected internal error"); \
  }
