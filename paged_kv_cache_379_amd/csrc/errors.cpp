// Thread-local error reporting of the C ABI.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" int pkv_abi_version(void) { return 4; }
