// Thread-local error text behind pkv_last_error().
#include "status.h"

#include <cstdarg>
#include <cstdio>

namespace {
thread_local char g_last_error[512] = "";
}

namespace pkv {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error; }

extern "C" int32_t pkv_version(void) { return 100; }  // 0.1.0
