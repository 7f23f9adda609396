// Status reporting shared by every translation unit of libpagedkv (host code only).
#pragma once
#include <cstdint>

#include "pagedkv.h"

namespace pkv {

// Records a printf-style message as this thread's last error and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pkv
