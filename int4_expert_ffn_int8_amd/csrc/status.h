// Thread-local error reporting for the C ABI.
#pragma once

#include <stdarg.h>
#include <stdio.h>

#include "../../include/moe.h"

namespace moe {

inline char* last_error_buffer() {
  static thread_local char buf[512] = {0};
  return buf;
}

inline moe_status_t fail(moe_status_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(last_error_buffer(), 512, fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace moe

using moe::fail;
