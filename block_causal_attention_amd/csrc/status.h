// Internal helpers shared by the host sources of libmagi_bca: the per-thread
// error message behind magi_last_error().
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "magi_bca.h"

namespace magi {

std::string& last_error_slot();

inline int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return code;
}

inline int32_t ok() {
  last_error_slot().clear();
  return MAGI_OK;
}

}  // namespace magi
