// Error reporting shared by the host and device halves of libpa.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"

namespace pa {

// Thread-local message behind pa_last_error().
std::string& last_error_slot();

// Records a printf-style message and returns `code`, so call sites read
// `return fail(PA_ERR_INVALID_ARG, "...", ...);`.
inline pa_status fail(pa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return code;
}

inline pa_status ok() {
  last_error_slot().clear();
  return PA_OK;
}

}  // namespace pa
