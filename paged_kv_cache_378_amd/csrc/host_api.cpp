// Library-wide entry points: error message and ABI version.
#include <string>

#include "pa.h"
#include "pa_status.h"

namespace pa {
std::string& last_error_slot() {
  thread_local std::string msg;
  return msg;
}
}  // namespace pa

extern "C" const char* pa_last_error(void) { return pa::last_error_slot().c_str(); }

extern "C" int32_t pa_abi_version(void) { return 3; }
