// Where a buffer handed to a kernel lives: device memory, or page-locked host memory that HIP
// maps into the device's address space at the same address (a kernel then reads and writes it
// over the bus).  Pageable host memory is rejected, so no kernel is launched on an address the
// device cannot reach.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_status.h"

namespace pa {

// *host = true for page-locked host memory, false for device memory; an error otherwise.
inline pa_status memory_kind(const char* who, const char* what, const void* p, bool* host) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARG, "%s: %s is neither device memory nor page-locked host memory",
                who, what);
  }
  if (at.type == hipMemoryTypeHost) {
    if (at.devicePointer != p || at.hostPointer != p)
      return fail(PA_ERR_INVALID_ARG, "%s: page-locked %s is not mapped at its host address", who,
                  what);
    *host = true;
    return ok();
  }
  if (at.type == hipMemoryTypeUnregistered)
    return fail(PA_ERR_INVALID_ARG, "%s: %s is pageable host memory", who, what);
  *host = false;
  return ok();
}

}  // namespace pa
