// Status and error-message plumbing shared by the C-ABI translation units.
#pragma once

#include <hip/hip_runtime_api.h>

#include "mt.h"

namespace mt {

// Records a printf-style message as this thread's last error; returns s.
mt_status set_error(mt_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace mt

#define MT_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t mt_e_ = (expr);                                                         \
    if (mt_e_ != hipSuccess)                                                           \
      return ::mt::set_error(MT_E_HIP, "%s failed: %s", #expr, hipGetErrorString(mt_e_)); \
  } while (0)

#define MT_CHECK(cond, status, ...)                                \
  do {                                                             \
    if (!(cond)) return ::mt::set_error((status), __VA_ARGS__);    \
  } while (0)
