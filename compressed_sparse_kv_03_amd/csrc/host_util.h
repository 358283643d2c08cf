// Host-side helpers: thread-local error text, argument checks, launch checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdarg.h>
#include "cskv.h"

namespace cskv {

void set_error(const char* fmt, ...);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace cskv

#define CSKV_REQUIRE(cond, code, ...)         \
  do {                                        \
    if (!(cond)) {                            \
      ::cskv::set_error(__VA_ARGS__);         \
      return (code);                          \
    }                                         \
  } while (0)

#define CSKV_LAUNCH_CHECK(what)                                                    \
  do {                                                                             \
    hipError_t e_ = hipGetLastError();                                             \
    if (e_ != hipSuccess) {                                                        \
      ::cskv::set_error("%s: HIP launch failed: %s", (what), hipGetErrorString(e_)); \
      return CSKV_EHIP;                                                            \
    }                                                                              \
  } while (0)
