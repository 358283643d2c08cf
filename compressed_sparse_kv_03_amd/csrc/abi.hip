// Library-wide C ABI: version, error strings, thread-local error text.
#include "host_util.h"
#include <string.h>

namespace cskv {
static thread_local char g_err[512];
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}
}  // namespace cskv

extern "C" CSKV_API int cskv_abi_version(void) { return CSKV_ABI_VERSION; }

extern "C" CSKV_API const char* cskv_strerror(int code) {
  switch (code) {
    case CSKV_OK: return "ok";
    case CSKV_EINVAL: return "invalid argument";
    case CSKV_ENOTSUP: return "shape not supported";
    case CSKV_EWORKSPACE: return "workspace missing or too small";
    case CSKV_EHIP: return "HIP launch failure";
    default: return "unknown error code";
  }
}

extern "C" CSKV_API const char* cskv_last_error(void) { return cskv::g_err; }
