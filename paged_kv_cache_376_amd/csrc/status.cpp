// Status strings and the thread-local last-error message of the C ABI.
#include <cstdio>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  try {
    g_last_error = std::string(pkv_status_string(s)) + ": " + buf;
  } catch (...) {  // no host memory even for the message: keep the status, drop the text
  }
  return s;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARGUMENT: return "PKV_ERR_INVALID_ARGUMENT";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    case PKV_ERR_NOT_FOUND: return "PKV_ERR_NOT_FOUND";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "PKV_ERR_WORKSPACE_TOO_SMALL";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_ALREADY_EXISTS: return "PKV_ERR_ALREADY_EXISTS";
    case PKV_ERR_HOST_MEMORY: return "PKV_ERR_HOST_MEMORY";
    default: return "PKV_ERR_UNKNOWN";
  }
}

extern "C" const char* pkv_version(void) { return "pagedkv 0.1.0 (gfx950)"; }
