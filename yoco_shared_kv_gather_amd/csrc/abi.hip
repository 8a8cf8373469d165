// Version, status strings and per-thread error messages of the C ABI.
#include <cstdarg>
#include <cstdio>

#include "yoco_internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace yoco {

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int32_t launch_result(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    return fail(YOCO_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(err));
  }
  return YOCO_OK;
}

}  // namespace yoco

extern "C" {

int32_t yoco_abi_version(void) { return YOCO_ABI_VERSION; }

const char* yoco_status_string(int32_t status) {
  switch (status) {
    case YOCO_OK: return "ok";
    case YOCO_ERR_INVALID_ARGUMENT: return "invalid argument";
    case YOCO_ERR_UNSUPPORTED: return "unsupported shape";
    case YOCO_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case YOCO_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* yoco_last_error_message(void) { return g_last_error; }

}  // extern "C"
