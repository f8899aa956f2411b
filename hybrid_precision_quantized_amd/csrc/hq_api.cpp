// Status strings, thread-local error messages and the ABI version.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "hq_common.h"

namespace hq {
namespace {
thread_local std::string g_last_error;
}

hq_status fail(hq_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

hq_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  clear_error();
  return HQ_OK;
}

}  // namespace hq

extern "C" const char *hq_status_string(hq_status s) {
  switch (static_cast<int>(s)) {
    case HQ_OK: return "ok";
    case HQ_ERR_INVALID_ARG: return "invalid argument";
    case HQ_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HQ_ERR_WORKSPACE: return "workspace too small";
    case HQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char *hq_last_error(void) { return hq::g_last_error.c_str(); }

extern "C" int hq_abi_version(void) { return HQ_ABI_VERSION; }
