// Status codes and the thread-local error text of libpa (host only, no HIP): every entry point
// returns a pa_status and leaves the detail of a failure in a per-thread buffer.
#include <cstdio>

#include "pa.h"
#include "pa_internal.h"

namespace {
thread_local char g_err[512];
}  // namespace

pa_status pa_fail(pa_status st, const char* msg) {
  std::snprintf(g_err, sizeof g_err, "%s", msg);
  return st;
}

pa_status pa_ok() {
  g_err[0] = '\0';
  return PA_OK;
}

extern "C" {

const char* pa_status_str(int32_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID";
    case PA_ERR_OOM: return "PA_ERR_OOM";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_err; }

int32_t pa_version(void) { return (2 << 16) | 3; }

}  // extern "C"
