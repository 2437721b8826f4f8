// Library-wide entry points: version and thread-local error text.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace dsa {

static thread_local char g_last_error[512] = "";

void set_last_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

dsa_status_t launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_error("%s: %s", what, hipGetErrorString(e));
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

}  // namespace dsa

extern "C" int dsa_version(void) { return 100; }

extern "C" const char* dsa_last_error(void) { return dsa::g_last_error; }
