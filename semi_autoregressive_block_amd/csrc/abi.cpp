// Library-wide entry points: version and the per-thread last-error string.
#include <string.h>

#include "common.h"

namespace {
thread_local char g_last_error[512] = {0};
}

namespace dspark_host {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = 0;
  return DSPARK_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace dspark_host

extern "C" int dspark_version(void) { return 100; }

extern "C" const char* dspark_last_error(void) { return g_last_error; }
