// Error reporting for the C ABI (one message per calling thread).
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.h"

namespace {
thread_local std::string g_last_error;
}

namespace graft {

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GRAFT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return GRAFT_OK;
}

void clear_error() { g_last_error.clear(); }

}  // namespace graft

extern "C" const char *graft_last_error(void) { return g_last_error.c_str(); }
extern "C" int graft_version(void) { return 1; }
