// Status codes and the per-thread last-error message of the C ABI.
#include <cstdio>

#include "lvsa_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace lvsa {

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return LVSA_OK;
}

}  // namespace lvsa

extern "C" const char *lvsa_last_error(void) { return g_msg; }

extern "C" int lvsa_version(void) { return LVSA_ABI_VERSION; }
