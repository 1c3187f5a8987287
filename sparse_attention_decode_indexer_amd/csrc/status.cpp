// Thread-local last-error string and library version.
#include "common.h"

namespace nsa {

static thread_local char g_last_error[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return NSA_OK;
}

}  // namespace nsa

extern "C" const char* nsa_last_error(void) { return nsa::g_last_error; }

extern "C" int nsa_version(void) { return 100; }  // 0.1.0
