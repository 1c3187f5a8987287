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

// Readers of the translation units' device error words (see common.h): a
// fixed table filled by static initialisers at library load, before any call.
static ErrorReader g_readers[32];
static int g_nreaders = 0;

int register_error_reader(ErrorReader f) {
  if (g_nreaders < 32) g_readers[g_nreaders] = f;
  return g_nreaders++;
}

}  // namespace nsa

extern "C" int nsa_check_device_errors(void* stream) {
  using namespace nsa;
  NSA_REQUIRE(g_nreaders <= 32, NSA_ERR_LAUNCH,
              "nsa_check_device_errors: %d error words, table holds 32", g_nreaders);
  uint32_t all = 0;
  for (int i = 0; i < g_nreaders; ++i) {
    uint32_t bits = 0;
    if (g_readers[i]((hipStream_t)stream, &bits) != 0) {
      const hipError_t e = hipGetLastError();
      return set_error(NSA_ERR_LAUNCH, "nsa_check_device_errors: %s",
                       hipGetErrorString(e));
    }
    all |= bits;
  }
  ok();
  return (int)(all & 0x7FFFFFFFu);
}

extern "C" const char* nsa_last_error(void) { return nsa::g_last_error; }

extern "C" int nsa_version(void) { return 200; }  // 0.2.0
