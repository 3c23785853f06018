// Thread-local last-error message for the C ABI.
#include <string>

#include "pkv.h"
#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {
// A message that cannot be stored (no host memory) leaves the previous one;
// the status code still reports the failure.
void set_error(const std::string& msg) {
  try {
    g_last_error = msg;
  } catch (...) {
  }
}
void clear_error() { g_last_error.clear(); }
}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1 gfx950"; }
