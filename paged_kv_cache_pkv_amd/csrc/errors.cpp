// Thread-local last-error message for the C ABI.
#include <string>

#include "pkv.h"
#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {
void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1 gfx950"; }
