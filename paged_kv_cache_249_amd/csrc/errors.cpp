// Host-side error text of libpagedkv: every call that fails records a message
// for pa_last_error() on the calling thread. Kept apart from the HIP sources
// so that the host block managers link without a GPU toolchain.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;
}  // namespace

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return pa::g_last_error.c_str(); }

int32_t pa_version(void) { return 200; }

}  // extern "C"
