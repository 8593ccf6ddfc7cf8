#include "errors.h"

#include <cstdarg>
#include <cstdio>
#include <string>

#include "splash.h"

namespace splash {
namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace splash

extern "C" const char* splash_last_error(void) {
  return splash::g_last_error.c_str();
}

extern "C" int splash_version(void) { return SPLASH_VERSION; }
