// Thread-local error message behind pwg_last_error().
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pwg_internal.h"

namespace pwg {
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

}  // namespace pwg

extern "C" const char* pwg_last_error(void) { return pwg::g_last_error.c_str(); }
extern "C" int pwg_version(void) { return PWG_VERSION; }
