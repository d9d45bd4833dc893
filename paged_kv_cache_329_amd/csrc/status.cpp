#include "status.h"

#include <cstdarg>
#include <cstdio>
#include <string>

namespace pkv {
namespace {
thread_local std::string g_last_error;
}

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }
extern "C" int pkv_abi_version(void) { return PKV_ABI_VERSION; }
