#include "status.h"

#include <cstdarg>
#include <cstdio>
#include <string>

namespace pkv {
namespace {
thread_local std::string g_last_error;
// Events the next measured kernel launched on this thread records (pkv_set_launch_events).
thread_local void* g_launch_start = nullptr;
thread_local void* g_launch_stop = nullptr;
}  // namespace

bool take_launch_events(void** start, void** stop) {
  *start = g_launch_start;
  *stop = g_launch_stop;
  g_launch_start = g_launch_stop = nullptr;
  return *start != nullptr || *stop != nullptr;
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

extern "C" pkv_status pkv_set_launch_events(void* start_event, void* stop_event) {
  pkv::g_launch_start = start_event;
  pkv::g_launch_stop = stop_event;
  return PKV_OK;
}
