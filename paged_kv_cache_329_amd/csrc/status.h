// Thread-local error message behind pkv_last_error() and helpers that set it.
#pragma once

#include <cstdint>
#include <initializer_list>

#include "pagedkv.h"

namespace pkv {

// Records a printf-style message for pkv_last_error() and returns `s`.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// The events set by pkv_set_launch_events for this thread (hipEvent_t handles, either may
// be null); clears the setting.  Returns true if any was set.
bool take_launch_events(void** start, void** stop);

// True when every non-null pointer is 16-byte aligned (the kernels move 16-byte chunks).
inline bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return false;
  return true;
}

}  // namespace pkv
