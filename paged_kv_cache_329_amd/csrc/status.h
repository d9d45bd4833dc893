// Thread-local error message behind pkv_last_error() and helpers that set it.
#pragma once

#include "pagedkv.h"

namespace pkv {

// Records a printf-style message for pkv_last_error() and returns `s`.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace pkv
