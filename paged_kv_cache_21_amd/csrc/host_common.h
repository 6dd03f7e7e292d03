// Host-side helpers shared by the C-ABI translation units: error reporting and
// argument checks.  No device code here.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

// Thread-local message behind pkv_last_error().
void set_error_message(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

template <typename... A>
inline pkv_status fail(pkv_status s, const char* fmt, A... args) {
  set_error_message(fmt, args...);
  return s;
}

inline pkv_status fail(pkv_status s, const char* msg) {
  set_error_message("%s", msg);
  return s;
}

}  // namespace pkv
