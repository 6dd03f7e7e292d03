// Error-message plumbing for the host-only sanitizer build of tests/native/host_stress.cpp
// (the library keeps these beside its device dispatch, which that build leaves out).
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {
thread_local std::string g_msg;
void set_error_message(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_msg = buf;
}
void clear_error() { g_msg.clear(); }
}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_msg.c_str(); }
extern "C" pkv_status pkv_copy_blocks_memcpy(int32_t, void* const*, const void* const*, const int64_t*, int64_t,
                                             int64_t, const int32_t*, const int32_t*, int32_t, void*) {
  return PKV_ERR_INVALID;  // device copies are not part of the host-only build
}
