// Error reporting of the C ABI (host code): a failed call returns a negative
// kv_status and leaves a message for kv_last_error() on the calling thread.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "errors.h"
#include "pagedkv.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace pagedkv {

kv_status report(kv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

kv_status report_ok() {
  g_last_error.clear();
  return KV_OK;
}

}  // namespace pagedkv

extern "C" const char* kv_last_error(void) { return g_last_error.c_str(); }
