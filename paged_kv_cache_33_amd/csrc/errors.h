// Error reporting shared by the C ABI's translation units: a failed call
// returns a negative kv_status and leaves a message for kv_last_error() on the
// calling thread.
#pragma once

#include "pagedkv.h"

namespace pagedkv {

// Record a printf-style message for kv_last_error() and return `code`.
kv_status report(kv_status code, const char* fmt, ...);
// Clear the message and return KV_OK.
kv_status report_ok();

}  // namespace pagedkv
