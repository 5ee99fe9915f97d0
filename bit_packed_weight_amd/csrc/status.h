// Thread-local error text behind bpw_last_error().
#pragma once

namespace bpw {

// Record a formatted error for this thread and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear this thread's error and return BPW_OK.
int ok();

}  // namespace bpw
