// Internal helpers shared by the host and device translation units of the
// draft-head library (not part of the public ABI).
#pragma once

#include <stdint.h>

namespace dh {

// Record `msg` as the calling thread's last error and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's last error and return DH_OK.
int ok();

}  // namespace dh
