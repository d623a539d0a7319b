// Internal helpers shared by the library's translation units (not installed).
#pragma once
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

#include "kvd.h"

namespace kvd {

// Record `code` and a printf-style message as this thread's last error and
// return `code` (so callers can write `return fail(KVD_EINVAL, "...")`).
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Forget the last error (called at the top of every entry point).
void clear_error();

}  // namespace kvd
