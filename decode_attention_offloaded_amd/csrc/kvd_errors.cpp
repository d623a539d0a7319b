// Thread-local error text behind kvd_last_error(), and the version string.
#include <stdio.h>

#include "kvd_internal.h"

namespace kvd {
namespace {
thread_local char g_last_error[512];
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace kvd

extern "C" const char* kvd_last_error(void) { return kvd::g_last_error; }

extern "C" const char* kvd_version(void) { return "kvd 0.1.0 gfx950"; }
