// Per-thread error message of the last failed entry point, and the ABI version.
#include "pa_error.h"

#include <cstdio>

#include "../../include/pagedkv.h"

namespace {
thread_local char g_msg[512] = {0};
}

namespace pagedkv {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pagedkv

extern "C" const char* pa_last_error(void) { return g_msg; }

extern "C" int32_t pa_abi_version(void) { return 8; }
