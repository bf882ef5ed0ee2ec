// Per-thread error message shared by the translation units of libpagedkv.
#pragma once

#include <cstdarg>

namespace pagedkv {

// Formats the message for pa_last_error() and returns `status` for tail calls.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the message (called at the start of every entry point).
void clear_error();

}  // namespace pagedkv
