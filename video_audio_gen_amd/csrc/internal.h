// Internal helpers shared by the host translation units of the library.
#pragma once

#include <stdarg.h>

namespace dit {
// Record a thread-local error message and return `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
}  // namespace dit
