// Per-thread error message shared by the C-ABI entry points.
#pragma once

namespace splash {

// Records a printf-style message for splash_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the calling thread's message (start of every entry point).
void clear_error();

}  // namespace splash
