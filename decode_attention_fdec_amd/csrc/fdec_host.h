// Host-side helpers shared by the libfdec translation units: the thread-local
// error message behind fdec_last_error().
#pragma once

#include <cstdarg>

void fdec_clear_error();
// Records a printf-style message for fdec_last_error() and returns `status`.
int fdec_fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
