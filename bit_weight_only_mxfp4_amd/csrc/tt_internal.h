// tt_internal.h -- host-side helpers shared by the entry points: the
// thread-local error message, argument checks and launch-error reporting.
#pragma once

#include <stdint.h>

#include "../../include/tt.h"

namespace tt {

// Record a failure for tt_last_error() and return its status.
tt_status fail(tt_status s, const char *fmt, ...);
// Clear the message at the start of a successful call.
void clear_error();

// Argument checks; each returns TT_OK or records and returns the failure.
tt_status check_ptr(const void *p, const char *name);
tt_status check_align(const void *p, int64_t align, const char *name);
tt_status check_range(int64_t v, int64_t lo, int64_t hi, const char *name);
tt_status check_dtype(int32_t d, const char *name);

}  // namespace tt

#define TT_TRY(expr)                 \
    do {                             \
        tt_status _st = (expr);      \
        if (_st != TT_OK) return _st; \
    } while (0)
