// abi.cpp -- version, error reporting, status names, format descriptions and
// the argument checks every entry point uses.
#include <stdarg.h>
#include <stdio.h>

#include "tt_internal.h"

namespace tt {

static thread_local char g_err[512];

tt_status fail(tt_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = 0; }

tt_status check_ptr(const void *p, const char *name) {
    if (!p) return fail(TT_E_NULL, "%s is NULL", name);
    return TT_OK;
}

tt_status check_align(const void *p, int64_t align, const char *name) {
    if (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(align))
        return fail(TT_E_ALIGN, "%s must be %lld-byte aligned", name,
                    static_cast<long long>(align));
    return TT_OK;
}

tt_status check_range(int64_t v, int64_t lo, int64_t hi, const char *name) {
    if (v < lo || v > hi)
        return fail(TT_E_SHAPE, "%s = %lld is outside [%lld, %lld]", name,
                    static_cast<long long>(v), static_cast<long long>(lo),
                    static_cast<long long>(hi));
    return TT_OK;
}

tt_status check_dtype(int32_t d, const char *name) {
    if (d != TT_F32 && d != TT_BF16)
        return fail(TT_E_DTYPE, "%s = %d is not TT_F32 or TT_BF16", name, d);
    return TT_OK;
}

}  // namespace tt

extern "C" {

int32_t tt_abi_version(void) { return TT_ABI_VERSION; }

const char *tt_last_error(void) { return tt::g_err; }

const char *tt_status_str(tt_status s) {
    switch (s) {
        case TT_OK: return "TT_OK";
        case TT_E_NULL: return "TT_E_NULL";
        case TT_E_SHAPE: return "TT_E_SHAPE";
        case TT_E_ALIGN: return "TT_E_ALIGN";
        case TT_E_DTYPE: return "TT_E_DTYPE";
        case TT_E_SIZE: return "TT_E_SIZE";
        case TT_E_RANGE: return "TT_E_RANGE";
        case TT_E_HIP: return "TT_E_HIP";
        default: return "TT_E_UNKNOWN";
    }
}

tt_status tt_format_info(int32_t format, int32_t *bits, int32_t *group,
                         int32_t *scale_kind, int32_t *has_zero) {
    int32_t b, g, sk, hz;
    if (format == TT_FMT_MXFP4) {
        b = 4; g = 32; sk = TT_SCALE_E8M0; hz = 0;
    } else if (format == TT_FMT_INT4_AFFINE) {
        b = 4; g = TT_INT4_GROUP; sk = TT_SCALE_F16; hz = 1;
    } else {
        return tt::fail(TT_E_DTYPE, "unknown weight format %d", format);
    }
    if (bits) *bits = b;
    if (group) *group = g;
    if (scale_kind) *scale_kind = sk;
    if (has_zero) *has_zero = hz;
    tt::clear_error();
    return TT_OK;
}

}  // extern "C"
