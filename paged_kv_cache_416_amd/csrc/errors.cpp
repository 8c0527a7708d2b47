// Thread-local last-error text and HIP status translation.
#include <cstdio>
#include <string>

#include "common.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return PKV_OK;
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace pkv

extern "C" const char *pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char *pkv_version(void) { return "pkv 0.1 gfx950"; }
