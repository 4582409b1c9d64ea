// api.hip -- version and per-thread error reporting of the C ABI.
#include <string>

#include "internal.hpp"

namespace {
thread_local std::string g_last_error;
}

namespace moe {

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return MOE_OK;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace moe

extern "C" int moe_version(void) { return 200; }

extern "C" const char* moe_last_error(void) { return g_last_error.c_str(); }
