// Status codes and thread-local error detail of the C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "moe_common.h"

namespace {
thread_local char g_detail[512] = "";
}

namespace moe {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return status;
}

int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace moe

extern "C" int moe_abi_version(void) { return 4; }

extern "C" const char* moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" const char* moe_last_error_detail(void) { return g_detail; }
