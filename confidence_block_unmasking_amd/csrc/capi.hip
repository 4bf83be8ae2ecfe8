// Host-side helpers of the C ABI: error text, HIP error mapping, device property cache.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.h"

namespace dllm {

static thread_local char g_err[512];

dllm_status fail(dllm_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

dllm_status check_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return DLLM_OK;
    return fail(DLLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace dllm

extern "C" const char *dllm_last_error(void) { return dllm::g_err; }
