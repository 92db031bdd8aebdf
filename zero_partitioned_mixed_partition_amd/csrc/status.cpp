// Status strings, thread-local error detail, and per-device properties.
#include <hip/hip_runtime_api.h>

#include <array>
#include <mutex>
#include <string>

#include "internal.hpp"

namespace {
thread_local std::string g_last_error;
}

namespace zero {

zero_status fail(zero_status st, const std::string& detail) {
    g_last_error = detail;
    return st;
}

zero_status check_hip(int hip_error, const char* what) {
    if (hip_error == hipSuccess) return ZERO_OK;
    return fail(ZERO_EHIP, std::string(what) + ": " +
                               hipGetErrorString(static_cast<hipError_t>(hip_error)));
}

void clear_error() { g_last_error.clear(); }

int device_cu_count() {
    static std::mutex mu;
    static std::array<int, 64> cache{};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

}  // namespace zero

extern "C" const char* zero_status_string(zero_status status) {
    switch (status) {
        case ZERO_OK: return "ok";
        case ZERO_EINVAL: return "invalid argument";
        case ZERO_ERANGE: return "size out of range";
        case ZERO_ENOMEM: return "out of host memory";
        case ZERO_EHIP: return "HIP runtime error";
        case ZERO_ENOSPACE: return "workspace or output capacity too small";
    }
    return "unknown status";
}

extern "C" const char* zero_last_error(void) { return g_last_error.c_str(); }
