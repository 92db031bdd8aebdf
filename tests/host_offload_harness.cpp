// Host-only check of zero_offload_adamw_step's pipeline logic (work split,
// slot reuse, per-chunk waits, error paths), built without a GPU. The HIP
// calls the pipeline makes are replaced by synchronous host stand-ins: a copy
// happens when it is queued, an event wait returns after a short random delay,
// and a chosen call can be made to fail. Built with ThreadSanitizer when the
// platform allows it. Prints "bad=<mismatches> copy_fail=<k>/<n> wait_fail=<k>/<n>".
#define target_clones(...) used   // one plain host variant is enough here
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

static std::atomic<int> g_copies{0}, g_copy_fail_at{-1}, g_waits{0}, g_wait_fail_at{-1};

static void jitter() {
    thread_local std::mt19937 rng(static_cast<unsigned>(std::hash<std::thread::id>()(std::this_thread::get_id())));
    std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
}

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    static int x[4];
    static int i = 0;
    *s = reinterpret_cast<hipStream_t>(&x[i++ % 4]);
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { *e = reinterpret_cast<hipEvent_t>(new int(0)); return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { delete reinterpret_cast<int*>(e); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) {
    jitter();
    const int k = ++g_waits;
    return (g_wait_fail_at >= 0 && k == g_wait_fail_at) ? hipErrorInvalidValue : hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* d, const void* s, size_t b, hipMemcpyKind, hipStream_t) {
    const int k = ++g_copies;
    if (g_copy_fail_at >= 0 && k == g_copy_fail_at) return hipErrorInvalidValue;
    std::memcpy(d, s, b);
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "host stand-in"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) { *n = 4; return hipSuccess; }
}

#include "offload.cpp"

static int run_case(int64_t n, int64_t chunk, int threads) {
    std::vector<float> p(n), m(n, 0.f), v(n, 0.f);
    std::vector<uint16_t> g(n), out(n, 0), out2(n, 0), staging(4 * chunk);
    for (int64_t i = 0; i < n; ++i) {
        p[i] = 0.001f * static_cast<float>((i * 7919) % 2001 - 1000);
        g[i] = static_cast<uint16_t>(0x3a00 + (i * 31) % 500);
    }
    std::vector<float> p2 = p, m2 = m, v2 = v;
    for (int t = 1; t <= 3; ++t) {
        if (zero_offload_adamw_step(p.data(), m.data(), v.data(), g.data(), out.data(), staging.data(),
                                    4 * chunk, n, t, 1e-3, 0.9, 0.999, 1e-8, 0.01, nullptr, threads,
                                    nullptr) != ZERO_OK)
            return 1;
        if (zero_host_adamw_step(p2.data(), m2.data(), v2.data(), g.data(), out2.data(), n, t, 1e-3,
                                 0.9, 0.999, 1e-8, 0.01, 1.0f, 1) != ZERO_OK)
            return 1;
    }
    return std::memcmp(p.data(), p2.data(), n * 4) || std::memcmp(m.data(), m2.data(), n * 4) ||
           std::memcmp(v.data(), v2.data(), n * 4) || std::memcmp(out.data(), out2.data(), n * 2);
}

static bool failed_call(int copy_at, int wait_at) {
    const int64_t n = 300007, chunk = 4096;
    std::vector<float> p(n, 0.1f), m(n), v(n);
    std::vector<uint16_t> g(n, 0x3a00), out(n), staging(4 * chunk);
    g_copies = 0;
    g_waits = 0;
    g_copy_fail_at = copy_at;
    g_wait_fail_at = wait_at;
    const zero_status st = zero_offload_adamw_step(p.data(), m.data(), v.data(), g.data(), out.data(),
                                                   staging.data(), 4 * chunk, n, 1, 1e-3, 0.9, 0.999,
                                                   1e-8, 0.01, nullptr, 16, nullptr);
    g_copy_fail_at = -1;
    g_wait_fail_at = -1;
    return st == ZERO_EHIP;
}

int main() {
    int bad = 0;
    for (int64_t n : {1, 1000, 65537, 300007, 2000003})
        for (int64_t chunk : {257, 4096, 65536, 1 << 20})
            for (int threads : {1, 3, 16}) bad += run_case(n, chunk, threads);
    int copy_fail = 0, copy_n = 0, wait_fail = 0, wait_n = 0;
    for (int k = 1; k <= 40; k += 3, ++copy_n) copy_fail += failed_call(k, -1);
    for (int k = 1; k <= 60; k += 7, ++wait_n) wait_fail += failed_call(-1, k);
    std::printf("bad=%d copy_fail=%d/%d wait_fail=%d/%d\n", bad, copy_fail, copy_n, wait_fail, wait_n);
    return bad != 0;
}
