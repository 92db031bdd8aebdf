// ZeRO-Offload step: fp32 AdamW on the host CPU, bf16 gradients in from the GPU
// and bf16 parameters back out, in overlapped chunks.
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "ZeRO-Offload Mechanics": the forward
// and backward passes stay on the GPU; gradients go to host DRAM over PCIe /
// CXL, the host runs the fp32 Adam step and updates the fp32 weights, and the
// parameters go back. The next section ("Communication Bandwidth Limits across
// Memory Biers", sic: tiers) has the parameter transfer overlap the optimizer.
//
// The host update applies exactly the device kernel's per-element operations
// (same order, IEEE fp32, no contraction, correctly rounded / and sqrt, the
// same bf16 rounding), so host and device steps give identical bits. The loop
// is compiled for AVX-512, AVX2 and baseline x86-64 and picked at load time;
// vector / and sqrt are IEEE-exact on all of them.
#include <hip/hip_runtime_api.h>

#include <sched.h>

#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace {

struct HostScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, step_size, sqrt_bc2, decay, clip;
};

inline uint16_t host_bf16(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

inline float host_widen(uint16_t h) {
    const uint32_t u = static_cast<uint32_t>(h) << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return x;
}

__attribute__((target_clones("avx512f", "avx2", "default")))
void host_adamw_range(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
                      const uint16_t* __restrict__ g, uint16_t* __restrict__ out, int64_t n,
                      const HostScalars c) {
    for (int64_t i = 0; i < n; ++i) {
        const float gi = host_widen(g[i]) * c.clip;
        const float bm = c.beta1 * m[i];
        const float gm = c.one_minus_beta1 * gi;
        const float mi = bm + gm;
        const float bv = c.beta2 * v[i];
        const float gg = gi * gi;
        const float gv = c.one_minus_beta2 * gg;
        const float vi = bv + gv;
        float pi = p[i] * c.decay;
        const float root = std::sqrt(vi);
        const float denom = root / c.sqrt_bc2 + c.eps;
        const float ratio = mi / denom;
        pi = pi - c.step_size * ratio;
        m[i] = mi;
        v[i] = vi;
        p[i] = pi;
        out[i] = host_bf16(pi);
    }
}

// A persistent pool of host workers: the offload pipeline runs one parallel
// update per chunk, many per step, and starting threads for each would cost
// more than a chunk's arithmetic. run() hands out `tasks` task indices; the
// caller's thread takes part and returns once every task has finished and no
// worker is still inside the hand-out loop (so the next run cannot be mixed
// with this one). Runs are serialised on run_mu_.
class HostPool {
  public:
    static HostPool& get() {
        static HostPool pool(affinity_cpus());
        return pool;
    }
    // Threads that can run tasks at the same time (the workers and the caller).
    int concurrency() const { return static_cast<int>(workers_.size()) + 1; }
    void run(int tasks, const std::function<void(int)>& fn) {
        std::lock_guard<std::mutex> serial(run_mu_);
        if (tasks <= 1 || workers_.empty()) {
            for (int t = 0; t < tasks; ++t) fn(t);
            return;
        }
        {
            std::unique_lock<std::mutex> lock(mu_);
            done_cv_.wait(lock, [&] { return active_ == 0; });   // late wakers of the last run
            fn_ = &fn;
            tasks_ = tasks;
            next_.store(0);
            pending_ = tasks;
            ++generation_;
        }
        cv_.notify_all();
        const int done = drain();
        std::unique_lock<std::mutex> lock(mu_);
        pending_ -= done;
        done_cv_.wait(lock, [&] { return pending_ == 0 && active_ == 0; });
        fn_ = nullptr;
    }
    ~HostPool() {
        {
            std::lock_guard<std::mutex> lock(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& w : workers_) w.join();
    }

    static int affinity_cpus() {
        cpu_set_t set;
        CPU_ZERO(&set);
        if (sched_getaffinity(0, sizeof(set), &set) == 0) {
            const int n = CPU_COUNT(&set);
            if (n > 0) return n;
        }
        const unsigned hw = std::thread::hardware_concurrency();
        return hw > 0 ? static_cast<int>(hw) : 1;
    }

  private:
    explicit HostPool(int threads) {
        for (int i = 1; i < threads; ++i) workers_.emplace_back([this] { loop(); });
    }
    // Takes task indices until none are left; returns how many it ran. tasks_
    // and fn_ stay fixed while any thread is in here (run() waits for that).
    int drain() {
        int done = 0;
        for (int t; (t = next_.fetch_add(1)) < tasks_; ++done) (*fn_)(t);
        return done;
    }
    void loop() {
        uint64_t seen = 0;
        for (;;) {
            {
                std::unique_lock<std::mutex> lock(mu_);
                cv_.wait(lock, [&] { return stop_ || generation_ != seen; });
                if (stop_) return;
                seen = generation_;
                ++active_;
            }
            const int done = drain();
            std::lock_guard<std::mutex> lock(mu_);
            pending_ -= done;
            --active_;
            if (active_ == 0) done_cv_.notify_all();
        }
    }

    std::vector<std::thread> workers_;
    std::mutex run_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int)>* fn_ = nullptr;
    std::atomic<int> next_{0};
    int tasks_ = 0, pending_ = 0, active_ = 0;
    uint64_t generation_ = 0;
    bool stop_ = false;
};

void host_adamw_parallel(float* p, float* m, float* v, const uint16_t* g, uint16_t* out,
                         int64_t n, const HostScalars& c, int threads) {
    if (threads <= 1 || n < (int64_t(1) << 16)) {
        host_adamw_range(p, m, v, g, out, n, c);
        return;
    }
    // 64-element pieces keep every task's start on a cache line of each array.
    const int64_t per = ((n + threads - 1) / threads + 63) / 64 * 64;
    const int tasks = static_cast<int>((n + per - 1) / per);
    HostPool::get().run(tasks, [=, &c](int t) {
        const int64_t lo = t * per;
        const int64_t len = n - lo < per ? n - lo : per;
        host_adamw_range(p + lo, m + lo, v + lo, g + lo, out + lo, len, c);
    });
}

zero_status make_scalars(int64_t step, double lr, double beta1, double beta2, double eps,
                         double weight_decay, HostScalars* c, const char* who) {
    using zero::fail;
    if (step < 1) return fail(ZERO_EINVAL, std::string(who) + ": step must be >= 1");
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
        return fail(ZERO_EINVAL, std::string(who) + ": betas must lie in [0, 1)");
    if (!(eps > 0.0) || !std::isfinite(eps))
        return fail(ZERO_EINVAL, std::string(who) + ": eps must be finite and > 0");
    if (!(lr >= 0.0) || !std::isfinite(lr) || !std::isfinite(weight_decay))
        return fail(ZERO_EINVAL, std::string(who) + ": lr and weight_decay must be finite, lr >= 0");
    const double bc1 = 1.0 - std::pow(beta1, static_cast<double>(step));
    const double bc2 = 1.0 - std::pow(beta2, static_cast<double>(step));
    if (!(bc1 > 0.0) || !(bc2 > 0.0))
        return fail(ZERO_EINVAL, std::string(who) + ": bias correction is zero");
    c->beta1 = static_cast<float>(beta1);
    c->one_minus_beta1 = static_cast<float>(1.0 - beta1);
    c->beta2 = static_cast<float>(beta2);
    c->one_minus_beta2 = static_cast<float>(1.0 - beta2);
    c->eps = static_cast<float>(eps);
    c->step_size = static_cast<float>(lr / bc1);
    c->sqrt_bc2 = static_cast<float>(std::sqrt(bc2));
    c->decay = static_cast<float>(1.0 - lr * weight_decay);
    c->clip = 1.0f;
    return ZERO_OK;
}

// 0 requests one task per CPU this process may run on.
int default_threads(int32_t requested) {
    return requested > 0 ? requested : HostPool::affinity_cpus();
}

// Two copy streams per device (default priority), made once.
struct CopyStreams {
    hipStream_t d2h = nullptr, h2d = nullptr;
};

zero_status copy_streams(CopyStreams* out) {
    static std::mutex mu;
    static CopyStreams per_dev[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return zero::fail(ZERO_EHIP, "zero_offload_adamw_step: no current device");
    std::lock_guard<std::mutex> lock(mu);
    CopyStreams& s = per_dev[dev];
    if (s.d2h == nullptr) {
        zero_status st = zero::check_hip(hipStreamCreateWithFlags(&s.d2h, hipStreamNonBlocking),
                                         "zero_offload_adamw_step: stream");
        if (st != ZERO_OK) return st;
        st = zero::check_hip(hipStreamCreateWithFlags(&s.h2d, hipStreamNonBlocking),
                             "zero_offload_adamw_step: stream");
        if (st != ZERO_OK) return st;
    }
    *out = s;
    return ZERO_OK;
}

// The offload pipeline as dataflow, one pool run per call. Worker w owns
// slice w of every chunk and walks the chunks in order: it waits until the
// chunk's gradients have landed in their staging slot (and, from chunk 2 on,
// until the parameters of the chunk two back have left the parameter slot it
// is about to fill), updates its slice, and counts the chunk done. The worker
// that completes a chunk queues that chunk's parameter copy, and the gradient
// copy of the chunk two ahead into the slot just freed. Nothing joins the
// workers between chunks; a worker blocks only on data that has not arrived.
struct Pipeline {
    int64_t n = 0, chunk = 0, chunks = 0;
    int tasks = 1;
    float *p = nullptr, *m = nullptr, *v = nullptr;
    const uint16_t* d_grad = nullptr;
    uint16_t* d_param = nullptr;
    uint16_t* gstage[2] = {nullptr, nullptr};
    uint16_t* pstage[2] = {nullptr, nullptr};
    hipStream_t d2h = nullptr, h2d = nullptr;
    hipEvent_t ev_in[2] = {nullptr, nullptr}, ev_out[2] = {nullptr, nullptr};
    HostScalars c{};
    std::mutex mu;                      // guards everything below
    std::condition_variable cv;
    std::vector<int> done;              // workers finished, per chunk
    std::vector<uint8_t> in_queued;     // gradient copy and its event queued, per chunk
    std::vector<uint8_t> out_queued;    // parameter copy and its event queued, per chunk
    // Per chunk: 0 nobody has waited for the copy's event yet, 1 one worker is
    // waiting for it, 2 the copy has completed. Exactly one worker calls the
    // HIP wait per event (the runtime serialises concurrent waits: ~7 us per
    // call from 16 threads, against 0.1 us from one); the others wait here.
    std::vector<uint8_t> in_state, out_state;
    zero_status status = ZERO_OK;       // first failure; every worker stops on it

    int64_t len(int64_t k) const { return n - k * chunk < chunk ? n - k * chunk : chunk; }

    // Called with mu held (or before the workers start).
    void queue_in(int64_t k) {
        if (status != ZERO_OK) return;
        const int s = static_cast<int>(k % 2);
        hipError_t e = hipMemcpyAsync(gstage[s], d_grad + k * chunk, len(k) * sizeof(uint16_t),
                                      hipMemcpyDeviceToHost, d2h);
        if (e == hipSuccess) e = hipEventRecord(ev_in[s], d2h);
        if (e != hipSuccess) {
            status = zero::check_hip(e, "zero_offload_adamw_step: grad copy");
            return;
        }
        in_queued[static_cast<size_t>(k)] = 1;
    }
    // Returns once chunk k's copy behind `ev` has completed (false on failure).
    bool await_copy(std::vector<uint8_t>& state, int64_t k, hipEvent_t ev) {
        const size_t i = static_cast<size_t>(k);
        std::unique_lock<std::mutex> lock(mu);
        if (state[i] == 0) {
            state[i] = 1;
            lock.unlock();
            const hipError_t e = hipEventSynchronize(ev);
            lock.lock();
            if (e != hipSuccess && status == ZERO_OK)
                status = zero::check_hip(e, "zero_offload_adamw_step: copy wait");
            state[i] = 2;
            cv.notify_all();
        } else {
            cv.wait(lock, [&] { return status != ZERO_OK || state[i] == 2; });
        }
        return status == ZERO_OK;
    }

    void worker(int w) {
        for (int64_t k = 0; k < chunks; ++k) {
            const int s = static_cast<int>(k % 2);
            {
                std::unique_lock<std::mutex> lock(mu);
                cv.wait(lock, [&] {
                    return status != ZERO_OK ||
                           (in_queued[static_cast<size_t>(k)] && (k < 2 || out_queued[static_cast<size_t>(k - 2)]));
                });
                if (status != ZERO_OK) return;
            }
            if (!await_copy(in_state, k, ev_in[s])) return;
            if (k >= 2 && !await_copy(out_state, k - 2, ev_out[s])) return;
            const int64_t off = k * chunk, lk = len(k);
            // 64-element pieces keep every slice's start on a cache line of each array.
            const int64_t per = ((lk + tasks - 1) / tasks + 63) / 64 * 64;
            const int64_t lo = w * per;
            if (lo < lk) {
                const int64_t cnt = lk - lo < per ? lk - lo : per;
                host_adamw_range(p + off + lo, m + off + lo, v + off + lo, gstage[s] + lo,
                                 pstage[s] + lo, cnt, c);
            }
            std::lock_guard<std::mutex> lock(mu);
            if (++done[static_cast<size_t>(k)] < tasks) continue;
            if (status != ZERO_OK) return;
            hipError_t e = hipMemcpyAsync(d_param + off, pstage[s], lk * sizeof(uint16_t), hipMemcpyHostToDevice, h2d);
            if (e == hipSuccess) e = hipEventRecord(ev_out[s], h2d);
            if (e != hipSuccess) {
                status = zero::check_hip(e, "zero_offload_adamw_step: param copy");
            } else {
                out_queued[static_cast<size_t>(k)] = 1;
                if (k + 2 < chunks) queue_in(k + 2);
            }
            cv.notify_all();
        }
    }
};

}  // namespace

extern "C" zero_status zero_host_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                            const uint16_t* grad, uint16_t* param_out, int64_t n,
                                            int64_t step, double lr, double beta1, double beta2,
                                            double eps, double weight_decay, float clip_scale,
                                            int32_t n_threads) {
    using zero::fail;
    zero::clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "zero_host_adamw_step: n < 0");
    HostScalars c;
    zero_status st = make_scalars(step, lr, beta1, beta2, eps, weight_decay, &c,
                                  "zero_host_adamw_step");
    if (st != ZERO_OK) return st;
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad || !param_out)
        return fail(ZERO_EINVAL, "zero_host_adamw_step: NULL array");
    {
        const size_t fb = static_cast<size_t>(n) * 4, hb = static_cast<size_t>(n) * 2;
        const zero::Span wr[] = {{master, fb, "master"}, {exp_avg, fb, "exp_avg"},
                                 {exp_avg_sq, fb, "exp_avg_sq"}, {param_out, hb, "param_out"}};
        const zero::Span rd[] = {{grad, hb, "grad"}};
        const std::string clash = zero::first_overlap(wr, 4, rd, 1);
        if (!clash.empty()) return fail(ZERO_EINVAL, "zero_host_adamw_step: " + clash);
    }
    if (!std::isfinite(clip_scale)) return ZERO_OK;        // a non-finite norm skips the step
    c.clip = clip_scale;
    host_adamw_parallel(master, exp_avg, exp_avg_sq, grad, param_out, n, c,
                        default_threads(n_threads));
    return ZERO_OK;
}

extern "C" zero_status zero_offload_adamw_step(float* h_master, float* h_exp_avg,
                                               float* h_exp_avg_sq, const uint16_t* d_grad,
                                               uint16_t* d_param_out, uint16_t* h_staging,
                                               int64_t staging_elems, int64_t n, int64_t step,
                                               double lr, double beta1, double beta2, double eps,
                                               double weight_decay, const float* d_clip_scale,
                                               int32_t n_threads, hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_offload_adamw_step";
    zero::clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "zero_offload_adamw_step: n < 0");
    HostScalars c;
    zero_status st = make_scalars(step, lr, beta1, beta2, eps, weight_decay, &c, who);
    if (st != ZERO_OK) return st;
    if (n == 0) return ZERO_OK;
    if (!h_master || !h_exp_avg || !h_exp_avg_sq || !d_grad || !d_param_out || !h_staging)
        return fail(ZERO_EINVAL, "zero_offload_adamw_step: NULL array");
    const int64_t chunk = staging_elems / 4;
    if (chunk < 1) return fail(ZERO_ENOSPACE, "zero_offload_adamw_step: staging holds < 4 elements");
    {
        const size_t fb = static_cast<size_t>(n) * 4, hb = static_cast<size_t>(n) * 2;
        const zero::Span wr[] = {{h_master, fb, "h_master"}, {h_exp_avg, fb, "h_exp_avg"},
                                 {h_exp_avg_sq, fb, "h_exp_avg_sq"},
                                 {h_staging, static_cast<size_t>(chunk) * 4 * 2, "h_staging"},
                                 {d_param_out, hb, "d_param_out"}};
        const zero::Span rd[] = {{d_grad, hb, "d_grad"}};
        const std::string clash = zero::first_overlap(wr, 5, rd, 1);
        if (!clash.empty()) return fail(ZERO_EINVAL, std::string(who) + ": " + clash);
    }
    CopyStreams cs;
    st = copy_streams(&cs);
    if (st != ZERO_OK) return st;
    const int threads = default_threads(n_threads);

    hipEvent_t start = nullptr, ev_in[2] = {nullptr, nullptr}, ev_out[2] = {nullptr, nullptr};
    // On every exit the copy streams have drained (staging is the caller's again)
    // and the events are gone.
    auto finish = [&](zero_status s) -> zero_status {
        (void)hipStreamSynchronize(cs.d2h);
        (void)hipStreamSynchronize(cs.h2d);
        if (start) (void)hipEventDestroy(start);
        for (int i = 0; i < 2; ++i) {
            if (ev_in[i]) (void)hipEventDestroy(ev_in[i]);
            if (ev_out[i]) (void)hipEventDestroy(ev_out[i]);
        }
        return s;
    };
#define ZERO_TRY(expr, what)                                                    \
    do {                                                                        \
        const hipError_t e_ = (expr);                                           \
        if (e_ != hipSuccess)                                                   \
            return finish(zero::check_hip(e_, "zero_offload_adamw_step: " what)); \
    } while (0)
    ZERO_TRY(hipEventCreateWithFlags(&start, hipEventDisableTiming), "event");
    for (int i = 0; i < 2; ++i) {
        ZERO_TRY(hipEventCreateWithFlags(&ev_in[i], hipEventDisableTiming), "event");
        ZERO_TRY(hipEventCreateWithFlags(&ev_out[i], hipEventDisableTiming), "event");
    }
    // Whatever `stream` holds before the call (the gradients' producer) comes first.
    ZERO_TRY(hipEventRecord(start, stream), "record");
    ZERO_TRY(hipStreamWaitEvent(cs.d2h, start, 0), "wait");
    ZERO_TRY(hipStreamWaitEvent(cs.h2d, start, 0), "wait");
    if (d_clip_scale != nullptr) {
        float clip = 1.0f;
        ZERO_TRY(hipMemcpyAsync(&clip, d_clip_scale, sizeof(float), hipMemcpyDeviceToHost, cs.d2h),
                 "clip copy");
        ZERO_TRY(hipStreamSynchronize(cs.d2h), "clip sync");
        if (!std::isfinite(clip)) return finish(ZERO_OK);   // a non-finite norm skips the step
        c.clip = clip;
    }
    // Staging: two gradient slots and two parameter slots of `chunk` elements;
    // chunk k uses slot k % 2 of each.
    Pipeline pl;
    pl.n = n;
    pl.chunk = chunk;
    pl.chunks = (n + chunk - 1) / chunk;
    pl.tasks = threads < HostPool::get().concurrency() ? threads : HostPool::get().concurrency();
    if (n < (int64_t(1) << 16)) pl.tasks = 1;
    pl.p = h_master;
    pl.m = h_exp_avg;
    pl.v = h_exp_avg_sq;
    pl.d_grad = d_grad;
    pl.d_param = d_param_out;
    pl.gstage[0] = h_staging;
    pl.gstage[1] = h_staging + chunk;
    pl.pstage[0] = h_staging + 2 * chunk;
    pl.pstage[1] = h_staging + 3 * chunk;
    pl.d2h = cs.d2h;
    pl.h2d = cs.h2d;
    for (int i = 0; i < 2; ++i) {
        pl.ev_in[i] = ev_in[i];
        pl.ev_out[i] = ev_out[i];
    }
    pl.c = c;
    try {
        pl.done.assign(static_cast<size_t>(pl.chunks), 0);
        pl.in_queued.assign(static_cast<size_t>(pl.chunks), 0);
        pl.out_queued.assign(static_cast<size_t>(pl.chunks), 0);
        pl.in_state.assign(static_cast<size_t>(pl.chunks), 0);
        pl.out_state.assign(static_cast<size_t>(pl.chunks), 0);
    } catch (const std::bad_alloc&) {
        return finish(fail(ZERO_ENOMEM, "zero_offload_adamw_step: allocation failed"));
    }
    pl.queue_in(0);
    if (pl.chunks > 1) pl.queue_in(1);
    if (pl.status == ZERO_OK) HostPool::get().run(pl.tasks, [&pl](int w) { pl.worker(w); });
    if (pl.status != ZERO_OK) return finish(pl.status);
    // Later work on `stream` sees the new parameters.
    ZERO_TRY(hipEventRecord(start, cs.h2d), "record");
    ZERO_TRY(hipStreamWaitEvent(stream, start, 0), "wait");
#undef ZERO_TRY
    return finish(ZERO_OK);
}
