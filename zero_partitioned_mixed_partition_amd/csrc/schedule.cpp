// AdamW's per-step scalars and a schedule's table of them (see schedule.hpp).
#include "schedule.hpp"

#include <cmath>
#include <string>

namespace zero {
namespace adam {

zero_status check_hyper(int64_t step, double lr, double beta1, double beta2, double eps,
                        double weight_decay, const char* who) {
    const std::string w(who);
    if (step < 1) return fail(ZERO_EINVAL, w + ": step must be >= 1");
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
        return fail(ZERO_EINVAL, w + ": betas must lie in [0, 1)");
    if (!(eps > 0.0) || !std::isfinite(eps))
        return fail(ZERO_EINVAL, w + ": eps must be finite and > 0");
    if (!(lr >= 0.0) || !std::isfinite(lr) || !std::isfinite(weight_decay))
        return fail(ZERO_EINVAL, w + ": lr and weight_decay must be finite, lr >= 0");
    return ZERO_OK;
}

zero_status step_scalars(int64_t step, double lr, double beta1, double beta2, double weight_decay,
                         double eps, StepScalars* c, const char* who) {
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
    return ZERO_OK;
}

int64_t settled_step(double beta1, double beta2, int64_t cap) {
    const double tiny = std::ldexp(1.0, -56);
    auto settled = [&](int64_t t) {
        const double x = static_cast<double>(t);
        return std::pow(beta1, x) < tiny && std::pow(beta2, x) < tiny;
    };
    if (cap < 1 || !settled(cap)) return -1;
    // beta^t falls with t, so the steps that satisfy it form a suffix: find its start.
    int64_t lo = 1, hi = cap;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (settled(mid)) hi = mid; else lo = mid + 1;
    }
    return lo;
}

zero_status schedule_table(const double* lr, int64_t n_lr, double beta1, double beta2, double eps,
                           double weight_decay, std::vector<StepScalars>* table, const char* who) {
    const std::string w(who);
    if (lr == nullptr || n_lr < 1) return fail(ZERO_EINVAL, w + ": no learning rate");
    if (n_lr > kMaxScheduleSteps)
        return fail(ZERO_ERANGE, w + ": more than " + std::to_string(kMaxScheduleSteps) + " learning rates");
    for (int64_t i = 0; i < n_lr; ++i) {
        const zero_status st = check_hyper(1, lr[i], beta1, beta2, eps, weight_decay, who);
        if (st != ZERO_OK) return st;
    }
    const int64_t settled = settled_step(beta1, beta2, kMaxScheduleSteps);
    if (settled < 0)
        return fail(ZERO_ERANGE, w + ": the bias corrections settle after more than " +
                                     std::to_string(kMaxScheduleSteps) + " steps (betas too close to 1)");
    const int64_t length = n_lr > settled ? n_lr : settled;
    table->assign(static_cast<size_t>(length), StepScalars{});
    for (int64_t t = 1; t <= length; ++t) {
        const double rate = lr[(t < n_lr ? t : n_lr) - 1];
        const zero_status st = step_scalars(t, rate, beta1, beta2, weight_decay, eps,
                                            &(*table)[static_cast<size_t>(t - 1)], who);
        if (st != ZERO_OK) return st;
    }
    return ZERO_OK;
}

}  // namespace adam
}  // namespace zero
