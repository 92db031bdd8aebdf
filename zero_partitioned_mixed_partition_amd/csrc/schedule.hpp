// AdamW's per-step fp32 scalars, computed on the host, and the table of them
// that a device-resident step schedule holds (host C++, no device code).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Static Memory Allocation" (fp32
// master weights, first and second moments) and "Execution Flow for ZeRO-1"
// step 3 (the rank updates its slice): the update's scalars depend only on the
// step t and the hyperparameters, so they are computed once per step, in fp64,
// each rounded once to fp32.
#pragma once

#include <cstdint>
#include <vector>

#include "internal.hpp"

namespace zero {
namespace adam {

// The scalars of one AdamW step, in the order the kernels use them.
struct StepScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, step_size, sqrt_bc2, decay;
};
static_assert(sizeof(StepScalars) == 32, "eight floats");

// The hyperparameter checks every AdamW entry point makes.
zero_status check_hyper(int64_t step, double lr, double beta1, double beta2, double eps,
                        double weight_decay, const char* who);

// The scalars of step `step` (>= 1): bias corrections 1 - beta^step in fp64,
// step size lr / (1 - beta1^step), sqrt(1 - beta2^step), decay factor
// 1 - lr * weight_decay, each rounded once to fp32. ZERO_EINVAL when a bias
// correction is zero.
zero_status step_scalars(int64_t step, double lr, double beta1, double beta2, double weight_decay,
                         double eps, StepScalars* out, const char* who);

// The first step t from which both bias corrections are exactly 1 in fp64:
// beta1^t and beta2^t both below 2^-56 (so below 2^-54 at every later step,
// whatever the last bit of pow, and 1 - beta^t rounds to 1). Every step from t
// on then has step t's scalars for the same lr. -1 when that step lies past
// `cap`.
int64_t settled_step(double beta1, double beta2, int64_t cap);

// Longest table a schedule holds (2^24 steps, 512 MB).
constexpr int64_t kMaxScheduleSteps = int64_t(1) << 24;

// A schedule's table: the scalars of steps 1..L, L = max(n_lr, settled step),
// step t with learning rate lr[min(t, n_lr) - 1]. Every step past L has step
// L's scalars. ZERO_EINVAL for bad hyperparameters, ZERO_ERANGE past
// kMaxScheduleSteps; throws std::bad_alloc.
zero_status schedule_table(const double* lr, int64_t n_lr, double beta1, double beta2, double eps,
                           double weight_decay, std::vector<StepScalars>* table, const char* who);

}  // namespace adam
}  // namespace zero
