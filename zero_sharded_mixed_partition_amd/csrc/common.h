// Internal helpers shared by the host and device translation units of the
// library (not part of the public ABI).
#pragma once
#include <cstdarg>
#include <cstdint>

#include "step_coef.h"
#include "zero_shard.h"

namespace zero_shard {

// Records a printf-style detail for zero_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Validates hp and fills c (fill_step_coef); returns ZERO_OK or an error
// status (with detail).
int prepare_adam(const zero_adam_params* hp, StepCoef* c);

// Validates the step-independent hyperparameters (no t, no loss scale).
int check_hyper(double lr, double beta1, double beta2, double eps, double weight_decay, double max_grad_norm);

}  // namespace zero_shard
