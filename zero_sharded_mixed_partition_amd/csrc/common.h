// Internal helpers shared by the host and device translation units of the
// library (not part of the public ABI).
#pragma once
#include <cstdarg>
#include <cstdint>

#include "zero_shard.h"

namespace zero_shard {

// Records a printf-style detail for zero_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Per-step AdamW coefficients, derived on the host in double from the
// hyperparameters and rounded once each to float (shared by the device and
// the host implementations of the step).
struct StepCoef {
    float beta1, omb1, beta2, omb2;   // beta, 1 - beta
    float step_size;                  // lr / (1 - beta1^t)
    float rsqrt_bc2;                  // 1 / sqrt(1 - beta2^t)
    float eps;
    float decay;                      // 1 - lr * wd
    float gscale_fixed;               // float(inv_scale), the gradient factor when clipping is off
    int clip;                         // max_grad_norm > 0
    double inv_scale, max_norm;
};

// Validates hp and fills c; returns ZERO_OK or an error status (with detail).
int prepare_adam(const zero_adam_params* hp, StepCoef* c);

}  // namespace zero_shard
