// Per-step AdamW coefficients, shared by the host translation units and the
// device code, so that a block formed on the host and one formed by a kernel
// from device-resident step state are bit-identical.
//
// Adam's bias corrections (Kingma & Ba) for the 1-based index t of the step
// being applied, and decoupled weight decay (Loshchilov & Hutter), each
// formed in IEEE double and rounded once to float.  beta^t is taken by
// binary exponentiation (exact IEEE multiplications, the same on both sides)
// rather than by a library pow, whose last bit may differ between the host
// and device math libraries.
#pragma once
#include <cmath>
#include <cstdint>

#if defined(__HIPCC__)
#define ZS_HD __host__ __device__
#else
#define ZS_HD
#endif

namespace zero_shard {

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

// b^e for e >= 0 by binary exponentiation.
ZS_HD inline double pow_int(double b, int64_t e) {
#pragma clang fp contract(off)
    double r = 1.0;
    while (e > 0) {
        if (e & 1) r = r * b;
        b = b * b;
        e >>= 1;
    }
    return r;
}

// Bias corrections 1 - beta^t (positive for beta in [0, 1) and t >= 1 unless
// beta^t rounds to 1).
ZS_HD inline double bias_correction(double beta, int64_t t) { return 1.0 - pow_int(beta, t); }

// Fills c for step t >= 1; the caller has validated the hyperparameters and
// checked that both bias corrections are positive.
ZS_HD inline void fill_step_coef(double lr, double beta1, double beta2, double eps, double weight_decay, int64_t t,
                                 double inv_scale, double max_grad_norm, StepCoef* c) {
#pragma clang fp contract(off)
    const double bc1 = bias_correction(beta1, t);
    const double bc2 = bias_correction(beta2, t);
    const bool clip = max_grad_norm > 0.0;
    c->beta1 = (float)beta1;
    c->omb1 = (float)(1.0 - beta1);
    c->beta2 = (float)beta2;
    c->omb2 = (float)(1.0 - beta2);
    c->step_size = (float)(lr / bc1);
    c->rsqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    c->eps = (float)eps;
    c->decay = (float)(1.0 - lr * weight_decay);
    c->gscale_fixed = (float)inv_scale;
    c->clip = clip ? 1 : 0;
    c->inv_scale = inv_scale;
    c->max_norm = clip ? max_grad_norm : 0.0;
}

}  // namespace zero_shard
