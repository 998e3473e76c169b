// Host-only part of the C ABI: partition plan, rank fragments, loss scaler,
// status strings and the thread-local error detail.
//
// Partition layout (ZeRO method entry, description; explainer "Data
// Parallelism Without the Copies", History entry "ZeRO" and "The 16 Bytes per
// Parameter Audit"): tensors end to end in list order, the flat buffer padded
// at its end to N_d equal partitions whose size is a multiple of `align`.
#include "zero_shard.h"
#include "common.h"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

namespace zero_shard {

static thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

void clear_error() { g_last_error.clear(); }

int check_hyper(double lr, double beta1, double beta2, double eps, double weight_decay, double max_grad_norm) {
    if (!(lr >= 0.0) || !std::isfinite(lr)) return fail(ZERO_EINVAL, "lr must be finite and >= 0");
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
        return fail(ZERO_EINVAL, "betas must lie in [0, 1)");
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(ZERO_EINVAL, "eps must be finite and >= 0");
    if (!(weight_decay >= 0.0) || !std::isfinite(weight_decay))
        return fail(ZERO_EINVAL, "weight_decay must be finite and >= 0");
    if (max_grad_norm > 0.0 && !std::isfinite(max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm must be finite");
    if (std::isnan(max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm is NaN");
    return ZERO_OK;
}

int prepare_adam(const zero_adam_params* hp, StepCoef* c) {
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    const zero_adam_params& h = *hp;
    const int st = check_hyper(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.max_grad_norm);
    if (st != ZERO_OK) return st;
    if (h.step < 1) return fail(ZERO_EINVAL, "step (1-based index of the step applied) must be >= 1");
    if (!(h.inv_loss_scale > 0.0) || !std::isfinite(h.inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    // bias corrections of the step being applied (Adam, 1-based t)
    if (!(bias_correction(h.beta1, h.step) > 0.0) || !(bias_correction(h.beta2, h.step) > 0.0))
        return fail(ZERO_ERANGE, "bias correction underflows to 0");
    fill_step_coef(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step, h.inv_loss_scale, h.max_grad_norm, c);
    return ZERO_OK;
}

namespace {

bool add_ovf(int64_t a, int64_t b, int64_t* out) { return __builtin_add_overflow(a, b, out); }
bool mul_ovf(int64_t a, int64_t b, int64_t* out) { return __builtin_mul_overflow(a, b, out); }

struct Plan {
    int64_t total = 0, S = 0, padded = 0;
};

// Walks the shape list once; fills offsets (may be null) and the plan.
int make_plan(const int64_t* dims, const int32_t* ndims, int32_t n_tensors, int32_t n_d,
              int64_t align, int64_t* offsets, Plan* plan) {
    if (n_tensors < 0) return fail(ZERO_EINVAL, "n_tensors < 0");
    if (n_tensors > 0 && ndims == nullptr) return fail(ZERO_EINVAL, "ndims is NULL");
    if (n_d < 1) return fail(ZERO_EINVAL, "n_d must be >= 1 (got %d)", n_d);
    if (align < 1) return fail(ZERO_EINVAL, "align must be >= 1 (got %lld)", (long long)align);
    int64_t off = 0, d = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (ndims[i] < 0) return fail(ZERO_EINVAL, "ndims[%d] < 0", i);
        if (ndims[i] > 0 && dims == nullptr) return fail(ZERO_EINVAL, "dims is NULL");
        int64_t numel = 1;
        for (int32_t k = 0; k < ndims[i]; ++k, ++d) {
            if (dims[d] < 0) return fail(ZERO_EINVAL, "tensor %d has a negative dimension", i);
            if (mul_ovf(numel, dims[d], &numel))
                return fail(ZERO_ERANGE, "tensor %d element count overflows int64", i);
        }
        if (offsets) offsets[i] = off;
        if (add_ovf(off, numel, &off)) return fail(ZERO_ERANGE, "total element count overflows int64");
    }
    int64_t unit;
    if (mul_ovf((int64_t)n_d, align, &unit)) return fail(ZERO_ERANGE, "n_d * align overflows int64");
    // S = align * ceil(T / (n_d * align)), padded = n_d * S (written to avoid T + unit - 1 overflow)
    int64_t units = off / unit + (off % unit != 0 ? 1 : 0);
    if (mul_ovf(units, align, &plan->S)) return fail(ZERO_ERANGE, "partition size overflows int64");
    if (mul_ovf(plan->S, (int64_t)n_d, &plan->padded))
        return fail(ZERO_ERANGE, "padded total overflows int64");
    plan->total = off;
    return ZERO_OK;
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" {

int zero_abi_version(void) { return ZERO_SHARD_ABI_VERSION; }

int zero_partition_plan(const int64_t* dims, const int32_t* ndims, int32_t n_tensors, int32_t n_d,
                        int64_t align, int64_t* tensor_offsets, int64_t* partition_numel,
                        int64_t* padded_total) {
    clear_error();
    if (partition_numel == nullptr || padded_total == nullptr)
        return fail(ZERO_EINVAL, "partition_numel / padded_total is NULL");
    if (n_tensors > 0 && tensor_offsets == nullptr) return fail(ZERO_EINVAL, "tensor_offsets is NULL");
    Plan p;
    int st = make_plan(dims, ndims, n_tensors, n_d, align, tensor_offsets, &p);
    if (st != ZERO_OK) return st;
    *partition_numel = p.S;
    *padded_total = p.padded;
    return ZERO_OK;
}

int zero_rank_fragments(const int64_t* dims, const int32_t* ndims, int32_t n_tensors, int32_t n_d,
                        int64_t align, int32_t rank, zero_fragment* out, int32_t capacity,
                        int32_t* count) {
    clear_error();
    if (count == nullptr) return fail(ZERO_EINVAL, "count is NULL");
    if (capacity < 0 || (capacity > 0 && out == nullptr)) return fail(ZERO_EINVAL, "bad out/capacity");
    Plan p;
    int st = make_plan(dims, ndims, n_tensors, n_d, align, nullptr, &p);
    if (st != ZERO_OK) return st;
    if (rank < 0 || rank >= n_d) return fail(ZERO_EINVAL, "rank %d outside [0, %d)", rank, n_d);
    const int64_t lo = (int64_t)rank * p.S, hi = lo + p.S;
    int64_t off = 0, d = 0;
    int32_t k = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        int64_t numel = 1;
        for (int32_t j = 0; j < ndims[i]; ++j, ++d) numel *= dims[d];   // checked by make_plan
        const int64_t a = off > lo ? off : lo;
        const int64_t b = off + numel < hi ? off + numel : hi;
        if (a < b) {
            if (k < capacity) {
                out[k].tensor = i;
                out[k].reserved = 0;
                out[k].tensor_begin = a - off;
                out[k].shard_begin = a - lo;
                out[k].numel = b - a;
            }
            ++k;
        }
        off += numel;
    }
    *count = k;
    if (k > capacity) return fail(ZERO_ENOSPC, "need %d fragments, capacity %d", k, capacity);
    return ZERO_OK;
}

int zero_loss_scaler_update(zero_loss_scaler* s, int32_t overflow, int32_t* skip_out) {
    clear_error();
    if (s == nullptr || skip_out == nullptr) return fail(ZERO_EINVAL, "NULL argument");
    if (!(s->scale > 0) || !(s->min_scale > 0) || !(s->backoff > 0) || !(s->growth > 0) ||
        s->growth_interval < 1 || s->good_steps < 0)
        return fail(ZERO_EINVAL, "invalid loss scaler state");
    if (overflow) {
        const double next = s->scale * s->backoff;
        s->scale = next > s->min_scale ? next : s->min_scale;
        s->good_steps = 0;
        *skip_out = 1;
        return ZERO_OK;
    }
    *skip_out = 0;
    s->good_steps += 1;
    if (s->good_steps >= s->growth_interval) {
        s->scale *= s->growth;
        s->good_steps = 0;
    }
    return ZERO_OK;
}

const char* zero_status_string(int status) {
    switch (status) {
        case ZERO_OK: return "ok";
        case ZERO_EINVAL: return "invalid argument";
        case ZERO_EALIGN: return "device pointer not 16-byte aligned";
        case ZERO_ERANGE: return "size out of range";
        case ZERO_ENOSPC: return "output or workspace too small";
        case ZERO_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* zero_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
