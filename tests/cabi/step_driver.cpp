// A C ABI client with no Python and no torch: device memory from hipMalloc,
// an explicit HIP stream, and the calls of include/zero_shard.h.  It checks
// one shard step against closed forms that need no oracle:
//   * the norm of a gradient made of +0.5 and -0.25 is n_odd/4 + n_even/16,
//     exactly, since every square and partial sum is a short binary fraction;
//   * the first Adam step from m = v = 0 (bias corrections 1 - beta) moves
//     each weight by -lr * g / (|g| + eps), sets m = (1 - beta1) g and
//     v = (1 - beta2) g^2;
//   * the 16-bit parameter copy is the round-to-nearest-even of the stored
//     fp32 master, bit for bit;
//   * an inf anywhere sets the flag and the step writes nothing;
//   * the step with the loss scaler in device memory gives the same bits;
//   * the norm pass without a workspace (its partials in the library's fixed
//     array) gives the same bits, and flags the inf;
//   * a misaligned pointer is rejected with ZERO_EALIGN and a detail string.
// Prints "ok" and exits 0 on success; anything else is a failure.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "zero_shard.h"

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                              \
        }                                                                          \
    } while (0)
#define CHECK(c, ...)                                                              \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, __VA_ARGS__);                                     \
            std::fputc('\n', stderr);                                              \
            return 1;                                                              \
        }                                                                          \
    } while (0)

namespace {

uint32_t bits32(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return u;
}

// bfloat16 round to nearest even from fp32 (finite inputs)
uint16_t bf16_rne(float x) {
    const uint32_t u = bits32(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

bool within(double got, double ref) { return std::fabs(got - ref) <= std::fmax(1e-5 * std::fabs(ref), 1e-7); }

struct Shard {
    float *P = nullptr, *M = nullptr, *V = nullptr;
    uint16_t *G = nullptr, *PO = nullptr;
};

int alloc_shard(Shard& s, int64_t n) {
    HIP_OK(hipMalloc((void**)&s.P, n * 4));
    HIP_OK(hipMalloc((void**)&s.M, n * 4));
    HIP_OK(hipMalloc((void**)&s.V, n * 4));
    HIP_OK(hipMalloc((void**)&s.G, n * 2));
    HIP_OK(hipMalloc((void**)&s.PO, n * 2));
    return 0;
}

void free_shard(Shard& s) {
    (void)hipFree(s.P);
    (void)hipFree(s.M);
    (void)hipFree(s.V);
    (void)hipFree(s.G);
    (void)hipFree(s.PO);
}

// the same five streams from the library's physically contiguous memory
int alloc_shard_contiguous(Shard& s, int64_t n) {
    int st = zero_device_alloc_contiguous((void**)&s.P, n * 4);
    if (st == ZERO_OK) st = zero_device_alloc_contiguous((void**)&s.M, n * 4);
    if (st == ZERO_OK) st = zero_device_alloc_contiguous((void**)&s.V, n * 4);
    if (st == ZERO_OK) st = zero_device_alloc_contiguous((void**)&s.G, n * 2);
    if (st == ZERO_OK) st = zero_device_alloc_contiguous((void**)&s.PO, n * 2);
    CHECK(st == ZERO_OK, "contiguous allocation: %s", zero_last_error());
    return 0;
}

void free_shard_contiguous(Shard& s) {
    (void)zero_device_free(s.P);
    (void)zero_device_free(s.M);
    (void)zero_device_free(s.V);
    (void)zero_device_free(s.G);
    (void)zero_device_free(s.PO);
}

}  // namespace

int main() {
    const int64_t n = 1000003;                       // not a multiple of 4, 8 or 256
    const float g_odd = 0.5f, g_even = -0.25f;       // exact in bfloat16
    std::vector<float> p0(n), zeros(n, 0.0f);
    std::vector<uint16_t> g(n);
    int64_t n_odd = 0;
    for (int64_t i = 0; i < n; ++i) {
        p0[i] = 1.0f + 0.125f * (float)(i % 7);
        g[i] = (uint16_t)(bits32(i & 1 ? g_odd : g_even) >> 16);
        n_odd += i & 1;
    }
    CHECK(zero_abi_version() == ZERO_SHARD_ABI_VERSION, "ABI version %d", zero_abi_version());

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    Shard a;
    if (alloc_shard(a, n)) return 1;
    double* d_sq;
    int32_t* d_ovf;
    void* d_ws;
    const size_t ws_bytes = zero_norm_workspace_bytes(n);
    HIP_OK(hipMalloc((void**)&d_sq, sizeof(double)));
    HIP_OK(hipMalloc((void**)&d_ovf, sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    HIP_OK(hipMemcpy(a.P, p0.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(a.M, zeros.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(a.V, zeros.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(a.G, g.data(), n * 2, hipMemcpyHostToDevice));

    // steps 1-2, then 3-4: t = 1, AdamW without decay or clipping, scale 1
    int st = zero_shard_unscale_norm_overflow(a.G, ZERO_BF16, n, 1.0, d_sq, d_ovf, d_ws, ws_bytes, stream);
    CHECK(st == ZERO_OK, "norm pass: %s (%s)", zero_status_string(st), zero_last_error());
    const zero_adam_params hp = {1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 0.0};
    st = zero_shard_adam_step(a.P, a.M, a.V, a.G, ZERO_BF16, a.PO, ZERO_BF16, n, &hp, d_sq, d_ovf, stream);
    CHECK(st == ZERO_OK, "update: %s (%s)", zero_status_string(st), zero_last_error());
    HIP_OK(hipStreamSynchronize(stream));

    double sq;
    int32_t ovf;
    HIP_OK(hipMemcpy(&sq, d_sq, sizeof(sq), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&ovf, d_ovf, sizeof(ovf), hipMemcpyDeviceToHost));
    const double sq_ref = 0.25 * (double)n_odd + 0.0625 * (double)(n - n_odd);
    CHECK(ovf == 0, "flag %d on a finite gradient", ovf);
    CHECK(sq == sq_ref, "sum of squares %.17g, closed form %.17g", sq, sq_ref);

    std::vector<float> p1(n), m1(n), v1(n);
    std::vector<uint16_t> par1(n);
    HIP_OK(hipMemcpy(p1.data(), a.P, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(m1.data(), a.M, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(v1.data(), a.V, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(par1.data(), a.PO, n * 2, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < n; ++i) {
        const double gi = i & 1 ? g_odd : g_even;
        const double p_ref = (double)p0[i] - hp.lr * gi / (std::fabs(gi) + hp.eps);
        CHECK(within(m1[i], (1.0 - hp.beta1) * gi), "m[%lld] = %.9g", (long long)i, m1[i]);
        CHECK(within(v1[i], (1.0 - hp.beta2) * gi * gi), "v[%lld] = %.9g", (long long)i, v1[i]);
        CHECK(within(p1[i], p_ref), "p[%lld] = %.9g, closed form %.9g", (long long)i, p1[i], p_ref);
        CHECK(par1[i] == bf16_rne(p1[i]), "param[%lld] = 0x%04x, RNE of master 0x%04x", (long long)i, par1[i],
              bf16_rne(p1[i]));
    }

    // an inf in the last element: flag set, nothing written
    const uint16_t inf_bf16 = 0x7F80;
    HIP_OK(hipMemcpy(a.G + (n - 1), &inf_bf16, 2, hipMemcpyHostToDevice));
    st = zero_shard_unscale_norm_overflow(a.G, ZERO_BF16, n, 1.0, d_sq, d_ovf, d_ws, ws_bytes, stream);
    CHECK(st == ZERO_OK, "norm pass: %s", zero_last_error());
    zero_adam_params hp2 = hp;
    hp2.step = 2;
    st = zero_shard_adam_step(a.P, a.M, a.V, a.G, ZERO_BF16, a.PO, ZERO_BF16, n, &hp2, d_sq, d_ovf, stream);
    CHECK(st == ZERO_OK, "update: %s", zero_last_error());
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(&ovf, d_ovf, sizeof(ovf), hipMemcpyDeviceToHost));
    CHECK(ovf == 1, "flag %d with an inf in the gradient", ovf);
    {
        std::vector<float> p2(n);
        std::vector<uint16_t> par2(n);
        HIP_OK(hipMemcpy(p2.data(), a.P, n * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(par2.data(), a.PO, n * 2, hipMemcpyDeviceToHost));
        CHECK(std::memcmp(p2.data(), p1.data(), n * 4) == 0, "a skipped step changed the master");
        CHECK(std::memcmp(par2.data(), par1.data(), n * 2) == 0, "a skipped step wrote the parameter copy");
    }

    // the same first step with the loss scaler and step counter in device memory
    Shard b;
    if (alloc_shard_contiguous(b, n)) return 1;        // this one from physically contiguous memory
    HIP_OK(hipMemcpy(b.P, p0.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(b.M, zeros.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(b.V, zeros.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(b.G, g.data(), n * 2, hipMemcpyHostToDevice));
    zero_step_state h_state;
    std::memset(&h_state, 0, sizeof(h_state));
    h_state.scaler = zero_loss_scaler{1.0, 1.0, 1.0, 1.0, 1000, 0};     // a static scale of 1
    zero_step_state* d_state;
    void* d_coef;
    HIP_OK(hipMalloc((void**)&d_state, sizeof(zero_step_state)));
    HIP_OK(hipMalloc(&d_coef, zero_adam_coef_bytes()));
    HIP_OK(hipMemcpy(d_state, &h_state, sizeof(h_state), hipMemcpyHostToDevice));
    const zero_adam_hyper hy = {hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_grad_norm};
    st = zero_shard_norm_decide_dev(b.G, ZERO_BF16, n, &hy, d_state, d_sq, d_ovf, d_coef, d_ws, ws_bytes, stream);
    CHECK(st == ZERO_OK, "norm and decision: %s", zero_last_error());
    st = zero_shard_adam_step_coef(b.P, b.M, b.V, b.G, ZERO_BF16, b.PO, ZERO_BF16, n, d_coef, d_sq, d_ovf, stream);
    CHECK(st == ZERO_OK, "update with device coefficients: %s", zero_last_error());
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(&h_state, d_state, sizeof(h_state), hipMemcpyDeviceToHost));
    CHECK(h_state.applied == 1 && h_state.skipped == 0 && h_state.last_overflow == 0, "state after one step");
    {
        std::vector<float> p3(n), m3(n), v3(n);
        std::vector<uint16_t> par3(n);
        HIP_OK(hipMemcpy(p3.data(), b.P, n * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(m3.data(), b.M, n * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(v3.data(), b.V, n * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(par3.data(), b.PO, n * 2, hipMemcpyDeviceToHost));
        CHECK(std::memcmp(p3.data(), p1.data(), n * 4) == 0 && std::memcmp(m3.data(), m1.data(), n * 4) == 0 &&
                  std::memcmp(v3.data(), v1.data(), n * 4) == 0 && std::memcmp(par3.data(), par1.data(), n * 2) == 0,
              "the device-state step differs from the host-scaled one");
    }

    // the norm pass that allocates nothing and takes no workspace: the closed
    // form on the finite gradient, the flag and +inf on the one holding an inf
    for (int rep = 0; rep < 2; ++rep) {
        st = zero_shard_unscale_norm_overflow_noalloc(b.G, ZERO_BF16, n, 1.0, d_sq, d_ovf, stream);
        CHECK(st == ZERO_OK, "norm pass without a workspace: %s", zero_last_error());
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(&sq, d_sq, sizeof(sq), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(&ovf, d_ovf, sizeof(ovf), hipMemcpyDeviceToHost));
        CHECK(ovf == 0 && sq == sq_ref, "no-workspace norm %.17g (flag %d), closed form %.17g", sq, ovf, sq_ref);
        st = zero_shard_unscale_norm_overflow_noalloc(a.G, ZERO_BF16, n, 1.0, d_sq, d_ovf, stream);
        CHECK(st == ZERO_OK, "norm pass without a workspace: %s", zero_last_error());
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(&sq, d_sq, sizeof(sq), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(&ovf, d_ovf, sizeof(ovf), hipMemcpyDeviceToHost));
        CHECK(ovf == 1 && std::isinf(sq) && sq > 0, "no-workspace norm with an inf: %.17g (flag %d)", sq, ovf);
    }

    // errors are reported, not launched: a master pointer off by 4 bytes
    st = zero_shard_adam_step(a.P + 1, a.M, a.V, a.G, ZERO_BF16, nullptr, 0, 16, &hp, d_sq, d_ovf, stream);
    CHECK(st == ZERO_EALIGN, "misaligned master: status %d", st);
    CHECK(zero_last_error()[0] != '\0' && zero_status_string(st) != nullptr, "no error detail");

    free_shard(a);
    free_shard_contiguous(b);
    (void)hipFree(d_sq);
    (void)hipFree(d_ovf);
    (void)hipFree(d_ws);
    (void)hipFree(d_state);
    (void)hipFree(d_coef);
    HIP_OK(hipStreamDestroy(stream));
    std::printf("ok\n");
    return 0;
}
