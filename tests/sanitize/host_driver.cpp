// Exercises the host half of libzero_shard (partition plan, rank fragments,
// loss scaler, host step and its thread pool, error paths) so that it can be
// run under AddressSanitizer + UndefinedBehaviorSanitizer and under
// ThreadSanitizer.  Built and run by tests/test_host_sanitizers.py; prints
// "ok" and exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zero_shard.h"

namespace {

int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {      // splitmix64
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
int64_t uniform(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

uint16_t f32_to_f16_bits(float x) {     // for inputs only: |x| well inside the normal fp16 range
    uint32_t u;
    std::memcpy(&u, &x, 4);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const int32_t e = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
    if (e <= 0) return (uint16_t)sign;
    return (uint16_t)(sign | ((uint32_t)e << 10) | ((u >> 13) & 0x3FFu));
}

void plans() {
    for (int trial = 0; trial < 300; ++trial) {
        const int32_t nt = (int32_t)uniform(0, 12);
        std::vector<int32_t> ndims(nt);
        std::vector<int64_t> dims;
        for (int32_t i = 0; i < nt; ++i) {
            ndims[i] = (int32_t)uniform(0, 3);
            for (int k = 0; k < ndims[i]; ++k) dims.push_back(uniform(0, 40));
        }
        const int32_t nd = (int32_t)uniform(1, 9);
        const int64_t align = uniform(1, 16);
        std::vector<int64_t> offs(nt + 1);
        int64_t S = -1, padded = -1;
        const int st = zero_partition_plan(dims.data(), ndims.data(), nt, nd, align, offs.data(), &S, &padded);
        CHECK(st == ZERO_OK);
        CHECK(S % align == 0 && padded == S * nd);
        int64_t covered = 0;
        for (int32_t r = 0; r < nd; ++r) {
            int32_t count = -1;
            const int st0 = zero_rank_fragments(dims.data(), ndims.data(), nt, nd, align, r, nullptr, 0, &count);
            CHECK(count >= 0 && st0 == (count > 0 ? ZERO_ENOSPC : ZERO_OK));
            std::vector<zero_fragment> fr(count > 0 ? count : 1);
            int32_t c2 = -1;
            CHECK(zero_rank_fragments(dims.data(), ndims.data(), nt, nd, align, r, fr.data(), count, &c2) == ZERO_OK);
            CHECK(c2 == count);
            for (int32_t k = 0; k < c2; ++k) {
                CHECK(fr[k].numel > 0 && fr[k].shard_begin >= 0 && fr[k].shard_begin + fr[k].numel <= S);
                covered += fr[k].numel;
            }
        }
        int64_t total = 0;
        for (int32_t i = 0, d = 0; i < nt; ++i) {
            int64_t numel = 1;
            for (int k = 0; k < ndims[i]; ++k) numel *= dims[d++];
            total += numel;
        }
        CHECK(covered == total);
    }
    // errors
    int64_t S, P, off[2];
    const int64_t big[2] = {INT64_MAX / 2, 4};
    const int32_t nd2[1] = {2};
    CHECK(zero_partition_plan(big, nd2, 1, 1, 1, off, &S, &P) == ZERO_ERANGE);
    CHECK(zero_partition_plan(big, nd2, 1, 0, 1, off, &S, &P) == ZERO_EINVAL);
    CHECK(zero_partition_plan(nullptr, nd2, 1, 1, 1, off, &S, &P) == ZERO_EINVAL);
    CHECK(std::strlen(zero_last_error()) > 0);
    for (int s = -6; s <= 0; ++s) CHECK(zero_status_string(s) != nullptr);
}

void scaler() {
    zero_loss_scaler s{65536.0, 1.0, 0.5, 2.0, 3, 0};
    for (int i = 0; i < 200; ++i) {
        int32_t skip = -1;
        CHECK(zero_loss_scaler_update(&s, (int32_t)(next_u64() % 5 == 0), &skip) == ZERO_OK);
        CHECK(skip == 0 || skip == 1);
        CHECK(s.scale >= 1.0 && s.good_steps >= 0 && s.good_steps < 3);
    }
    zero_loss_scaler bad{0.0, 1.0, 0.5, 2.0, 3, 0};
    int32_t skip;
    CHECK(zero_loss_scaler_update(&bad, 0, &skip) == ZERO_EINVAL);
    CHECK(zero_loss_scaler_update(nullptr, 0, &skip) == ZERO_EINVAL);
}

void host_step() {
    const int64_t sizes[] = {0, 1, 3, 4, 5, 63, 64, 65, 1000, 65537, 200003};
    for (int64_t n : sizes) {
        std::vector<uint16_t> g16(n);
        std::vector<float> g32(n);
        for (int64_t i = 0; i < n; ++i) {
            const float x = (float)((double)(int64_t)(next_u64() % 2001) - 1000.0) * 1e-3f;
            g32[i] = x;
            g16[i] = f32_to_f16_bits(x);
        }
        for (int32_t dt : {ZERO_F16, ZERO_F32}) {
            const void* g = dt == ZERO_F32 ? (const void*)g32.data() : (const void*)g16.data();
            double sq1 = -1, sq8 = -2;
            int32_t o1 = -1, o8 = -1;
            CHECK(zero_cpu_shard_unscale_norm_overflow(g, dt, n, 0.5, &sq1, &o1, 1) == ZERO_OK);
            CHECK(zero_cpu_shard_unscale_norm_overflow(g, dt, n, 0.5, &sq8, &o8, 8) == ZERO_OK);
            CHECK(sq1 == sq8 && o1 == 0 && o8 == 0);
            std::vector<float> p1(n), m1(n), v1(n), p3, m3, v3;
            for (int64_t i = 0; i < n; ++i) {
                p1[i] = 0.02f * (float)((int64_t)(next_u64() % 201) - 100) / 100.0f;
                m1[i] = 1e-4f;
                v1[i] = 1e-6f;
            }
            p3 = p1, m3 = m1, v3 = v1;
            std::vector<uint16_t> out1(n), out3(n);
            const zero_adam_params hp{1e-3, 0.9, 0.999, 1e-8, 0.01, 7, 0.5, 1.0};
            CHECK(zero_cpu_shard_adam_step(p1.data(), m1.data(), v1.data(), g, dt, out1.data(), ZERO_BF16, n, &hp,
                                           sq1, 0, 1) == ZERO_OK);
            CHECK(zero_cpu_shard_adam_step(p3.data(), m3.data(), v3.data(), g, dt, out3.data(), ZERO_BF16, n, &hp,
                                           sq1, 0, 3) == ZERO_OK);
            CHECK(p1 == p3 && m1 == m3 && v1 == v3 && out1 == out3);
            // overflow leaves everything untouched
            std::vector<float> keep = p1;
            CHECK(zero_cpu_shard_adam_step(p1.data(), m1.data(), v1.data(), g, dt, nullptr, 0, n, &hp, sq1, 1, 4) ==
                  ZERO_OK);
            CHECK(p1 == keep);
        }
        if (n > 2) {
            g16[n / 2] = 0x7C00;   // +inf
            double sq;
            int32_t o;
            CHECK(zero_cpu_shard_unscale_norm_overflow(g16.data(), ZERO_F16, n, 1.0, &sq, &o, 5) == ZERO_OK);
            CHECK(o == 1 && std::isinf(sq));
        }
    }
    double sq;
    int32_t o;
    CHECK(zero_cpu_shard_unscale_norm_overflow(nullptr, ZERO_F16, 4, 1.0, &sq, &o, 1) == ZERO_EINVAL);
    CHECK(zero_cpu_shard_unscale_norm_overflow(&sq, 9, 4, 1.0, &sq, &o, 1) == ZERO_EINVAL);
    float a[4] = {0}, b[4] = {0}, c[4] = {0};
    uint16_t g[4] = {0};
    const zero_adam_params bad{1e-3, 1.5, 0.999, 1e-8, 0.0, 1, 1.0, 0.0};
    CHECK(zero_cpu_shard_adam_step(a, b, c, g, ZERO_F16, nullptr, 0, 4, &bad, 0.0, 0, 1) == ZERO_EINVAL);
    CHECK(zero_cpu_shard_adam_step(a, a, c, g, ZERO_F16, nullptr, 0, 4, &bad, 0.0, 0, 1) == ZERO_EINVAL);
}

}  // namespace

int main() {
    plans();
    scaler();
    host_step();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
