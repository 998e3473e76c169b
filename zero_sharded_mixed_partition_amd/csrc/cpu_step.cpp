// Host (CPU) implementation of one rank's shard step, for optimizer states
// kept in host memory: the CPU-offload lineage (explainer "Data Parallelism
// Without the Copies", Legacy, card "The trillion-parameter claim": later
// work carried the stages on to offloading into CPU memory and NVMe; the
// glossary entry's description lists CPU offloading beside ZeRO).  The step is
// the same one the device kernels compute (unscale, inf/NaN test, squared
// norm; clip; bias-corrected AdamW; 16-bit writeback), with the per-step
// coefficients from the same host routine, on host cores over host memory.
//
// Work is cut into fixed chunks of kChunk elements handed to a persistent
// pool of threads.  The squared norm is summed in float64 per chunk in a fixed order
// and the chunk sums are combined in chunk order, so the result does not
// depend on the number of threads.  The inner loops are written so the
// compiler vectorizes them; target_clones builds AVX-512, AVX2 and generic
// versions and picks one at load time.  Floating-point contraction is off, so
// every version rounds identically.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include <immintrin.h>
#include <unistd.h>

#include "common.h"
#include "zero_shard.h"

#pragma clang fp contract(off)

namespace zero_shard {
namespace {

constexpr int64_t kChunk = int64_t(1) << 16;   // elements per work item / norm partial
constexpr int kTile = 2048;                    // elements converted per inner pass (stack buffers)

// Per-ISA clones of the hot loops (AVX-512, AVX2 with FMA, baseline), picked
// at load time by resolvers the dynamic loader runs.  The AdamW loop uses
// fused multiply-adds: the two vector clones issue them in hardware; the
// baseline clone (x86-64 without FMA) calls the C library's fmaf, which
// rounds the same way, slowly.  A ThreadSanitizer build compiles
// them once: its runtime is not up yet when the loader runs the resolvers.
#if defined(__has_feature)
#if __has_feature(thread_sanitizer)
#define ZS_SINGLE_ISA 1
#endif
#endif
#if defined(__SANITIZE_THREAD__)
#define ZS_SINGLE_ISA 1
#endif
#ifdef ZS_SINGLE_ISA
#define ZS_CLONES
#else
#define ZS_CLONES __attribute__((target_clones("avx512f", "arch=haswell", "default")))
#endif

inline uint32_t f2u(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}
inline float u2f(uint32_t u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// ---------------------------------------------------------------- 16-bit formats (IEEE 754 definitions)

// binary16 -> binary32, exact.  Subnormals (exponent field 0) are m * 2^-24;
// inf/NaN keep their fraction; normals rebias the exponent (15 -> 127).
inline float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t em = h & 0x7FFFu;
    float r;
    if (em < 0x0400u) r = (float)em * 0x1p-24f;
    else if (em >= 0x7C00u) r = u2f((em << 13) | 0x7F800000u);
    else r = u2f((em << 13) + 0x38000000u);
    return u2f(f2u(r) | sign);
}

inline float bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

// binary32 -> binary16, round to nearest, ties to even; overflow to inf; NaN to a quiet NaN.
inline uint16_t f32_to_f16(float f) {
    const uint32_t x = f2u(f);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const uint32_t a = x & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u);
    if (a >= 0x477FF000u) return sign | 0x7C00u;            // >= 65520 rounds to inf
    if (a < 0x38800000u) {                                   // below 2^-14: subnormal (or 0)
        // |f| * 2^24 is exact and below 1024; rounding it to an integer (ties
        // to even, the default rounding mode) gives the subnormal fraction;
        // 1024 is the smallest normal's encoding
        const float scaled = u2f(a) * 0x1p24f;
        return sign | (uint16_t)std::nearbyint(scaled);
    }
    // normal: rebias the exponent, keep 10 fraction bits, round on the 13 dropped bits
    uint32_t r = (((a >> 23) - 112u) << 10) | ((a >> 13) & 0x3FFu);
    const uint32_t rem = a & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r += 1;   // a carry rolls into the exponent
    return sign | (uint16_t)r;
}

// binary32 -> bfloat16 (the upper half), round to nearest, ties to even; NaN to a quiet NaN.
inline uint16_t f32_to_bf16(float f) {
    const uint32_t x = f2u(f);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x0040u);
    const uint32_t lsb = (x >> 16) & 1u;
    return (uint16_t)((x + 0x7FFFu + lsb) >> 16);
}

// ---------------------------------------------------------------- vectorizable inner passes

ZS_CLONES void decode_f16(const uint16_t* __restrict in, float* __restrict out, int n) {
    for (int i = 0; i < n; ++i) out[i] = f16_to_f32(in[i]);
}
ZS_CLONES void decode_bf16(const uint16_t* __restrict in, float* __restrict out, int n) {
    for (int i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}
ZS_CLONES void encode_f16(const float* __restrict in, uint16_t* __restrict out, int n) {
    for (int i = 0; i < n; ++i) out[i] = f32_to_f16(in[i]);
}
ZS_CLONES void encode_bf16(const float* __restrict in, uint16_t* __restrict out, int n) {
    for (int i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

// sum of squares of g[0..n) in float64 with 8 interleaved accumulators
// (element i goes to accumulator i % 8), combined in a fixed order
ZS_CLONES double sum_squares(const float* __restrict g, int n) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int i = 0;
    for (; i + 8 <= n; i += 8)
        for (int k = 0; k < 8; ++k) {
            const double x = (double)g[i + k];
            acc[k] += x * x;
        }
    for (; i < n; ++i) {
        const double x = (double)g[i];
        acc[i & 7] += x * x;
    }
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// 1 if any 16-bit (mask 0x7C00 / 0x7F80) or fp32 (0x7F800000) value has an all-ones exponent
ZS_CLONES int any_nonfinite16(const uint16_t* __restrict h, int n, uint16_t mask) {
    int bad = 0;
    for (int i = 0; i < n; ++i) bad |= (h[i] & mask) == mask;
    return bad;
}
ZS_CLONES int any_nonfinite32(const float* __restrict g, int n) {
    int bad = 0;
    for (int i = 0; i < n; ++i) bad |= (f2u(g[i]) & 0x7F800000u) == 0x7F800000u;
    return bad;
}

// AdamW on n elements in place on p, m, v; g holds the raw gradient values
// (decoded to float) and gscale the unscale-and-clip factor.  The same
// float32 operations in the same order as the device update (fused
// multiply-adds where it has them), so host and device steps agree bit for bit.
ZS_CLONES void adam_f32(float* __restrict p, float* __restrict m, float* __restrict v, const float* __restrict g,
                        int n, float gscale, float b1, float omb1, float b2, float omb2, float step_size,
                        float rsqrt_bc2, float eps, float decay) {
    for (int i = 0; i < n; ++i) {
        const float gi = g[i] * gscale;
        const float mi = std::fma(b1, m[i], omb1 * gi);
        const float vi = std::fma(b2, v[i], (omb2 * gi) * gi);   // finite wherever v is (g g alone overflows past 2^64)
        const float denom = std::fma(std::sqrt(vi), rsqrt_bc2, eps);
        p[i] = std::fma(p[i], decay, -((step_size * mi) / denom));
        m[i] = mi;
        v[i] = vi;
    }
}

// dst[0, n) = src[0, n) for the 16-bit parameter copy, with non-temporal
// (streaming) stores from the first 32-byte boundary of dst on: the host
// never reads the copy back, so its cache lines need not be fetched before
// they are written (the write-allocate read, 2 bytes per element).  Ordinary
// stores cover the unaligned head and the tail.  The caller issues an sfence
// before the copy is handed on.
typedef uint16_t u16x16 __attribute__((vector_size(32)));
ZS_CLONES void store_stream16(uint16_t* __restrict dst, const uint16_t* __restrict src, int n) {
    int i = 0;
    while (i < n && (reinterpret_cast<uintptr_t>(dst + i) & 31u) != 0) {
        dst[i] = src[i];
        ++i;
    }
    for (; i + 16 <= n; i += 16) {
        u16x16 v;
        std::memcpy(&v, src + i, sizeof(v));
        __builtin_nontemporal_store(v, reinterpret_cast<u16x16*>(dst + i));
    }
    for (; i < n; ++i) dst[i] = src[i];
}

// dst = src over n floats, in the same vectorized store style as adam_f32
ZS_CLONES void copy_f32(float* __restrict dst, const float* __restrict src, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = src[i];
}

// ---------------------------------------------------------------- threading

int resolve_threads(int32_t nthreads, int64_t nchunks) {
    int t = nthreads > 0 ? nthreads : (int)std::thread::hardware_concurrency();
    if (t < 1) t = 1;
    if ((int64_t)t > nchunks) t = (int)(nchunks > 0 ? nchunks : 1);
    return t;
}

// A persistent pool of worker threads, started on first use and kept for
// the life of the process, so a call costs a wake-up rather than thread
// creation.  One job runs at a time (calls from several host threads queue on
// job_mutex).  A job hands out chunk indices from an atomic counter to the
// calling thread plus up to threads - 1 workers.
class Pool {
  public:
    static Pool& get() {
        static Pool pool;
        return pool;
    }

    int size() const { return (int)workers_.size() + 1; }

    template <typename F>
    void run(int64_t nchunks, int threads, F& fn) {
        std::lock_guard<std::mutex> job(job_mutex_);
        next_.store(0);
        auto body = [&]() {
            for (int64_t c; (c = next_.fetch_add(1)) < nchunks;) fn(c);
        };
        // a forked child inherits the pool object but not its threads
        const int helpers = getpid() == owner_ ? std::min(threads - 1, (int)workers_.size()) : 0;
        if (helpers <= 0) {
            body();
            return;
        }
        {
            std::lock_guard<std::mutex> lk(m_);
            task_ = [&body]() { body(); };
            wanted_ = helpers;
            done_ = 0;
            ++generation_;
        }
        cv_.notify_all();
        body();
        std::unique_lock<std::mutex> lk(m_);
        done_cv_.wait(lk, [&] { return done_ == helpers; });
        task_ = nullptr;
    }

  private:
    Pool() : owner_(getpid()) {
        const int hw = (int)std::thread::hardware_concurrency();
        for (int i = 0; i + 1 < (hw > 1 ? hw : 1); ++i) workers_.emplace_back([this, i] { loop(i); });
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> lk(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : workers_) t.join();
    }

    void loop(int index) {
        uint64_t seen = 0;
        for (;;) {
            std::function<void()> task;
            {
                std::unique_lock<std::mutex> lk(m_);
                cv_.wait(lk, [&] { return stop_ || generation_ != seen; });
                if (stop_) return;
                seen = generation_;
                if (index >= wanted_) continue;      // not needed for this job
                task = task_;
            }
            task();
            {
                std::lock_guard<std::mutex> lk(m_);
                ++done_;
            }
            done_cv_.notify_one();
        }
    }

    const pid_t owner_;
    std::vector<std::thread> workers_;
    std::mutex job_mutex_, m_;
    std::condition_variable cv_, done_cv_;
    std::function<void()> task_;
    std::atomic<int64_t> next_{0};
    uint64_t generation_ = 0;
    int wanted_ = 0, done_ = 0;
    bool stop_ = false;
};

// runs fn(chunk index) for every chunk on `threads` threads (dynamic assignment)
template <typename F>
void for_chunks(int64_t nchunks, int threads, F fn) {
    Pool::get().run(nchunks, threads, fn);
}

// decodes gradient elements [e, e + cnt) (cnt <= kTile) to float
inline void grad_tile(const void* grad, int32_t dt, int64_t e, int cnt, float* out) {
    if (dt == ZERO_F32) std::memcpy(out, static_cast<const float*>(grad) + e, (size_t)cnt * 4);
    else if (dt == ZERO_F16) decode_f16(static_cast<const uint16_t*>(grad) + e, out, cnt);
    else decode_bf16(static_cast<const uint16_t*>(grad) + e, out, cnt);
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" {

int zero_cpu_shard_unscale_norm_overflow(const void* grad, int32_t grad_dtype, int64_t n, double inv_loss_scale,
                                         double* sqnorm, int32_t* overflow, int32_t nthreads) {
    clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    if (sqnorm == nullptr || overflow == nullptr) return fail(ZERO_EINVAL, "NULL output pointer");
    if (n > 0 && grad == nullptr) return fail(ZERO_EINVAL, "grad is NULL");
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    std::vector<double> part((size_t)nchunks, 0.0);
    std::vector<int> bad((size_t)nchunks, 0);
    const uint16_t mask = grad_dtype == ZERO_F16 ? 0x7C00u : 0x7F80u;
    for_chunks(nchunks, resolve_threads(nthreads, nchunks), [&](int64_t c) {
        float buf[kTile];
        const int64_t lo = c * kChunk, hi = lo + kChunk < n ? lo + kChunk : n;
        double s = 0.0;
        int b = 0;
        for (int64_t e = lo; e < hi; e += kTile) {
            const int cnt = (int)(hi - e < kTile ? hi - e : kTile);
            if (grad_dtype == ZERO_F32) b |= any_nonfinite32(static_cast<const float*>(grad) + e, cnt);
            else b |= any_nonfinite16(static_cast<const uint16_t*>(grad) + e, cnt, mask);
            grad_tile(grad, grad_dtype, e, cnt, buf);
            s += sum_squares(buf, cnt);
        }
        part[(size_t)c] = s;
        bad[(size_t)c] = b;
    });
    double total = 0.0;
    int any = 0;
    for (int64_t c = 0; c < nchunks; ++c) {   // chunk order: independent of the thread count
        total += part[(size_t)c];
        any |= bad[(size_t)c];
    }
    *sqnorm = total * (inv_loss_scale * inv_loss_scale);
    *overflow = any ? 1 : 0;
    return ZERO_OK;
}

int zero_cpu_shard_adam_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, int32_t grad_dtype,
                             void* param_out, int32_t param_dtype, int64_t n, const zero_adam_params* hp,
                             double global_sqnorm, int32_t global_overflow, int32_t nthreads) {
    clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (param_out != nullptr && param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "unknown param_dtype %d", param_dtype);
    StepCoef c;
    const int pst = prepare_adam(hp, &c);
    if (pst != ZERO_OK) return pst;
    if (global_overflow) return ZERO_OK;          // skipped step: nothing is written
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad) return fail(ZERO_EINVAL, "NULL shard pointer");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    const int64_t b32 = n * 4, b16 = n * 2, bg = n * (grad_dtype == ZERO_F32 ? 4 : 2);
    if (overlaps(grad, bg, master, b32) || overlaps(grad, bg, exp_avg, b32) || overlaps(grad, bg, exp_avg_sq, b32) ||
        (param_out && overlaps(grad, bg, param_out, b16)) || overlaps(master, b32, exp_avg, b32) ||
        overlaps(master, b32, exp_avg_sq, b32) || overlaps(exp_avg, b32, exp_avg_sq, b32) ||
        (param_out && (overlaps(param_out, b16, master, b32) || overlaps(param_out, b16, exp_avg, b32) ||
                       overlaps(param_out, b16, exp_avg_sq, b32))))
        return fail(ZERO_EINVAL, "shard buffers overlap");
    float gscale = c.gscale_fixed;
    if (c.clip) {
        // the same double-precision clip coefficient the device path forms
        const double norm = std::sqrt(global_sqnorm);
        double coef = c.max_norm / (norm + 1e-6);
        if (!(coef < 1.0)) coef = 1.0;
        gscale = (float)(c.inv_scale * coef);
    }
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    for_chunks(nchunks, resolve_threads(nthreads, nchunks), [&](int64_t ch) {
        float g[kTile];
        uint16_t p16[kTile];
        const int64_t lo = ch * kChunk, hi = lo + kChunk < n ? lo + kChunk : n;
        for (int64_t e = lo; e < hi; e += kTile) {
            const int cnt = (int)(hi - e < kTile ? hi - e : kTile);
            grad_tile(grad, grad_dtype, e, cnt, g);
            adam_f32(master + e, exp_avg + e, exp_avg_sq + e, g, cnt, gscale, c.beta1, c.omb1, c.beta2, c.omb2,
                     c.step_size, c.rsqrt_bc2, c.eps, c.decay);
            if (param_out != nullptr) {
                if (param_dtype == ZERO_F16) encode_f16(master + e, p16, cnt);
                else encode_bf16(master + e, p16, cnt);
                store_stream16(static_cast<uint16_t*>(param_out) + e, p16, cnt);
            }
        }
        // the streaming stores are weakly ordered: complete them before this
        // chunk counts as done (the caller may hand the copy to a DMA engine)
        _mm_sfence();
    });
    return ZERO_OK;
}

int zero_cpu_copy_reference(void* dst, const void* src, int64_t bytes, int32_t nthreads) {
    clear_error();
    if (bytes < 0 || (bytes & 3)) return fail(ZERO_EINVAL, "bytes must be a non-negative multiple of 4");
    if (bytes == 0) return ZERO_OK;
    if (dst == nullptr || src == nullptr) return fail(ZERO_EINVAL, "NULL pointer");
    if (overlaps(dst, bytes, src, bytes)) return fail(ZERO_EINVAL, "dst and src overlap");
    const int64_t n = bytes / 4;
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    for_chunks(nchunks, resolve_threads(nthreads, nchunks), [&](int64_t ch) {
        const int64_t lo = ch * kChunk, hi = lo + kChunk < n ? lo + kChunk : n;
        copy_f32(static_cast<float*>(dst) + lo, static_cast<const float*>(src) + lo, hi - lo);
    });
    return ZERO_OK;
}

}  // extern "C"
