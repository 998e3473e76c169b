// Device part of the C ABI: the two streaming passes of one ZeRO rank's
// mixed-precision Adam step over its shard, for gfx950 (MI355X, CDNA4).
//
// What is computed follows the explainer "Data Parallelism Without the
// Copies" of "ZeRO: Memory Optimizations Toward Training Trillion Parameter
// Models": "The 16 Bytes per Parameter Audit" and Ch.02 "The Three Stages"
// (fp16 weight + fp32 master + two fp32 moments per parameter; each rank
// updates only its own partition).  The update rule itself is bias-corrected
// Adam (Kingma & Ba 2015) with decoupled weight decay (Loshchilov & Hutter
// 2019); loss scaling and inf/NaN skipping follow Micikevicius et al. 2018;
// clipping is global max-norm clipping (Pascanu et al. 2013).
//
// Both passes are HBM-bandwidth bound elementwise streams (no contraction, so
// no MFMA): threads move whole vectors (16 bytes of fp32, 8 or 16 bytes of
// 16-bit values), consecutive lanes touch consecutive vectors so every wave64
// access instruction is one contiguous run, and the streams are read once, so
// loads and stores are marked non-temporal.
//
//  pass 1  sqnorm_partials + sqnorm_finalize: reads the 2-byte gradient once
//          (2 B/element), ORs an exponent-bits inf/NaN test, sums exact fp64
//          squares per thread in a fixed order, reduces within a wave by
//          xor-shuffles and across the block's four waves through LDS, then a
//          one-block kernel combines the block partials in a fixed order.
//          Only the first block touches the ragged remainder.
//  pass 2  adam_update: 28 B/element (2 grad + 4 master + 4 m + 4 v read,
//          4 + 4 + 4 written back, 2 param written).  One wave64 per
//          workgroup, lane l owning 4 consecutive elements, so each access
//          instruction is one contiguous, fully used run of cache lines; the
//          number of resident waves per CU is capped (see kAdamLdsReserve).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.h"
#include "zero_shard.h"

namespace zero_shard {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;              // four wave64s
constexpr int kWaves = kBlock / 64;
// norm pass: 512 blocks of 256 threads (2 per CU), each step of the
// grid-stride loop reads a 16 KiB chunk per block; chosen by measurement on
// MI355X (~7.1 TB/s on a 2 GB gradient shard)
constexpr int kNormMaxBlocks = 512;
constexpr int kNormUnroll = 4;                          // 16-byte loads in flight per thread
constexpr int64_t kNormChunk = (int64_t)kBlock * kNormUnroll;   // vectors per block per step
// fused update: one wave64 per workgroup, 4 consecutive elements per lane
constexpr int kAdamThreads = 64;
constexpr int kAdamTask = 4 * kAdamThreads;             // elements per workgroup per task
// Occupancy cap.  With eight streams in flight HBM sustains more bytes per
// second when fewer waves compete for DRAM rows: 12 KiB of LDS per
// workgroup leaves room for 13 resident one-wave workgroups per CU (160 KiB
// of LDS per CU on gfx950).  Chosen by measurement on MI355X over 0-32 KiB
// (0 KiB: ~75% of HBM peak; 12 KiB: ~82%; 32 KiB: ~55%).
constexpr size_t kAdamLdsReserve = 12 * 1024;
constexpr int64_t kAdamMaxGrid = (int64_t(1) << 26) - 1;   // grid * 64 work-items < 2^32

// ---------------------------------------------------------------- 16-bit helpers

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// low and high 16-bit halves of a 32-bit word as float
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
    if constexpr (DT == ZERO_F16) {
        lo = f16_to_f32(w & 0xFFFFu);
        hi = f16_to_f32(w >> 16);
    } else {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xFFFF0000u);
    }
}

// round-to-nearest-even float -> 16-bit bits (hardware conversion under the
// default round-to-nearest-even mode: v_cvt_f16_f32 / v_cvt_pk_bf16_f32)
template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
    if constexpr (DT == ZERO_F16) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
    } else {
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    }
}

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_stream(T v, T* p) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- block reduction

__device__ __forceinline__ void block_reduce(double& acc, uint32_t& bad, double* s_sq, uint32_t* s_bad) {
    for (int off = 32; off > 0; off >>= 1) {
        acc += __shfl_xor(acc, off, 64);
        bad |= __shfl_xor(bad, off, 64);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        s_sq[wave] = acc;
        s_bad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = s_sq[0];
        uint32_t b = s_bad[0];
        for (int w = 1; w < kWaves; ++w) {
            t += s_sq[w];
            b |= s_bad[w];
        }
        acc = t;
        bad = b;
    }
}

// ---------------------------------------------------------------- pass 1

// Per 32-bit word of two 16-bit values: (w & E) + C sets bit 15 (bit 31) iff
// the low (high) half has an all-ones exponent field, i.e. is inf or NaN;
// no carry crosses from the low half into the high half.  OR-accumulating
// these words and testing kNonfiniteBits at the end is an exact inf/NaN test.
template <int DT>
struct Exp16 {
    static constexpr uint32_t mask2 = DT == ZERO_F16 ? 0x7C007C00u : 0x7F807F80u;
    static constexpr uint32_t carry2 = DT == ZERO_F16 ? 0x04000400u : 0x00800080u;
};
constexpr uint32_t kNonfiniteBits = 0x80008000u;

template <int DT>
__device__ __forceinline__ void accumulate_vec(u32x4 q, double& acc, uint32_t& bad) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float lo, hi;
        unpack2<DT>(q[k], lo, hi);
        bad |= (q[k] & Exp16<DT>::mask2) + Exp16<DT>::carry2;
        const double a = (double)lo, b = (double)hi;   // exact; squares exact in fp64
        acc = fma(a, a, acc);
        acc = fma(b, b, acc);
    }
}

// Grid-stride over chunks of kNormChunk consecutive 16-byte vectors: at every
// step the grid reads one contiguous window, and each wave's four loads are
// consecutive 1 KiB runs.  The grid size depends only on n, so the summation
// order (and the result) is the same on every run.
template <int DT>
__global__ __launch_bounds__(kBlock) void sqnorm_partials(const u32x4* __restrict__ g, int64_t nvec,
                                                          const uint16_t* __restrict__ tail, int tail_n,
                                                          double* __restrict__ part_sq,
                                                          uint32_t* __restrict__ part_bad) {
    __shared__ double s_sq[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    double acc = 0.0;
    uint32_t bad = 0;
    const int64_t nchunks = nvec / kNormChunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const u32x4* base = g + c * kNormChunk + threadIdx.x;
        u32x4 q[kNormUnroll];
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) q[u] = ld_stream(base + u * kBlock);
#pragma unroll
        for (int u = 0; u < kNormUnroll; ++u) accumulate_vec<DT>(q[u], acc, bad);
    }
    if (blockIdx.x == 0) {
        // fewer than kNormChunk vectors left over, then fewer than 8 elements
        for (int64_t i = nchunks * kNormChunk + threadIdx.x; i < nvec; i += kBlock)
            accumulate_vec<DT>(ld_stream(g + i), acc, bad);
        if (threadIdx.x == 0) {
            for (int k = 0; k < tail_n; ++k) {
                const uint32_t h = tail[k];
                const float x = DT == ZERO_F16 ? f16_to_f32(h) : bf16_to_f32(h);
                bad |= (h & Exp16<DT>::mask2) + Exp16<DT>::carry2;
                const double a = (double)x;
                acc = fma(a, a, acc);
            }
        }
    }
    bad = (bad & kNonfiniteBits) != 0;
    block_reduce(acc, bad, s_sq, s_bad);
    if (threadIdx.x == 0) {
        part_sq[blockIdx.x] = acc;
        part_bad[blockIdx.x] = bad;
    }
}

__global__ __launch_bounds__(kBlock) void sqnorm_finalize(const double* __restrict__ part_sq,
                                                          const uint32_t* __restrict__ part_bad,
                                                          int nparts, double inv2,
                                                          double* __restrict__ d_sq,
                                                          int32_t* __restrict__ d_ovf) {
    __shared__ double s_sq[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    double acc = 0.0;
    uint32_t bad = 0;
    for (int i = threadIdx.x; i < nparts; i += kBlock) {
        acc += part_sq[i];
        bad |= part_bad[i];
    }
    block_reduce(acc, bad, s_sq, s_bad);
    if (threadIdx.x == 0) {
        *d_sq = acc * inv2;
        *d_ovf = bad ? 1 : 0;
    }
}

int norm_blocks(int64_t n) {
    int64_t b = (n / 8) / kNormChunk;      // one block per full chunk, at most kNormMaxBlocks
    if (b < 1) b = 1;
    if (b > kNormMaxBlocks) b = kNormMaxBlocks;
    return (int)b;
}

// ---------------------------------------------------------------- pass 2

struct AdamCoef {
    float beta1, omb1, beta2, omb2;   // beta, 1 - beta (each rounded once from double)
    float step_size;                  // lr / (1 - beta1^t)
    float rsqrt_bc2;                  // 1 / sqrt(1 - beta2^t)
    float eps;
    float decay;                      // 1 - lr * wd
    float gscale_fixed;               // float(inv_scale) when clipping is off
    int clip;
    double inv_scale, max_norm;
};

__device__ __forceinline__ void adam_elem(const AdamCoef& c, float gscale, float graw, float& p, float& m,
                                          float& v) {
    const float g = graw * gscale;
    m = fmaf(c.beta1, m, c.omb1 * g);
    v = fmaf(c.beta2, v, c.omb2 * (g * g));
    const float denom = fmaf(sqrtf(v), c.rsqrt_bc2, c.eps);
    p = fmaf(p, c.decay, -(c.step_size * m) / denom);
}

template <int GDT, int PDT, bool WRITE_P>
__global__ __launch_bounds__(kAdamThreads) void adam_update(float* __restrict__ P, float* __restrict__ M,
                                                            float* __restrict__ V,
                                                            const uint16_t* __restrict__ G,
                                                            uint16_t* __restrict__ Pout, int64_t n, AdamCoef c,
                                                            const double* __restrict__ d_sq,
                                                            const int32_t* __restrict__ d_ovf) {
    // Dynamic LDS reserved by the launcher only to cap how many of these
    // workgroups (one wave each) are resident per CU; it is never read.
    extern __shared__ float occupancy_pad[];
    // skipped step: the whole grid sees the same flag and writes nothing
    if (d_ovf != nullptr && *d_ovf != 0) return;
    float gscale = c.gscale_fixed;
    if (c.clip) {
        const double norm = sqrt(*d_sq);
        double coef = c.max_norm / (norm + 1e-6);
        if (!(coef < 1.0)) coef = 1.0;
        gscale = (float)(c.inv_scale * coef);
    }
    const int lane = threadIdx.x;
    const int64_t ntasks = (n + kAdamTask - 1) / kAdamTask;
    for (int64_t t = blockIdx.x; t < ntasks; t += gridDim.x) {
        // lane owns elements [e0, e0 + 4): every access instruction of the wave
        // covers one contiguous run (1 KiB per fp32 stream, 512 B per 16-bit one)
        const int64_t e0 = t * kAdamTask + 4 * lane;
        if (e0 + 4 <= n) {
            const int64_t q = e0 >> 2;
            f32x4* p4 = reinterpret_cast<f32x4*>(P) + q;
            f32x4* m4 = reinterpret_cast<f32x4*>(M) + q;
            f32x4* v4 = reinterpret_cast<f32x4*>(V) + q;
            f32x4 p = ld_stream(p4), m = ld_stream(m4), v = ld_stream(v4);
            const u32x2 gq = ld_stream(reinterpret_cast<const u32x2*>(G) + q);
            float g[4];
            unpack2<GDT>(gq[0], g[0], g[1]);
            unpack2<GDT>(gq[1], g[2], g[3]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float pk = p[k], mk = m[k], vk = v[k];
                adam_elem(c, gscale, g[k], pk, mk, vk);
                p[k] = pk;
                m[k] = mk;
                v[k] = vk;
            }
            st_stream(p, p4);
            st_stream(m, m4);
            st_stream(v, v4);
            if constexpr (WRITE_P) {
                u32x2 out16;
                out16[0] = to16<PDT>(p[0]) | (to16<PDT>(p[1]) << 16);
                out16[1] = to16<PDT>(p[2]) | (to16<PDT>(p[3]) << 16);
                st_stream(out16, reinterpret_cast<u32x2*>(Pout) + q);
            }
        } else if (e0 < n) {
            // ragged tail: the last 1-3 elements, scalar accesses
            for (int64_t e = e0; e < n; ++e) {
                const uint32_t h = G[e];
                const float graw = GDT == ZERO_F16 ? f16_to_f32(h) : bf16_to_f32(h);
                float p = P[e], m = M[e], v = V[e];
                adam_elem(c, gscale, graw, p, m, v);
                P[e] = p;
                M[e] = m;
                V[e] = v;
                if constexpr (WRITE_P) Pout[e] = (uint16_t)to16<PDT>(p);
            }
        }
    }
    if (n < 0) occupancy_pad[lane] = 0.0f;   // never taken (n >= 0): keeps the reservation referenced
}

// ---------------------------------------------------------------- host helpers

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

template <int GDT, int PDT, bool WRITE_P>
void launch_adam(dim3 grid, hipStream_t s, float* P, float* M, float* V, const void* G, void* Pout,
                 int64_t n, const AdamCoef& c, const double* d_sq, const int32_t* d_ovf) {
    hipLaunchKernelGGL((adam_update<GDT, PDT, WRITE_P>), grid, dim3(kAdamThreads), kAdamLdsReserve, s, P, M, V,
                       static_cast<const uint16_t*>(G), static_cast<uint16_t*>(Pout), n, c, d_sq, d_ovf);
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" {

size_t zero_norm_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    const size_t b = (size_t)norm_blocks(n);
    return ((b * (sizeof(double) + sizeof(uint32_t))) + 255) & ~(size_t)255;
}

int zero_shard_unscale_norm_overflow(const void* grad, int32_t grad_dtype, int64_t n, double inv_loss_scale,
                                     double* d_sqnorm, int32_t* d_overflow, void* d_workspace,
                                     size_t workspace_bytes, void* hip_stream) {
    clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16) return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    if (d_sqnorm == nullptr || d_overflow == nullptr || d_workspace == nullptr)
        return fail(ZERO_EINVAL, "NULL output or workspace pointer");
    if (n > 0 && grad == nullptr) return fail(ZERO_EINVAL, "grad is NULL");
    if ((n > 0 && !aligned16(grad)) || !aligned16(d_workspace))
        return fail(ZERO_EALIGN, "grad and workspace must be 16-byte aligned");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u))
        return fail(ZERO_EALIGN, "d_sqnorm / d_overflow misaligned");
    if (workspace_bytes < zero_norm_workspace_bytes(n))
        return fail(ZERO_ENOSPC, "workspace %zu bytes, need %zu", workspace_bytes, zero_norm_workspace_bytes(n));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int nb = norm_blocks(n);
    double* part_sq = static_cast<double*>(d_workspace);
    uint32_t* part_bad = reinterpret_cast<uint32_t*>(part_sq + nb);
    const int64_t nvec = n / 8;
    const int tail_n = (int)(n - nvec * 8);
    const uint16_t* tail = static_cast<const uint16_t*>(grad) + nvec * 8;
    if (n > 0) {
        if (grad_dtype == ZERO_F16)
            hipLaunchKernelGGL(sqnorm_partials<ZERO_F16>, dim3(nb), dim3(kBlock), 0, s,
                               static_cast<const u32x4*>(grad), nvec, tail, tail_n, part_sq, part_bad);
        else
            hipLaunchKernelGGL(sqnorm_partials<ZERO_BF16>, dim3(nb), dim3(kBlock), 0, s,
                               static_cast<const u32x4*>(grad), nvec, tail, tail_n, part_sq, part_bad);
        const int st = launch_status("sqnorm_partials");
        if (st != ZERO_OK) return st;
    }
    hipLaunchKernelGGL(sqnorm_finalize, dim3(1), dim3(kBlock), 0, s, part_sq, part_bad, n > 0 ? nb : 0,
                       inv_loss_scale * inv_loss_scale, d_sqnorm, d_overflow);
    return launch_status("sqnorm_finalize");
}

int zero_shard_adam_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, int32_t grad_dtype,
                         void* param_out, int32_t param_dtype, int64_t n, const zero_adam_params* hp,
                         const double* d_global_sqnorm, const int32_t* d_global_overflow, void* hip_stream) {
    clear_error();
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16) return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (param_out != nullptr && param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "unknown param_dtype %d", param_dtype);
    const zero_adam_params& h = *hp;
    if (!(h.lr >= 0.0) || !std::isfinite(h.lr)) return fail(ZERO_EINVAL, "lr must be finite and >= 0");
    if (!(h.beta1 >= 0.0 && h.beta1 < 1.0) || !(h.beta2 >= 0.0 && h.beta2 < 1.0))
        return fail(ZERO_EINVAL, "betas must lie in [0, 1)");
    if (!(h.eps >= 0.0) || !std::isfinite(h.eps)) return fail(ZERO_EINVAL, "eps must be finite and >= 0");
    if (!(h.weight_decay >= 0.0) || !std::isfinite(h.weight_decay))
        return fail(ZERO_EINVAL, "weight_decay must be finite and >= 0");
    if (h.step < 1) return fail(ZERO_EINVAL, "step (1-based index of the step applied) must be >= 1");
    if (!(h.inv_loss_scale > 0.0) || !std::isfinite(h.inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    const bool clip = h.max_grad_norm > 0.0;
    if (clip && !std::isfinite(h.max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm must be finite");
    if (clip && d_global_sqnorm == nullptr) return fail(ZERO_EINVAL, "clipping needs d_global_sqnorm");
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad) return fail(ZERO_EINVAL, "NULL shard pointer");
    if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(grad) ||
        (param_out && !aligned16(param_out)))
        return fail(ZERO_EALIGN, "shard pointers must be 16-byte aligned");
    if (d_global_sqnorm && ((uintptr_t)d_global_sqnorm & 7u)) return fail(ZERO_EALIGN, "d_global_sqnorm misaligned");
    if (d_global_overflow && ((uintptr_t)d_global_overflow & 3u)) return fail(ZERO_EALIGN, "d_global_overflow misaligned");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    const int64_t b32 = n * 4, b16 = n * 2;
    if (overlaps(grad, b16, master, b32) || overlaps(grad, b16, exp_avg, b32) ||
        overlaps(grad, b16, exp_avg_sq, b32) || (param_out && overlaps(grad, b16, param_out, b16)))
        return fail(ZERO_EINVAL, "grad aliases an output");
    if (overlaps(master, b32, exp_avg, b32) || overlaps(master, b32, exp_avg_sq, b32) ||
        overlaps(exp_avg, b32, exp_avg_sq, b32) ||
        (param_out && (overlaps(param_out, b16, master, b32) || overlaps(param_out, b16, exp_avg, b32) ||
                       overlaps(param_out, b16, exp_avg_sq, b32))))
        return fail(ZERO_EINVAL, "state buffers overlap");

    // per-step coefficients: derived in double, each rounded once to float
    AdamCoef c;
    const double t = (double)h.step;
    const double bc1 = 1.0 - std::pow(h.beta1, t);
    const double bc2 = 1.0 - std::pow(h.beta2, t);
    if (!(bc1 > 0.0) || !(bc2 > 0.0)) return fail(ZERO_ERANGE, "bias correction underflows to 0");
    c.beta1 = (float)h.beta1;
    c.omb1 = (float)(1.0 - h.beta1);
    c.beta2 = (float)h.beta2;
    c.omb2 = (float)(1.0 - h.beta2);
    c.step_size = (float)(h.lr / bc1);
    c.rsqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    c.eps = (float)h.eps;
    c.decay = (float)(1.0 - h.lr * h.weight_decay);
    c.gscale_fixed = (float)h.inv_loss_scale;
    c.clip = clip ? 1 : 0;
    c.inv_scale = h.inv_loss_scale;
    c.max_norm = clip ? h.max_grad_norm : 0.0;

    int64_t ntasks = (n + kAdamTask - 1) / kAdamTask;
    if (ntasks > kAdamMaxGrid) ntasks = kAdamMaxGrid;   // the kernel strides over the rest
    const dim3 grid((unsigned)ntasks);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool wp = param_out != nullptr;
    const int pdt = wp ? param_dtype : ZERO_F16;
#define ZS_LAUNCH(G, P, W) launch_adam<G, P, W>(grid, s, master, exp_avg, exp_avg_sq, grad, param_out, n, c, \
                                                 d_global_sqnorm, d_global_overflow)
    if (grad_dtype == ZERO_F16) {
        if (!wp) ZS_LAUNCH(ZERO_F16, ZERO_F16, false);
        else if (pdt == ZERO_F16) ZS_LAUNCH(ZERO_F16, ZERO_F16, true);
        else ZS_LAUNCH(ZERO_F16, ZERO_BF16, true);
    } else {
        if (!wp) ZS_LAUNCH(ZERO_BF16, ZERO_BF16, false);
        else if (pdt == ZERO_BF16) ZS_LAUNCH(ZERO_BF16, ZERO_BF16, true);
        else ZS_LAUNCH(ZERO_BF16, ZERO_F16, true);
    }
#undef ZS_LAUNCH
    return launch_status("adam_update");
}

}  // extern "C"
