// Device part of the C ABI: the streaming passes of one ZeRO rank's
// mixed-precision Adam step over its shard, for gfx950 (MI355X, CDNA4).
//
// What is computed follows the explainer "Data Parallelism Without the
// Copies" of "ZeRO: Memory Optimizations Toward Training Trillion Parameter
// Models": "The 16 Bytes per Parameter Audit" and Ch.02 "The Three Stages"
// (fp16 weight + fp32 master + two fp32 moments per parameter, optionally an
// fp32 copy of the gradient; each rank updates only its own partition).  The
// update rule itself is bias-corrected Adam (Kingma & Ba 2015) with decoupled
// weight decay (Loshchilov & Hutter 2019); loss scaling and inf/NaN skipping
// follow Micikevicius et al. 2018; clipping is global max-norm clipping
// (Pascanu et al. 2013).
//
// Every pass is an HBM-bandwidth bound elementwise stream (no contraction,
// so no MFMA): threads move whole vectors (16 bytes of fp32, 8 or 16 bytes of
// 16-bit values), consecutive lanes touch consecutive vectors so every wave64
// access instruction is one contiguous run, and the streams are read once, so
// loads and stores are marked non-temporal.
//
//  sqnorm_partials + sqnorm_finalize: reads the gradient once (2 B/element,
//          4 for an fp32 gradient), ORs an exponent-bits inf/NaN test, sums
//          exact fp64 squares per thread in a fixed order, reduces within a
//          wave by xor-shuffles and across the block's four waves through
//          LDS, then a one-block kernel combines the block partials in a
//          fixed order (and multiplies by 1/scale^2).  Only the first block
//          touches the ragged remainder.
//  adam_update: 28 B/element (2 grad + 4 master + 4 m + 4 v read, 4 + 4 + 4
//          written back, 2 param written; 30 with an fp32 gradient).  One
//          wave64 per workgroup, lane l owning 4 consecutive elements, so
//          each access instruction is one contiguous, fully used run of
//          cache lines; the number of resident waves per CU is capped.
//          adam_update_devcoef is the same body with its coefficients read
//          from device memory.
//  grad_accumulate: acc = (first ? 0 : acc) + g * inv_scale into the fp32
//          gradient copy, 10 B/element (6 for the first micro-batch), the
//          same lane layout as adam_update but with no occupancy cap.
//  grad_reduce: acc = sum over K ranks' 16-bit slices * inv_scale, in slice
//          order (the local half of the gradient reduce-scatter), 2K + 4 B.
//  grad_sum_norm + task_partials_reduce: the accumulation or the reduction
//          with the norm of the result formed in the same pass (one fp64
//          partial per one-wave task, folded in a fixed order), so the
//          norm pass over the fp32 copy is not needed.
//  step_decide (and sqnorm_finalize's decision): with the loss scaler and
//          step counter in device memory, one thread forms the step's
//          coefficient block and advances the scaler from the overflow flag.
// The host-side entry points at the end check every argument before
// enqueuing anything, and the step-graph calls record these passes as HIP
// graphs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <type_traits>
#include <utility>

#include "common.h"
#include "zero_shard.h"

namespace zero_shard {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;              // four wave64s
constexpr int kWaves = kBlock / 64;
// norm pass: at most 512 blocks of 256 threads (2 per CU); each step of the
// grid-stride loop reads a 16 KiB chunk per block.  Chosen by measurement on
// MI355X (~7.1 TB/s on a 2 GB gradient shard).
constexpr int kNormMaxBlocks = 512;
// 16-byte loads in flight per thread: 4 for a 16-bit gradient, 8 for an fp32
// one (fp32: 7.1 TB/s with 8 against 6.5 with 4 on a 3.9 GB gradient; 16-bit:
// 4 is best at 0.5 and 2 GB), so a block step covers 8K elements either way.
// elementwise passes: one wave64 per workgroup, 4 consecutive elements per lane
constexpr int kEwThreads = 64;
constexpr int kEwTask = 4 * kEwThreads;                         // elements per workgroup per task
// AdamW pass.  Each one-wave workgroup takes kAdamTasks consecutive tasks
// and issues all their loads before any math; an LDS reservation that is
// never read caps how many such workgroups are resident per CU (160 KiB of
// LDS per CU on gfx950).  With eight streams in flight HBM sustains more bytes
// per second when fewer waves compete for DRAM rows.  Chosen by measurement on
// MI355X, a 976M-element shard on physically contiguous buffers, all shapes in
// one process: 1 task with 14 KiB (11 workgroups per CU) 83.5% of HBM peak
// for a bf16 gradient and 83.2% for an fp32 one, 15 KiB the same, 13 KiB
// 83.3% / 82.6%, 12 KiB 82.7% / 82.3% (0 KiB ~75%, 32 KiB ~55%); 2 tasks at
// 18-22 KiB 82.5-82.9% / 80.5-80.9%; 4 tasks at 24-32 KiB 74-82%.  More tasks
// per workgroup make a skipped step cheaper (every workgroup reads the flag
// and exits: 0.81, 0.41 and 0.21 ms for 1, 2 and 4 tasks on that shard), but
// skipped steps are rare and applied ones are not.
// Task t goes to workgroup t, so consecutive 1 KiB runs of each stream go to
// the 8 XCDs in turn and the chip streams one narrow window of every buffer.
// Measured over several processes each on the 976M-element shard: XCDs
// streaming their own contiguous eighths ~76%, 2 or 4 consecutive tasks per
// XCD ~80.5% / ~78%, and 512 B tasks (2 elements per lane) ~75-76%, against
// ~81.7% for this layout.
constexpr size_t kAdamLdsReserve = 14 * 1024;
constexpr int kAdamTasks = 1;
constexpr int kAdamGroup = kAdamTasks * kEwTask;                 // elements per workgroup
// The accumulation pass of a later micro-batch (fp32 copy read and written,
// 16-bit gradient read) is fastest as one task per uncapped one-wave
// workgroup: 83.8% of HBM peak on a 976M-element shard (2 tasks 78.8-82.1%,
// 4 tasks 74.6-81.0% over 0-16 KiB caps).  The first micro-batch only writes
// the copy (2 bytes read, 4 written per element): there two tasks per
// workgroup, loads first, with a 7 KiB reservation (22 resident per CU) run at
// 84.1%, the rate of a plain copy reading 8 and writing 16 bytes per lane
// (84.7%), against 77.3% for one uncapped task; 6 and 8-10 KiB 80.6-83.2%.
// The reduction and the fused copy-and-norm pass compiled for 5-8 slices
// (nine or ten streams) gain from a light cap: 6 KiB per one-wave workgroup
// (26 resident per CU instead of 32) took 8 slices on a 976M-element shard
// from 6.49 to 6.63 TB/s (reduction) and from 6.47 to 6.60 TB/s (fused);
// 8 KiB and more lose 10-45%.  Capacities 1-4 and 16, and the accumulation
// kernels, are fastest, or within noise, uncapped.
constexpr size_t kSlices8Lds = 6 * 1024;
constexpr int kAccFirstTasks = 2;
constexpr size_t kAccFirstLds = 7 * 1024;
constexpr int64_t kEwMaxGrid = (int64_t(1) << 26) - 1;          // grid * 64 work-items < 2^32
// gfx950 has 8 XCDs, each with its own L2; consecutive workgroups of a launch
// go to them in turn.  Small per-workgroup results that neighbouring
// workgroups write into one array are laid out XCD by XCD (slot of task t:
// (t % kXcds) * per_xcd + t / kXcds) so each L2 fills whole lines instead of
// eight L2s writing back the same lines sector by sector.
constexpr int kXcds = 8;

// ---------------------------------------------------------------- gradient formats

// Per gradient format: values per 16-byte vector, and the exponent-field test.
// For a 32-bit word w, (w & mask) + carry sets bit 15 (low 16-bit half) or
// bit 31 (high half, or the whole fp32 value) exactly when that value's
// exponent field is all ones, i.e. it is inf or NaN; no carry crosses into
// the neighbouring field.  OR-accumulating these words and testing
// kNonfiniteBits at the end is an exact inf/NaN test.
template <int DT>
struct GradFmt;
template <>
struct GradFmt<ZERO_F16> {
    static constexpr int per_vec = 8;
    static constexpr int norm_unroll = 4;
    static constexpr uint32_t mask = 0x7C007C00u, carry = 0x04000400u;
};
template <>
struct GradFmt<ZERO_BF16> {
    static constexpr int per_vec = 8;
    static constexpr int norm_unroll = 4;
    static constexpr uint32_t mask = 0x7F807F80u, carry = 0x00800080u;
};
template <>
struct GradFmt<ZERO_F32> {
    static constexpr int per_vec = 4;
    static constexpr int norm_unroll = 8;
    static constexpr uint32_t mask = 0x7F800000u, carry = 0x00800000u;
};
constexpr uint32_t kNonfiniteBits = 0x80008000u;

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
// default round-to-nearest-even mode: v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
// x is the float32 master as stored.  The empty asm makes it an opaque
// register value, so the compiler cannot fuse the conversion into the
// arithmetic that produced it: a fused v_fma_mixlo_f16 rounds the unrounded
// result straight to fp16, which differs from rounding the stored float32
// master in the rare cases where the two roundings meet a tie.
template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
    __asm__("" : "+v"(x));
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

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), as straight-line code
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// the 4 gradient values of element group q (elements 4q .. 4q+3)
template <int DT>
__device__ __forceinline__ void load_grad4(const void* G, int64_t q, float g[4]) {
    if constexpr (DT == ZERO_F32) {
        const f32x4 v = ld_stream(static_cast<const f32x4*>(G) + q);
        g[0] = v[0];
        g[1] = v[1];
        g[2] = v[2];
        g[3] = v[3];
    } else {
        const u32x2 w = ld_stream(static_cast<const u32x2*>(G) + q);
        unpack2<DT>(w[0], g[0], g[1]);
        unpack2<DT>(w[1], g[2], g[3]);
    }
}

template <int DT>
__device__ __forceinline__ float load_grad1(const void* G, int64_t e) {
    if constexpr (DT == ZERO_F32) {
        return static_cast<const float*>(G)[e];
    } else {
        const uint32_t h = static_cast<const uint16_t*>(G)[e];
        return DT == ZERO_F16 ? f16_to_f32(h) : bf16_to_f32(h);
    }
}

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

// ---------------------------------------------------------------- norm pass

template <int DT>
__device__ __forceinline__ void accumulate_vec(u32x4 q, double& acc, uint32_t& bad) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bad |= (q[k] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
        if constexpr (DT == ZERO_F32) {
            const double a = (double)__uint_as_float(q[k]);   // exact; square exact in fp64
            acc = fma(a, a, acc);
        } else {
            float lo, hi;
            unpack2<DT>(q[k], lo, hi);
            const double a = (double)lo, b = (double)hi;
            acc = fma(a, a, acc);
            acc = fma(b, b, acc);
        }
    }
}

// Grid-stride over chunks of kChunk consecutive 16-byte vectors: at every
// step the grid reads one contiguous window, and each wave's four loads are
// consecutive 1 KiB runs.  The grid size depends only on n, so the summation
// order (and the result) is the same on every run.
template <int DT>
__global__ __launch_bounds__(kBlock) void sqnorm_partials(const u32x4* __restrict__ g, int64_t nvec,
                                                          const void* __restrict__ tail, int tail_n,
                                                          double* __restrict__ part_sq,
                                                          uint32_t* __restrict__ part_bad) {
    __shared__ double s_sq[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    double acc = 0.0;
    uint32_t bad = 0;
    constexpr int kUnroll = GradFmt<DT>::norm_unroll;
    constexpr int64_t kChunk = (int64_t)kBlock * kUnroll;
    const int64_t nchunks = nvec / kChunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const u32x4* base = g + c * kChunk + threadIdx.x;
        u32x4 q[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) q[u] = ld_stream(base + u * kBlock);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) accumulate_vec<DT>(q[u], acc, bad);
    }
    if (blockIdx.x == 0) {
        // fewer than kChunk vectors left over, then less than one vector
        for (int64_t i = nchunks * kChunk + threadIdx.x; i < nvec; i += kBlock)
            accumulate_vec<DT>(ld_stream(g + i), acc, bad);
        if (threadIdx.x == 0) {
            for (int k = 0; k < tail_n; ++k) {
                uint32_t w;
                if constexpr (DT == ZERO_F32) w = static_cast<const uint32_t*>(tail)[k];
                else w = static_cast<const uint16_t*>(tail)[k];
                bad |= (w & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                const double a = (double)load_grad1<DT>(tail, k);
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

// ---------------------------------------------------------------- device-resident step state

struct HyperArgs {
    double lr, beta1, beta2, eps, weight_decay, max_grad_norm;
};

// After the (global) overflow flag is known: the coefficient block of step
// t = applied + 1 at the current loss scale, then the loss scale and the step
// counts advanced exactly as zero_loss_scaler_update does on the host.  The
// update kernel that follows reads the block and the flag.  One thread.
__device__ void decide_step(zero_step_state* __restrict__ st, int32_t ovf, const HyperArgs& h, int unscaled_grad,
                            StepCoef* __restrict__ coef) {
    zero_loss_scaler s = st->scaler;
    const double inv = unscaled_grad ? 1.0 : 1.0 / s.scale;
    StepCoef c;
    fill_step_coef(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, st->applied + 1, inv, h.max_grad_norm, &c);
    *coef = c;
    if (ovf) {
        const double next = s.scale * s.backoff;
        s.scale = next > s.min_scale ? next : s.min_scale;
        s.good_steps = 0;
        st->skipped += 1;
    } else {
        st->applied += 1;
        s.good_steps += 1;
        if (s.good_steps >= s.growth_interval) {
            s.scale *= s.growth;
            s.good_steps = 0;
        }
    }
    st->scaler = s;
    st->last_overflow = ovf;
}

__global__ __launch_bounds__(64) void step_decide(zero_step_state* __restrict__ st, const int32_t* __restrict__ d_ovf,
                                                  HyperArgs h, int unscaled_grad, StepCoef* __restrict__ coef) {
    if (threadIdx.x == 0) decide_step(st, *d_ovf != 0 ? 1 : 0, h, unscaled_grad, coef);
}

// d_scale (device loss scale) or, if NULL, inv2 by value: the factor applied
// to the raw sum of squares is (1/scale)^2.
// With st_decide set (a single rank, whose flag is the global one), thread 0
// also makes the step's decision (decide_step) from the flag it just formed.
__global__ __launch_bounds__(kBlock) void sqnorm_finalize(const double* __restrict__ part_sq,
                                                          const uint32_t* __restrict__ part_bad,
                                                          int nparts, double inv2,
                                                          const double* __restrict__ d_scale,
                                                          double* __restrict__ d_sq,
                                                          int32_t* __restrict__ d_ovf,
                                                          zero_step_state* __restrict__ st_decide, HyperArgs h,
                                                          int unscaled_grad, StepCoef* __restrict__ coef) {
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
        if (d_scale != nullptr) {
            const double inv = 1.0 / *d_scale;
            inv2 = inv * inv;
        }
        *d_sq = acc * inv2;
        *d_ovf = bad ? 1 : 0;
        if (st_decide != nullptr) decide_step(st_decide, bad ? 1 : 0, h, unscaled_grad, coef);
    }
}

// blocks for a gradient of n elements: one per full block step (8K elements
// in every format), at most kNormMaxBlocks
constexpr int64_t kNormChunkElems = 8192;
int norm_blocks(int64_t n) {
    int64_t b = n / kNormChunkElems;
    if (b < 1) b = 1;
    if (b > kNormMaxBlocks) b = kNormMaxBlocks;
    return (int)b;
}

// ---------------------------------------------------------------- fused AdamW

__device__ __forceinline__ void adam_elem(const StepCoef& c, float gscale, float graw, float& p, float& m,
                                          float& v) {
    const float g = graw * gscale;
    m = fmaf(c.beta1, m, c.omb1 * g);
    // (1 - beta2) g^2 as ((1 - beta2) g) g: the same three roundings as
    // (1 - beta2)(g g), but finite wherever the stored moment is, where g g
    // alone would overflow float32 once |g| passes 2^64
    v = fmaf(c.beta2, v, (c.omb2 * g) * g);
    const float denom = fmaf(sqrtf(v), c.rsqrt_bc2, c.eps);
    p = fmaf(p, c.decay, -(c.step_size * m) / denom);
}

template <int GDT, int PDT, bool WRITE_P>
__device__ __forceinline__ void adam_body(float* __restrict__ P, float* __restrict__ M, float* __restrict__ V,
                                          const void* __restrict__ G, uint16_t* __restrict__ Pout, int64_t n,
                                          const StepCoef& c, const double* __restrict__ d_sq,
                                          const int32_t* __restrict__ d_ovf, float* occupancy_pad) {
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
    const int64_t ngroups = (n + kAdamGroup - 1) / kAdamGroup;
    for (int64_t t = blockIdx.x; t < ngroups; t += gridDim.x) {
        const int64_t base = t * kAdamGroup;
        if (base + kAdamGroup <= n) {
            // lane owns elements [4q, 4q + 4) of each task: every access
            // instruction of the wave covers one contiguous run (1 KiB per
            // fp32 stream, 512 B per 16-bit one)
            f32x4 p[kAdamTasks], m[kAdamTasks], v[kAdamTasks];
            float g[kAdamTasks][4];
            // straight-line code per task (no loop): a loop whose store
            // addresses become invariant gets its stores promoted by LICM,
            // which drops their non-temporal hint
            static_for<kAdamTasks>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int64_t q = (base >> 2) + k * kEwThreads + lane;
                p[k] = ld_stream(reinterpret_cast<f32x4*>(P) + q);
                m[k] = ld_stream(reinterpret_cast<f32x4*>(M) + q);
                v[k] = ld_stream(reinterpret_cast<f32x4*>(V) + q);
                load_grad4<GDT>(G, q, g[k]);
            });
            static_for<kAdamTasks>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int64_t q = (base >> 2) + k * kEwThreads + lane;
                f32x4 po, mo, vo;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float pj = p[k][j], mj = m[k][j], vj = v[k][j];
                    adam_elem(c, gscale, g[k][j], pj, mj, vj);
                    po[j] = pj;
                    mo[j] = mj;
                    vo[j] = vj;
                }
                st_stream(po, reinterpret_cast<f32x4*>(P) + q);
                st_stream(mo, reinterpret_cast<f32x4*>(M) + q);
                st_stream(vo, reinterpret_cast<f32x4*>(V) + q);
                if constexpr (WRITE_P) {
                    u32x2 out16;
                    out16[0] = to16<PDT>(po[0]) | (to16<PDT>(po[1]) << 16);
                    out16[1] = to16<PDT>(po[2]) | (to16<PDT>(po[3]) << 16);
                    st_stream(out16, reinterpret_cast<u32x2*>(Pout) + q);
                }
            });
        } else {
            // the last, partial group: whole vectors, then the 1-3 element
            // ragged tail with scalar accesses
            for (int64_t e0 = base + 4 * lane; e0 < n; e0 += kEwTask) {
                if (e0 + 4 <= n) {
                    const int64_t q = e0 >> 2;
                    f32x4* p4 = reinterpret_cast<f32x4*>(P) + q;
                    f32x4* m4 = reinterpret_cast<f32x4*>(M) + q;
                    f32x4* v4 = reinterpret_cast<f32x4*>(V) + q;
                    f32x4 pv = ld_stream(p4), mv = ld_stream(m4), vv = ld_stream(v4);
                    float gv[4];
                    load_grad4<GDT>(G, q, gv);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float pj = pv[j], mj = mv[j], vj = vv[j];
                        adam_elem(c, gscale, gv[j], pj, mj, vj);
                        pv[j] = pj;
                        mv[j] = mj;
                        vv[j] = vj;
                    }
                    st_stream(pv, p4);
                    st_stream(mv, m4);
                    st_stream(vv, v4);
                    if constexpr (WRITE_P) {
                        u32x2 out16;
                        out16[0] = to16<PDT>(pv[0]) | (to16<PDT>(pv[1]) << 16);
                        out16[1] = to16<PDT>(pv[2]) | (to16<PDT>(pv[3]) << 16);
                        st_stream(out16, reinterpret_cast<u32x2*>(Pout) + q);
                    }
                } else {
                    for (int64_t e = e0; e < n; ++e) {
                        float pe = P[e], me = M[e], ve = V[e];
                        adam_elem(c, gscale, load_grad1<GDT>(G, e), pe, me, ve);
                        P[e] = pe;
                        M[e] = me;
                        V[e] = ve;
                        if constexpr (WRITE_P) Pout[e] = (uint16_t)to16<PDT>(pe);
                    }
                }
            }
        }
    }
    if (n < 0) occupancy_pad[lane] = 0.0f;   // never taken (n >= 0): keeps the reservation referenced
}

// Coefficients by value (one launch per step).
template <int GDT, int PDT, bool WRITE_P>
__global__ __launch_bounds__(kEwThreads) void adam_update(float* __restrict__ P, float* __restrict__ M,
                                                          float* __restrict__ V, const void* __restrict__ G,
                                                          uint16_t* __restrict__ Pout, int64_t n, StepCoef c,
                                                          const double* __restrict__ d_sq,
                                                          const int32_t* __restrict__ d_ovf) {
    // Dynamic LDS reserved by the launcher only to cap how many of these
    // workgroups (one wave each) are resident per CU; it is never read.
    extern __shared__ float occupancy_pad[];
    adam_body<GDT, PDT, WRITE_P>(P, M, V, G, Pout, n, c, d_sq, d_ovf, occupancy_pad);
}

// Coefficients read from device memory at run time, so a captured graph can
// be replayed with the coefficients of each new step.
template <int GDT, int PDT, bool WRITE_P>
__global__ __launch_bounds__(kEwThreads) void adam_update_devcoef(float* __restrict__ P, float* __restrict__ M,
                                                                  float* __restrict__ V, const void* __restrict__ G,
                                                                  uint16_t* __restrict__ Pout, int64_t n,
                                                                  const StepCoef* __restrict__ pc,
                                                                  const double* __restrict__ d_sq,
                                                                  const int32_t* __restrict__ d_ovf) {
    extern __shared__ float occupancy_pad[];
    const StepCoef c = *pc;
    adam_body<GDT, PDT, WRITE_P>(P, M, V, G, Pout, n, c, d_sq, d_ovf, occupancy_pad);
}

// ---------------------------------------------------------------- gradient accumulation

// T consecutive tasks per one-wave workgroup, all loads issued before any
// math (straight-line code per task, as in the AdamW pass).
template <int DT, bool FIRST, int T>
__global__ __launch_bounds__(kEwThreads) void grad_accumulate(float* __restrict__ A, const void* __restrict__ G,
                                                              int64_t n, float inv,
                                                              const double* __restrict__ d_scale,
                                                              int32_t* __restrict__ d_ovf) {
    // dynamic LDS reserved by the launcher for the first micro-batch only, to
    // cap residency; never read
    extern __shared__ float occupancy_pad[];
    if (d_scale != nullptr) inv = (float)(1.0 / *d_scale);    // device-resident loss scale
    uint32_t bad = 0;
    const int lane = threadIdx.x;
    constexpr int64_t group = (int64_t)T * kEwTask;
    const int64_t ngroups = (n + group - 1) / group;
    for (int64_t t = blockIdx.x; t < ngroups; t += gridDim.x) {
        const int64_t base = t * group;
        if (base + group <= n) {
            u32x2 w[T];
            f32x4 a[T];
            static_for<T>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int64_t q = (base >> 2) + k * kEwThreads + lane;
                w[k] = ld_stream(static_cast<const u32x2*>(G) + q);
                if constexpr (!FIRST) a[k] = ld_stream(reinterpret_cast<f32x4*>(A) + q);
            });
            static_for<T>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int64_t q = (base >> 2) + k * kEwThreads + lane;
                bad |= (w[k][0] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                bad |= (w[k][1] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                float g[4];
                unpack2<DT>(w[k][0], g[0], g[1]);
                unpack2<DT>(w[k][1], g[2], g[3]);
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = FIRST ? g[j] * inv : fmaf(g[j], inv, a[k][j]);   // one rounding
                st_stream(o, reinterpret_cast<f32x4*>(A) + q);
            });
        } else {
            // the last, partial group: whole vectors, then the 1-3 element
            // ragged tail with scalar accesses
            for (int64_t e0 = base + 4 * lane; e0 < n; e0 += kEwTask) {
                if (e0 + 4 <= n) {
                    const int64_t q = e0 >> 2;
                    const u32x2 w = ld_stream(static_cast<const u32x2*>(G) + q);
                    bad |= (w[0] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                    bad |= (w[1] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                    float g[4];
                    unpack2<DT>(w[0], g[0], g[1]);
                    unpack2<DT>(w[1], g[2], g[3]);
                    f32x4* a4 = reinterpret_cast<f32x4*>(A) + q;
                    f32x4 a;
                    if constexpr (FIRST) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) a[k] = g[k] * inv;
                    } else {
                        a = ld_stream(a4);
#pragma unroll
                        for (int k = 0; k < 4; ++k) a[k] = fmaf(g[k], inv, a[k]);
                    }
                    st_stream(a, a4);
                } else {
                    for (int64_t e = e0; e < n; ++e) {
                        const uint32_t h = static_cast<const uint16_t*>(G)[e];
                        bad |= (h & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                        const float g = load_grad1<DT>(G, e);
                        A[e] = FIRST ? g * inv : fmaf(g, inv, A[e]);
                    }
                }
            }
        }
    }
    if (n < 0) occupancy_pad[lane] = 0.0f;   // never taken (n >= 0): keeps the reservation referenced
    if (d_ovf != nullptr && (bad & kNonfiniteBits) != 0) atomicOr(d_ovf, 1);
}

// ---------------------------------------------------------------- gradient reduction over ranks

// The K ranks' 16-bit gradients of this partition, summed in slice order into
// fp32 with one rounding per addition; the same operations, in the same
// order, as K passes of grad_accumulate (first on slice 0).
// Slice pointers passed by value; MAXK is the capacity compiled in.
template <int MAXK>
struct SlicesOf {
    const void* p[MAXK];
};

template <int DT, int MAXK>
__global__ __launch_bounds__(kEwThreads) void grad_reduce(float* __restrict__ A, SlicesOf<MAXK> sl, int k, int64_t n,
                                                          float inv, const double* __restrict__ d_scale,
                                                          int32_t* __restrict__ d_ovf) {
    // dynamic LDS reserved by the launcher for capacity 8 only, to cap
    // residency; never read
    extern __shared__ float occupancy_pad[];
    if (n < 0) occupancy_pad[threadIdx.x] = 0.0f;
    if (d_scale != nullptr) inv = (float)(1.0 / *d_scale);    // device-resident loss scale
    uint32_t bad = 0;
    const int lane = threadIdx.x;
    const int64_t ntasks = (n + kEwTask - 1) / kEwTask;
    for (int64_t t = blockIdx.x; t < ntasks; t += gridDim.x) {
        const int64_t e0 = t * kEwTask + 4 * lane;
        if (e0 + 4 <= n) {
            const int64_t q = e0 >> 2;
            u32x2 w[MAXK];
            // every slice's load in flight before any math (k is uniform)
#pragma unroll
            for (int r = 0; r < MAXK; ++r)
                if (r < k) w[r] = ld_stream(static_cast<const u32x2*>(sl.p[r]) + q);
            f32x4 a;
#pragma unroll
            for (int r = 0; r < MAXK; ++r) {
                if (r < k) {
                    bad |= (w[r][0] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                    bad |= (w[r][1] & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                    float g[4];
                    unpack2<DT>(w[r][0], g[0], g[1]);
                    unpack2<DT>(w[r][1], g[2], g[3]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[j] = r == 0 ? g[j] * inv : fmaf(g[j], inv, a[j]);
                }
            }
            st_stream(a, reinterpret_cast<f32x4*>(A) + q);
        } else if (e0 < n) {
            for (int64_t e = e0; e < n; ++e) {
                float a = 0.0f;
                for (int r = 0; r < k; ++r) {
                    const uint32_t h = static_cast<const uint16_t*>(sl.p[r])[e];
                    bad |= (h & GradFmt<DT>::mask) + GradFmt<DT>::carry;
                    const float g = load_grad1<DT>(sl.p[r], e);
                    a = r == 0 ? g * inv : fmaf(g, inv, a);
                }
                A[e] = a;
            }
        }
    }
    if (d_ovf != nullptr && (bad & kNonfiniteBits) != 0) atomicOr(d_ovf, 1);
}

// ---------------------------------------------------------------- wave sum through DPP

// v + (v moved by the DPP control CTRL within the rows in ROW_MASK; lanes with
// no source, or outside ROW_MASK, add 0), on both 32-bit halves of a double.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add(double v) {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    const int mlo = __builtin_amdgcn_update_dpp(0, lo, CTRL, ROW_MASK, 0xF, true);
    const int mhi = __builtin_amdgcn_update_dpp(0, hi, CTRL, ROW_MASK, 0xF, true);
    return v + __hiloint2double(mhi, mlo);
}

// Sum over the 64 lanes of a wave (all lanes active), in a fixed order, with
// VALU data movement only: shifts right by 1, 2, 4, 8 within each 16-lane row
// leave the row sums in lanes 15, 31, 47, 63; lane 15's row sum is broadcast
// into row 1 and lane 47's into row 3, then lane 31 into rows 2 and 3, so
// lane 63 holds the total, which every lane reads back.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
__device__ __forceinline__ double wave_sum(double v) {
    v = dpp_add<kDppRowShr1, 0xF>(v);
    v = dpp_add<kDppRowShr2, 0xF>(v);
    v = dpp_add<kDppRowShr4, 0xF>(v);
    v = dpp_add<kDppRowShr8, 0xF>(v);
    v = dpp_add<kDppRowBcast15, 0xA>(v);
    v = dpp_add<kDppRowBcast31, 0xC>(v);
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
    return __hiloint2double(hi, lo);
}

// ---------------------------------------------------------------- fp32 copy with its norm in the same pass

// acc = (ADD ? acc : 0) + sum_k slice_k * inv in slice order (the same
// operations as grad_accumulate / grad_reduce), and, per one-wave task, the
// fp64 sum of the squares of the 256 results it wrote: one partial per task
// in part_task (at task t's XCD-major slot, per_xcd slots per XCD), summed
// over the wave in a fixed order (wave_sum).  A
// non-finite result makes its partial non-finite (the square of a finite
// fp32 value, and any sum of up to 2^40 of them, stays finite in fp64), so
// the overflow flag is read off the partials.
template <int DT, bool ADD, int MAXK>
__global__ __launch_bounds__(kEwThreads) void grad_sum_norm(float* __restrict__ A, SlicesOf<MAXK> sl, int k, int64_t n,
                                                            float inv, const double* __restrict__ d_scale,
                                                            double* __restrict__ part_task, int64_t per_xcd) {
    // dynamic LDS reserved by the launcher for capacity 8 only, to cap
    // residency; never read
    extern __shared__ float occupancy_pad[];
    if (n < 0) occupancy_pad[threadIdx.x] = 0.0f;
    if (d_scale != nullptr) inv = (float)(1.0 / *d_scale);    // device-resident loss scale
    const int lane = threadIdx.x;
    const int64_t ntasks = (n + kEwTask - 1) / kEwTask;
    for (int64_t t = blockIdx.x; t < ntasks; t += gridDim.x) {
        double sq = 0.0;
        const int64_t e0 = t * kEwTask + 4 * lane;
        if (e0 + 4 <= n) {
            const int64_t q = e0 >> 2;
            u32x2 w[MAXK];
#pragma unroll
            for (int r = 0; r < MAXK; ++r)
                if (r < k) w[r] = ld_stream(static_cast<const u32x2*>(sl.p[r]) + q);
            f32x4 a;
            if constexpr (ADD) a = ld_stream(reinterpret_cast<const f32x4*>(A) + q);
#pragma unroll
            for (int r = 0; r < MAXK; ++r) {
                if (r < k) {
                    float g[4];
                    unpack2<DT>(w[r][0], g[0], g[1]);
                    unpack2<DT>(w[r][1], g[2], g[3]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) a[j] = (!ADD && r == 0) ? g[j] * inv : fmaf(g[j], inv, a[j]);
                }
            }
            st_stream(a, reinterpret_cast<f32x4*>(A) + q);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double x = (double)a[j];
                sq = fma(x, x, sq);
            }
        } else if (e0 < n) {
            for (int64_t e = e0; e < n; ++e) {
                float a = ADD ? A[e] : 0.0f;
                for (int r = 0; r < k; ++r) {
                    const float g = load_grad1<DT>(sl.p[r], e);
                    a = (!ADD && r == 0) ? g * inv : fmaf(g, inv, a);
                }
                A[e] = a;
                const double x = (double)a;
                sq = fma(x, x, sq);
            }
        }
        sq = wave_sum(sq);
        // a cached store into this XCD's run of slots: the 8-byte partials of
        // the tasks one XCD runs fill whole lines of its L2 before write-back
        if (lane == 0) part_task[(t % kXcds) * per_xcd + t / kXcds] = sq;
    }
}

// The task partials into at most kNormMaxBlocks block partials: block b sums
// its contiguous range of slots in a fixed order, skipping the slots no task
// maps to (the last slot of an XCD when kXcds does not divide ntasks); bad =
// any non-finite partial.
__global__ __launch_bounds__(kBlock) void task_partials_reduce(const double* __restrict__ part_task, int64_t ntasks,
                                                               int64_t per_xcd, int64_t per_block,
                                                               double* __restrict__ part_sq,
                                                               uint32_t* __restrict__ part_bad) {
    __shared__ double s_sq[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    const int64_t nslots = per_xcd * kXcds;
    const int64_t lo = (int64_t)blockIdx.x * per_block;
    const int64_t hi = lo + per_block < nslots ? lo + per_block : nslots;
    double acc = 0.0;
    uint32_t bad = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) {
        const int64_t xcd = i / per_xcd;
        if ((i - xcd * per_xcd) * kXcds + xcd >= ntasks) continue;     // no task writes this slot
        const double x = part_task[i];
        bad |= ((__double_as_longlong(x) >> 52) & 0x7FF) == 0x7FF ? 1u : 0u;
        acc += x;
    }
    block_reduce(acc, bad, s_sq, s_bad);
    if (threadIdx.x == 0) {
        part_sq[blockIdx.x] = acc;
        part_bad[blockIdx.x] = bad;
    }
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

int grad_bytes(int32_t dt) { return dt == ZERO_F32 ? 4 : 2; }

dim3 elementwise_grid(int64_t n, int64_t per_group = kEwTask) {
    int64_t ngroups = (n + per_group - 1) / per_group;
    if (ngroups > kEwMaxGrid) ngroups = kEwMaxGrid;   // the kernels stride over the rest
    return dim3((unsigned)ngroups);
}

template <int DT>
void launch_norm(int nb, hipStream_t s, const void* grad, int64_t n, double* part_sq, uint32_t* part_bad) {
    const int64_t nvec = n / GradFmt<DT>::per_vec;
    const int tail_n = (int)(n - nvec * GradFmt<DT>::per_vec);
    const void* tail = static_cast<const char*>(grad) + nvec * 16;
    hipLaunchKernelGGL(sqnorm_partials<DT>, dim3(nb), dim3(kBlock), 0, s, static_cast<const u32x4*>(grad), nvec,
                       tail, tail_n, part_sq, part_bad);
}

// d_coef == nullptr: coefficients c by value; otherwise read from d_coef on the device
template <int GDT, int PDT, bool WRITE_P>
void launch_adam(dim3 grid, hipStream_t s, float* P, float* M, float* V, const void* G, void* Pout,
                 int64_t n, const StepCoef& c, const StepCoef* d_coef, const double* d_sq, const int32_t* d_ovf) {
    if (d_coef == nullptr)
        hipLaunchKernelGGL((adam_update<GDT, PDT, WRITE_P>), grid, dim3(kEwThreads), kAdamLdsReserve, s, P, M, V,
                           G, static_cast<uint16_t*>(Pout), n, c, d_sq, d_ovf);
    else
        hipLaunchKernelGGL((adam_update_devcoef<GDT, PDT, WRITE_P>), grid, dim3(kEwThreads), kAdamLdsReserve, s,
                           P, M, V, G, static_cast<uint16_t*>(Pout), n, d_coef, d_sq, d_ovf);
}

template <int GDT>
void launch_adam_p(dim3 grid, hipStream_t s, bool wp, int pdt, float* P, float* M, float* V, const void* G,
                   void* Pout, int64_t n, const StepCoef& c, const StepCoef* d_coef, const double* d_sq,
                   const int32_t* d_ovf) {
    if (!wp) launch_adam<GDT, ZERO_F16, false>(grid, s, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
    else if (pdt == ZERO_F16) launch_adam<GDT, ZERO_F16, true>(grid, s, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
    else launch_adam<GDT, ZERO_BF16, true>(grid, s, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
}

void launch_adam_any(int32_t gdt, dim3 grid, hipStream_t s, bool wp, int pdt, float* P, float* M, float* V,
                     const void* G, void* Pout, int64_t n, const StepCoef& c, const StepCoef* d_coef,
                     const double* d_sq, const int32_t* d_ovf) {
    if (gdt == ZERO_F16) launch_adam_p<ZERO_F16>(grid, s, wp, pdt, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
    else if (gdt == ZERO_BF16) launch_adam_p<ZERO_BF16>(grid, s, wp, pdt, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
    else launch_adam_p<ZERO_F32>(grid, s, wp, pdt, P, M, V, G, Pout, n, c, d_coef, d_sq, d_ovf);
}

// argument checks shared by the AdamW entry points (coefficients aside)
int check_step_args(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, int32_t grad_dtype,
                    void* param_out, int32_t param_dtype, int64_t n, const double* d_sq, const int32_t* d_ovf) {
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (param_out != nullptr && param_dtype != ZERO_F16 && param_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "unknown param_dtype %d", param_dtype);
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad) return fail(ZERO_EINVAL, "NULL shard pointer");
    if (!aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(grad) ||
        (param_out && !aligned16(param_out)))
        return fail(ZERO_EALIGN, "shard pointers must be 16-byte aligned");
    if (d_sq && ((uintptr_t)d_sq & 7u)) return fail(ZERO_EALIGN, "d_global_sqnorm misaligned");
    if (d_ovf && ((uintptr_t)d_ovf & 3u)) return fail(ZERO_EALIGN, "d_global_overflow misaligned");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    const int64_t b32 = n * 4, b16 = n * 2, bg = n * grad_bytes(grad_dtype);
    if (overlaps(grad, bg, master, b32) || overlaps(grad, bg, exp_avg, b32) || overlaps(grad, bg, exp_avg_sq, b32) ||
        (param_out && overlaps(grad, bg, param_out, b16)))
        return fail(ZERO_EINVAL, "grad aliases an output");
    if (overlaps(master, b32, exp_avg, b32) || overlaps(master, b32, exp_avg_sq, b32) ||
        overlaps(exp_avg, b32, exp_avg_sq, b32) ||
        (param_out && (overlaps(param_out, b16, master, b32) || overlaps(param_out, b16, exp_avg, b32) ||
                       overlaps(param_out, b16, exp_avg_sq, b32))))
        return fail(ZERO_EINVAL, "state buffers overlap");
    // every workgroup reads the flag and the norm while others write the shard
    for (const auto& sc : {std::make_pair((const void*)d_sq, (int64_t)sizeof(double)),
                           std::make_pair((const void*)d_ovf, (int64_t)sizeof(int32_t))}) {
        if (sc.first == nullptr) continue;
        if (overlaps(sc.first, sc.second, master, b32) || overlaps(sc.first, sc.second, exp_avg, b32) ||
            overlaps(sc.first, sc.second, exp_avg_sq, b32) || (param_out && overlaps(sc.first, sc.second, param_out, b16)))
            return fail(ZERO_EINVAL, "d_global_sqnorm / d_global_overflow lies in a buffer the update writes");
    }
    return ZERO_OK;
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" {

size_t zero_norm_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    // one (double, uint32) partial per norm block; the block count depends on n only
    const size_t b = (size_t)norm_blocks(n);
    return ((b * (sizeof(double) + sizeof(uint32_t))) + 255) & ~(size_t)255;
}

}  // extern "C"

// The norm pass's block partials for zero_shard_unscale_norm_overflow_noalloc:
// a fixed array in device memory, one copy per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: host code only ever uses the address hipGetSymbolAddress returns for
// the current device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[8192];

namespace zero_shard {
namespace {

constexpr size_t kScratchBytes = sizeof(scratch);
static_assert(((kNormMaxBlocks * (sizeof(double) + sizeof(uint32_t))) + 255) / 256 * 256 <= kScratchBytes,
              "the norm pass's partials for any n fit the scratch array");

constexpr int kMaxScratchDevices = 256;
std::atomic<void*> g_scratch[kMaxScratchDevices];

// The device address of `scratch` on the current device, looked up on the
// first call on each device and kept.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ZERO_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(ZERO_ERANGE, "device %d beyond %d", dev, kMaxScratchDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(ZERO_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return ZERO_OK;
}

}  // namespace
}  // namespace zero_shard

namespace zero_shard {
namespace {

// The norm pass; the (1/scale)^2 factor is inv2 by value, or read from d_scale.
int norm_pass(const void* grad, int32_t grad_dtype, int64_t n, double inv2, const double* d_scale, double* d_sqnorm,
              int32_t* d_overflow, void* d_workspace, size_t workspace_bytes, hipStream_t s,
              zero_step_state* st_decide = nullptr, const HyperArgs& h = HyperArgs{}, StepCoef* coef = nullptr) {
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (d_sqnorm == nullptr || d_overflow == nullptr || d_workspace == nullptr)
        return fail(ZERO_EINVAL, "NULL output or workspace pointer");
    if (n > 0 && grad == nullptr) return fail(ZERO_EINVAL, "grad is NULL");
    if ((n > 0 && !aligned16(grad)) || !aligned16(d_workspace))
        return fail(ZERO_EALIGN, "grad and workspace must be 16-byte aligned");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u))
        return fail(ZERO_EALIGN, "d_sqnorm / d_overflow misaligned");
    const size_t need = zero_norm_workspace_bytes(n);
    if (workspace_bytes < need)
        return fail(ZERO_ENOSPC, "workspace %zu bytes, need %zu", workspace_bytes, need);
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    if ((n > 0 && overlaps(grad, n * (grad_dtype == ZERO_F32 ? 4 : 2), d_workspace, (int64_t)need)) ||
        overlaps(d_sqnorm, sizeof(double), d_workspace, (int64_t)need) ||
        overlaps(d_overflow, sizeof(int32_t), d_workspace, (int64_t)need) ||
        overlaps(d_sqnorm, sizeof(double), d_overflow, sizeof(int32_t)))
        return fail(ZERO_EINVAL, "workspace, d_sqnorm and d_overflow must not overlap each other or grad");
    const int nb = norm_blocks(n);
    double* part_sq = static_cast<double*>(d_workspace);
    uint32_t* part_bad = reinterpret_cast<uint32_t*>(part_sq + nb);
    if (n > 0) {
        if (grad_dtype == ZERO_F16) launch_norm<ZERO_F16>(nb, s, grad, n, part_sq, part_bad);
        else if (grad_dtype == ZERO_BF16) launch_norm<ZERO_BF16>(nb, s, grad, n, part_sq, part_bad);
        else launch_norm<ZERO_F32>(nb, s, grad, n, part_sq, part_bad);
        const int st = launch_status("sqnorm_partials");
        if (st != ZERO_OK) return st;
    }
    hipLaunchKernelGGL(sqnorm_finalize, dim3(1), dim3(kBlock), 0, s, part_sq, part_bad, n > 0 ? nb : 0, inv2, d_scale,
                       d_sqnorm, d_overflow, st_decide, h, grad_dtype == ZERO_F32 ? 1 : 0, coef);
    return launch_status("sqnorm_finalize");
}

int check_state(const zero_step_state* d_state) {
    if (d_state == nullptr) return fail(ZERO_EINVAL, "d_state is NULL");
    if ((uintptr_t)d_state & 7u) return fail(ZERO_EALIGN, "d_state must be 8-byte aligned");
    return ZERO_OK;
}

}  // namespace
}  // namespace zero_shard

extern "C" {

int zero_shard_unscale_norm_overflow(const void* grad, int32_t grad_dtype, int64_t n, double inv_loss_scale,
                                     double* d_sqnorm, int32_t* d_overflow, void* d_workspace,
                                     size_t workspace_bytes, void* hip_stream) {
    clear_error();
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    return norm_pass(grad, grad_dtype, n, inv_loss_scale * inv_loss_scale, nullptr, d_sqnorm, d_overflow,
                     d_workspace, workspace_bytes, static_cast<hipStream_t>(hip_stream));
}

int zero_shard_unscale_norm_overflow_noalloc(const void* grad, int32_t grad_dtype, int64_t n,
                                             double inv_loss_scale, double* d_sqnorm, int32_t* d_overflow,
                                             void* hip_stream) {
    clear_error();
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    // every argument is checked before the device is touched
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (d_sqnorm == nullptr || d_overflow == nullptr) return fail(ZERO_EINVAL, "NULL output pointer");
    if (n > 0 && grad == nullptr) return fail(ZERO_EINVAL, "grad is NULL");
    if (n > 0 && !aligned16(grad)) return fail(ZERO_EALIGN, "grad must be 16-byte aligned");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u))
        return fail(ZERO_EALIGN, "d_sqnorm / d_overflow misaligned");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    const size_t need = zero_norm_workspace_bytes(n);
    if (need > kScratchBytes)
        return fail(ZERO_ENOSPC, "the norm pass needs %zu bytes of scratch, the fixed array holds %zu", need,
                    kScratchBytes);
    void* ws = nullptr;
    const int st = scratch_address(&ws);
    if (st != ZERO_OK) return st;
    // the partials kernel writes every slot the combine reads: nothing to clear
    return norm_pass(grad, grad_dtype, n, inv_loss_scale * inv_loss_scale, nullptr, d_sqnorm, d_overflow, ws,
                     kScratchBytes, static_cast<hipStream_t>(hip_stream));
}

int zero_shard_unscale_norm_overflow_dev(const void* grad, int32_t grad_dtype, int64_t n,
                                         const zero_step_state* d_state, double* d_sqnorm, int32_t* d_overflow,
                                         void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    clear_error();
    const int st = check_state(d_state);
    if (st != ZERO_OK) return st;
    // an fp32 gradient is the accumulation or reduction copy, already unscaled
    const double* d_scale = grad_dtype == ZERO_F32 ? nullptr : &d_state->scaler.scale;
    return norm_pass(grad, grad_dtype, n, 1.0, d_scale, d_sqnorm, d_overflow, d_workspace, workspace_bytes,
                     static_cast<hipStream_t>(hip_stream));
}

int zero_shard_adam_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, int32_t grad_dtype,
                         void* param_out, int32_t param_dtype, int64_t n, const zero_adam_params* hp,
                         const double* d_global_sqnorm, const int32_t* d_global_overflow, void* hip_stream) {
    clear_error();
    StepCoef c;
    const int pst = prepare_adam(hp, &c);
    if (pst != ZERO_OK) return pst;
    if (c.clip && d_global_sqnorm == nullptr) return fail(ZERO_EINVAL, "clipping needs d_global_sqnorm");
    const int st = check_step_args(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n,
                                   d_global_sqnorm, d_global_overflow);
    if (st != ZERO_OK || n == 0) return st;
    launch_adam_any(grad_dtype, elementwise_grid(n, kAdamGroup), static_cast<hipStream_t>(hip_stream), param_out != nullptr,
                    param_dtype, master, exp_avg, exp_avg_sq, grad, param_out, n, c, nullptr, d_global_sqnorm,
                    d_global_overflow);
    return launch_status("adam_update");
}

size_t zero_adam_coef_bytes(void) { return sizeof(StepCoef); }

int zero_adam_prepare(const zero_adam_params* hp, void* coef_out) {
    clear_error();
    if (coef_out == nullptr) return fail(ZERO_EINVAL, "coef_out is NULL");
    StepCoef c;
    const int pst = prepare_adam(hp, &c);
    if (pst != ZERO_OK) return pst;
    std::memcpy(coef_out, &c, sizeof(c));
    return ZERO_OK;
}

int zero_shard_adam_step_coef(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                              int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                              const void* d_coef, const double* d_global_sqnorm,
                              const int32_t* d_global_overflow, void* hip_stream) {
    clear_error();
    if (d_coef == nullptr || ((uintptr_t)d_coef & 7u)) return fail(ZERO_EINVAL, "d_coef NULL or not 8-byte aligned");
    if (d_global_sqnorm == nullptr) return fail(ZERO_EINVAL, "d_global_sqnorm is required");
    const int st = check_step_args(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n,
                                   d_global_sqnorm, d_global_overflow);
    if (st != ZERO_OK || n == 0) return st;
    const StepCoef unused{};
    launch_adam_any(grad_dtype, elementwise_grid(n, kAdamGroup), static_cast<hipStream_t>(hip_stream), param_out != nullptr,
                    param_dtype, master, exp_avg, exp_avg_sq, grad, param_out, n, unused,
                    static_cast<const StepCoef*>(d_coef), d_global_sqnorm, d_global_overflow);
    return launch_status("adam_update_devcoef");
}

int zero_shard_norm_decide_dev(const void* grad, int32_t grad_dtype, int64_t n, const zero_adam_hyper* hp,
                               zero_step_state* d_state, double* d_sqnorm, int32_t* d_overflow, void* d_coef,
                               void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    clear_error();
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    int st = check_hyper(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm);
    if (st != ZERO_OK) return st;
    st = check_state(d_state);
    if (st != ZERO_OK) return st;
    if (d_coef == nullptr || ((uintptr_t)d_coef & 7u)) return fail(ZERO_EINVAL, "d_coef NULL or not 8-byte aligned");
    const HyperArgs h{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm};
    const double* d_scale = grad_dtype == ZERO_F32 ? nullptr : &d_state->scaler.scale;
    return norm_pass(grad, grad_dtype, n, 1.0, d_scale, d_sqnorm, d_overflow, d_workspace, workspace_bytes,
                     static_cast<hipStream_t>(hip_stream), d_state, h, static_cast<StepCoef*>(d_coef));
}

int zero_step_decide_dev(const zero_adam_hyper* hp, int32_t grad_dtype, zero_step_state* d_state,
                         const int32_t* d_global_overflow, void* d_coef, void* hip_stream) {
    clear_error();
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    int st = check_hyper(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm);
    if (st != ZERO_OK) return st;
    st = check_state(d_state);
    if (st != ZERO_OK) return st;
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32)
        return fail(ZERO_EINVAL, "unknown grad_dtype %d", grad_dtype);
    if (d_global_overflow == nullptr || ((uintptr_t)d_global_overflow & 3u))
        return fail(ZERO_EINVAL, "d_global_overflow NULL or misaligned");
    if (d_coef == nullptr || ((uintptr_t)d_coef & 7u)) return fail(ZERO_EINVAL, "d_coef NULL or not 8-byte aligned");
    const HyperArgs h{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm};
    hipLaunchKernelGGL(step_decide, dim3(1), dim3(64), 0, static_cast<hipStream_t>(hip_stream), d_state,
                       d_global_overflow, h, grad_dtype == ZERO_F32 ? 1 : 0, static_cast<StepCoef*>(d_coef));
    return launch_status("step_decide");
}

int zero_shard_adam_step_dev(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, int32_t grad_dtype,
                             void* param_out, int32_t param_dtype, int64_t n, const zero_adam_hyper* hp,
                             zero_step_state* d_state, const double* d_global_sqnorm,
                             const int32_t* d_global_overflow, void* d_coef, void* hip_stream) {
    clear_error();
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    if (d_global_sqnorm == nullptr && hp->max_grad_norm > 0.0) return fail(ZERO_EINVAL, "clipping needs d_global_sqnorm");
    // everything is checked before anything is enqueued
    int st = check_step_args(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n, d_global_sqnorm,
                             d_global_overflow);
    if (st != ZERO_OK) return st;
    // the decision and the state update run even for an empty shard: every rank advances together
    st = zero_step_decide_dev(hp, grad_dtype, d_state, d_global_overflow, d_coef, hip_stream);
    if (st != ZERO_OK || n == 0) return st;
    const StepCoef unused{};
    launch_adam_any(grad_dtype, elementwise_grid(n, kAdamGroup), static_cast<hipStream_t>(hip_stream),
                    param_out != nullptr, param_dtype, master, exp_avg, exp_avg_sq, grad, param_out, n, unused,
                    static_cast<const StepCoef*>(d_coef), d_global_sqnorm, d_global_overflow);
    return launch_status("adam_update_devcoef");
}

}  // extern "C"

namespace zero_shard {
namespace {

// The slice-taking kernels are compiled for slice capacities 1, 2, 4, 8 and 16
// and launched with the smallest one that holds n_slices: each pointer held
// costs two scalar registers, and at capacity 16 their count limits
// occupancy to 7 waves per SIMD (8 below).
template <int MAXK>
SlicesOf<MAXK> first_slices(const SlicesOf<ZERO_MAX_SLICES>& sl) {
    SlicesOf<MAXK> r{};
    for (int i = 0; i < MAXK; ++i) r.p[i] = sl.p[i];
    return r;
}

template <int DT, bool ADD>
void launch_sum_norm(dim3 grid, hipStream_t s, float* acc, const SlicesOf<ZERO_MAX_SLICES>& sl, int32_t k, int64_t n,
                     float inv, const double* d_scale, double* part_task, int64_t per_xcd) {
#define ZS_SUM(M) hipLaunchKernelGGL((grad_sum_norm<DT, ADD, M>), grid, dim3(kEwThreads), (M) == 8 ? kSlices8Lds : 0, s, acc, \
                                     first_slices<M>(sl), (int)k, n, inv, d_scale, part_task, per_xcd)
    if (k <= 1) ZS_SUM(1);
    else if (k <= 2) ZS_SUM(2);
    else if (k <= 4) ZS_SUM(4);
    else if (k <= 8) ZS_SUM(8);
    else ZS_SUM(16);
#undef ZS_SUM
}

template <int DT>
void launch_reduce(dim3 grid, hipStream_t s, float* acc, const SlicesOf<ZERO_MAX_SLICES>& sl, int32_t k, int64_t n,
                   float inv, const double* d_scale, int32_t* d_overflow) {
#define ZS_RED(M) hipLaunchKernelGGL((grad_reduce<DT, M>), grid, dim3(kEwThreads), (M) == 8 ? kSlices8Lds : 0, s, acc, first_slices<M>(sl), \
                                     (int)k, n, inv, d_scale, d_overflow)
    if (k <= 1) ZS_RED(1);
    else if (k <= 2) ZS_RED(2);
    else if (k <= 4) ZS_RED(4);
    else if (k <= 8) ZS_RED(8);
    else ZS_RED(16);
#undef ZS_RED
}

int accumulate(float* acc, const void* grad, int32_t grad_dtype, int64_t n, double inv_loss_scale,
               const double* d_scale, int32_t first, int32_t* d_overflow, hipStream_t s) {
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "grad_dtype must be ZERO_F16 or ZERO_BF16 (got %d)", grad_dtype);
    if (n == 0) return ZERO_OK;
    if (acc == nullptr || grad == nullptr) return fail(ZERO_EINVAL, "NULL acc or grad");
    if (!aligned16(acc) || !aligned16(grad)) return fail(ZERO_EALIGN, "acc and grad must be 16-byte aligned");
    if (d_overflow && ((uintptr_t)d_overflow & 3u)) return fail(ZERO_EALIGN, "d_overflow misaligned");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    if (overlaps(acc, n * 4, grad, n * 2)) return fail(ZERO_EINVAL, "acc aliases grad");
    if (d_overflow && overlaps(acc, n * 4, d_overflow, sizeof(int32_t))) return fail(ZERO_EINVAL, "d_overflow lies in acc");
    const float inv = (float)inv_loss_scale;
    // the first micro-batch: kAccFirstTasks tasks per workgroup, capped
    // residency; later ones: one task per uncapped workgroup
    const dim3 grid = elementwise_grid(n, first ? (int64_t)kAccFirstTasks * kEwTask : kEwTask);
#define ZS_ACC(DT)                                                                                             \
    do {                                                                                                       \
        if (first)                                                                                             \
            hipLaunchKernelGGL((grad_accumulate<DT, true, kAccFirstTasks>), grid, dim3(kEwThreads),            \
                               kAccFirstLds, s, acc, grad, n, inv, d_scale, d_overflow);                       \
        else                                                                                                   \
            hipLaunchKernelGGL((grad_accumulate<DT, false, 1>), grid, dim3(kEwThreads), 0, s, acc, grad, n,    \
                               inv, d_scale, d_overflow);                                                      \
    } while (0)
    if (grad_dtype == ZERO_F16) ZS_ACC(ZERO_F16);
    else ZS_ACC(ZERO_BF16);
#undef ZS_ACC
    return launch_status("grad_accumulate");
}

int reduce(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype, int64_t n,
           double inv_loss_scale, const double* d_scale, int32_t* d_overflow, hipStream_t s) {
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (n_slices < 1 || n_slices > ZERO_MAX_SLICES)
        return fail(ZERO_EINVAL, "n_slices must lie in [1, %d] (got %d)", ZERO_MAX_SLICES, n_slices);
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "grad_dtype must be ZERO_F16 or ZERO_BF16 (got %d)", grad_dtype);
    if (n == 0) return ZERO_OK;
    if (acc == nullptr || slices == nullptr) return fail(ZERO_EINVAL, "NULL acc or slices");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    if (!aligned16(acc)) return fail(ZERO_EALIGN, "acc must be 16-byte aligned");
    if (d_overflow && ((uintptr_t)d_overflow & 3u)) return fail(ZERO_EALIGN, "d_overflow misaligned");
    SlicesOf<ZERO_MAX_SLICES> sl{};
    for (int32_t r = 0; r < n_slices; ++r) {
        if (slices[r] == nullptr) return fail(ZERO_EINVAL, "slice %d is NULL", r);
        if (!aligned16(slices[r])) return fail(ZERO_EALIGN, "slice %d must be 16-byte aligned", r);
        if (overlaps(acc, n * 4, slices[r], n * 2)) return fail(ZERO_EINVAL, "acc aliases slice %d", r);
        sl.p[r] = slices[r];
    }
    if (d_overflow && overlaps(acc, n * 4, d_overflow, sizeof(int32_t))) return fail(ZERO_EINVAL, "d_overflow lies in acc");
    const dim3 grid = elementwise_grid(n);
    const float inv = (float)inv_loss_scale;
    if (grad_dtype == ZERO_F16) launch_reduce<ZERO_F16>(grid, s, acc, sl, n_slices, n, inv, d_scale, d_overflow);
    else launch_reduce<ZERO_BF16>(grid, s, acc, sl, n_slices, n, inv, d_scale, d_overflow);
    return launch_status("grad_reduce");
}

// Layout of the fused pass's workspace: kXcds * per_xcd task slots (one
// double per task, XCD-major), then the block partials of the norm pass
// (double, uint32).
struct SumNormLayout {
    int64_t ntasks;
    int64_t per_xcd;
    int nb;
    int64_t per_block;
    size_t bytes;
};

SumNormLayout sum_norm_layout(int64_t n) {
    SumNormLayout l;
    l.ntasks = (n + kEwTask - 1) / kEwTask;
    l.per_xcd = (l.ntasks + kXcds - 1) / kXcds;
    const int64_t nslots = l.per_xcd * kXcds;
    int64_t nb = l.ntasks / 1024;
    if (nb < 1) nb = 1;
    if (nb > kNormMaxBlocks) nb = kNormMaxBlocks;
    l.nb = (int)nb;
    l.per_block = (nslots + nb - 1) / nb;
    const size_t raw = (size_t)(nslots + nb) * sizeof(double) + (size_t)nb * sizeof(uint32_t);
    l.bytes = (raw + 255) & ~(size_t)255;
    return l;
}

int sum_norm(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype, int64_t n, int32_t add,
             double inv_loss_scale, const double* d_scale, double* d_sqnorm, int32_t* d_overflow, void* d_workspace,
             size_t workspace_bytes, hipStream_t s, zero_step_state* st_decide, const HyperArgs& h, StepCoef* coef) {
    if (n < 0) return fail(ZERO_EINVAL, "n < 0");
    if (n_slices < 1 || n_slices > ZERO_MAX_SLICES)
        return fail(ZERO_EINVAL, "n_slices must lie in [1, %d] (got %d)", ZERO_MAX_SLICES, n_slices);
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16)
        return fail(ZERO_EINVAL, "grad_dtype must be ZERO_F16 or ZERO_BF16 (got %d)", grad_dtype);
    if (d_sqnorm == nullptr || d_overflow == nullptr || d_workspace == nullptr)
        return fail(ZERO_EINVAL, "NULL norm output or workspace");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u) || !aligned16(d_workspace))
        return fail(ZERO_EALIGN, "norm outputs or workspace misaligned");
    if (n > INT64_MAX / 4) return fail(ZERO_ERANGE, "n too large");
    const SumNormLayout l = sum_norm_layout(n);
    if (workspace_bytes < l.bytes) return fail(ZERO_ENOSPC, "workspace %zu bytes, need %zu", workspace_bytes, l.bytes);
    const int64_t wsb = (int64_t)l.bytes;
    if (overlaps(d_sqnorm, sizeof(double), d_workspace, wsb) || overlaps(d_overflow, sizeof(int32_t), d_workspace, wsb) ||
        overlaps(d_sqnorm, sizeof(double), d_overflow, sizeof(int32_t)))
        return fail(ZERO_EINVAL, "workspace, d_sqnorm and d_overflow must not overlap");
    SlicesOf<ZERO_MAX_SLICES> sl{};
    if (n > 0) {
        if (acc == nullptr || slices == nullptr) return fail(ZERO_EINVAL, "NULL acc or slices");
        if (!aligned16(acc)) return fail(ZERO_EALIGN, "acc must be 16-byte aligned");
        if (overlaps(acc, n * 4, d_workspace, wsb)) return fail(ZERO_EINVAL, "acc aliases workspace");
        if (overlaps(acc, n * 4, d_sqnorm, sizeof(double)) || overlaps(acc, n * 4, d_overflow, sizeof(int32_t)))
            return fail(ZERO_EINVAL, "d_sqnorm / d_overflow lies in acc");
        for (int32_t r = 0; r < n_slices; ++r) {
            if (slices[r] == nullptr) return fail(ZERO_EINVAL, "slice %d is NULL", r);
            if (!aligned16(slices[r])) return fail(ZERO_EALIGN, "slice %d must be 16-byte aligned", r);
            if (overlaps(acc, n * 4, slices[r], n * 2)) return fail(ZERO_EINVAL, "acc aliases slice %d", r);
            if (overlaps(slices[r], n * 2, d_workspace, wsb)) return fail(ZERO_EINVAL, "slice %d aliases workspace", r);
            sl.p[r] = slices[r];
        }
    }
    double* part_task = static_cast<double*>(d_workspace);
    double* part_sq = part_task + l.per_xcd * kXcds;
    uint32_t* part_bad = reinterpret_cast<uint32_t*>(part_sq + l.nb);
    int nparts = 0;
    if (n > 0) {
        const dim3 grid = elementwise_grid(n);
        const float inv = (float)inv_loss_scale;
        if (grad_dtype == ZERO_F16) {
            if (add) launch_sum_norm<ZERO_F16, true>(grid, s, acc, sl, n_slices, n, inv, d_scale, part_task, l.per_xcd);
            else launch_sum_norm<ZERO_F16, false>(grid, s, acc, sl, n_slices, n, inv, d_scale, part_task, l.per_xcd);
        } else {
            if (add) launch_sum_norm<ZERO_BF16, true>(grid, s, acc, sl, n_slices, n, inv, d_scale, part_task, l.per_xcd);
            else launch_sum_norm<ZERO_BF16, false>(grid, s, acc, sl, n_slices, n, inv, d_scale, part_task, l.per_xcd);
        }
        int st = launch_status("grad_sum_norm");
        if (st != ZERO_OK) return st;
        hipLaunchKernelGGL(task_partials_reduce, dim3(l.nb), dim3(kBlock), 0, s, part_task, l.ntasks, l.per_xcd,
                           l.per_block, part_sq, part_bad);
        st = launch_status("task_partials_reduce");
        if (st != ZERO_OK) return st;
        nparts = l.nb;
    }
    // the copy is already unscaled: the factor on the sum of squares is 1
    hipLaunchKernelGGL(sqnorm_finalize, dim3(1), dim3(kBlock), 0, s, part_sq, part_bad, nparts, 1.0, nullptr, d_sqnorm,
                       d_overflow, st_decide, h, 1, coef);
    return launch_status("sqnorm_finalize");
}

}  // namespace
}  // namespace zero_shard

extern "C" {

int zero_shard_grad_accumulate(float* acc, const void* grad, int32_t grad_dtype, int64_t n, double inv_loss_scale,
                               int32_t first, int32_t* d_overflow, void* hip_stream) {
    clear_error();
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    return accumulate(acc, grad, grad_dtype, n, inv_loss_scale, nullptr, first, d_overflow,
                      static_cast<hipStream_t>(hip_stream));
}

int zero_shard_grad_accumulate_dev(float* acc, const void* grad, int32_t grad_dtype, int64_t n,
                                   const zero_step_state* d_state, int32_t first, int32_t* d_overflow,
                                   void* hip_stream) {
    clear_error();
    const int st = check_state(d_state);
    if (st != ZERO_OK) return st;
    return accumulate(acc, grad, grad_dtype, n, 1.0, &d_state->scaler.scale, first, d_overflow,
                      static_cast<hipStream_t>(hip_stream));
}

int zero_shard_grad_reduce(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype, int64_t n,
                           double inv_loss_scale, int32_t* d_overflow, void* hip_stream) {
    clear_error();
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    return reduce(acc, slices, n_slices, grad_dtype, n, inv_loss_scale, nullptr, d_overflow,
                  static_cast<hipStream_t>(hip_stream));
}

int zero_shard_grad_reduce_dev(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                               int64_t n, const zero_step_state* d_state, int32_t* d_overflow, void* hip_stream) {
    clear_error();
    const int st = check_state(d_state);
    if (st != ZERO_OK) return st;
    return reduce(acc, slices, n_slices, grad_dtype, n, 1.0, &d_state->scaler.scale, d_overflow,
                  static_cast<hipStream_t>(hip_stream));
}

size_t zero_sum_norm_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    return sum_norm_layout(n).bytes;
}

int zero_shard_grad_sum_norm(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype, int64_t n,
                             int32_t add_to_acc, double inv_loss_scale, double* d_sqnorm, int32_t* d_overflow,
                             void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    clear_error();
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    return sum_norm(acc, slices, n_slices, grad_dtype, n, add_to_acc, inv_loss_scale, nullptr, d_sqnorm, d_overflow,
                    d_workspace, workspace_bytes, static_cast<hipStream_t>(hip_stream), nullptr, HyperArgs{}, nullptr);
}

int zero_shard_grad_sum_norm_dev(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                                 int64_t n, int32_t add_to_acc, const zero_adam_hyper* hp, zero_step_state* d_state,
                                 double* d_sqnorm, int32_t* d_overflow, void* d_coef, void* d_workspace,
                                 size_t workspace_bytes, void* hip_stream) {
    clear_error();
    int st = check_state(d_state);
    if (st != ZERO_OK) return st;
    HyperArgs h{};
    if (hp != nullptr) {
        st = check_hyper(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm);
        if (st != ZERO_OK) return st;
        if (d_coef == nullptr || ((uintptr_t)d_coef & 7u))
            return fail(ZERO_EINVAL, "d_coef NULL or not 8-byte aligned");
        h = HyperArgs{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm};
    }
    return sum_norm(acc, slices, n_slices, grad_dtype, n, add_to_acc, 1.0, &d_state->scaler.scale, d_sqnorm,
                    d_overflow, d_workspace, workspace_bytes, static_cast<hipStream_t>(hip_stream),
                    hp != nullptr ? d_state : nullptr, h, static_cast<StepCoef*>(d_coef));
}

// ---------------------------------------------------------------- step graphs

struct zero_step_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;       // recorded after every launch
    StepCoef* h_coef = nullptr;      // pinned host: the next step's coefficients
    int32_t* h_flag = nullptr;       // pinned host: the last step's overflow flag
    StepCoef* d_coef = nullptr;      // device copy read by the update kernel
    double inv_loss_scale = 1.0;
    bool launched = false;
    bool device_state = false;       // recorded by zero_step_graph_create_dev: no host blocks
};

static void release_graph(zero_step_graph* g) {
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    if (g->done) (void)hipEventDestroy(g->done);
    if (g->h_coef) (void)hipHostFree(g->h_coef);
    if (g->h_flag) (void)hipHostFree(g->h_flag);
    if (g->d_coef) (void)hipFree(g->d_coef);
    delete g;
}

int zero_step_graph_create(zero_step_graph** out, float* master, float* exp_avg, float* exp_avg_sq,
                           const void* grad, int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                           double inv_loss_scale, double* d_sqnorm, int32_t* d_overflow, void* d_workspace,
                           size_t workspace_bytes) {
    clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "out is NULL");
    *out = nullptr;
    if (!(inv_loss_scale > 0.0) || !std::isfinite(inv_loss_scale))
        return fail(ZERO_EINVAL, "inv_loss_scale must be finite and > 0");
    if (d_sqnorm == nullptr || d_overflow == nullptr || d_workspace == nullptr)
        return fail(ZERO_EINVAL, "NULL norm output or workspace");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u) || !aligned16(d_workspace))
        return fail(ZERO_EALIGN, "norm outputs or workspace misaligned");
    if (workspace_bytes < zero_norm_workspace_bytes(n)) return fail(ZERO_ENOSPC, "workspace too small");
    int st = check_step_args(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n, d_sqnorm,
                             d_overflow);
    if (st != ZERO_OK) return st;
    zero_step_graph* g = new zero_step_graph();
    g->inv_loss_scale = inv_loss_scale;
    hipStream_t cs = nullptr;
    hipError_t e = hipHostMalloc((void**)&g->h_coef, sizeof(StepCoef), hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&g->h_flag, sizeof(int32_t), hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void**)&g->d_coef, sizeof(StepCoef));
    if (e == hipSuccess) e = hipEventCreateWithFlags(&g->done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreate(&cs);
    if (e != hipSuccess) {
        if (cs) (void)hipStreamDestroy(cs);
        release_graph(g);
        return fail(ZERO_EHIP, "step graph resources: %s", hipGetErrorString(e));
    }
    std::memset(g->h_coef, 0, sizeof(StepCoef));
    *g->h_flag = 0;
    // record: coefficients in, norm pass, fused update, flag out
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        e = hipMemcpyAsync(g->d_coef, g->h_coef, sizeof(StepCoef), hipMemcpyHostToDevice, cs);
        if (e == hipSuccess)
            st = zero_shard_unscale_norm_overflow(grad, grad_dtype, n, inv_loss_scale, d_sqnorm, d_overflow,
                                                  d_workspace, workspace_bytes, cs);
        if (e == hipSuccess && st == ZERO_OK)
            st = zero_shard_adam_step_coef(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n,
                                           g->d_coef, d_sqnorm, d_overflow, cs);
        if (e == hipSuccess && st == ZERO_OK)
            e = hipMemcpyAsync(g->h_flag, d_overflow, sizeof(int32_t), hipMemcpyDeviceToHost, cs);
        const hipError_t e2 = hipStreamEndCapture(cs, &g->graph);
        if (e == hipSuccess) e = e2;
    }
    if (e == hipSuccess && st == ZERO_OK) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cs);
    if (e != hipSuccess || st != ZERO_OK) {
        release_graph(g);
        if (st != ZERO_OK) return st;
        return fail(ZERO_EHIP, "step graph capture: %s", hipGetErrorString(e));
    }
    *out = g;
    return ZERO_OK;
}

int zero_step_graph_launch(zero_step_graph* g, const zero_adam_params* hp, void* hip_stream) {
    clear_error();
    if (g == nullptr) return fail(ZERO_EINVAL, "graph is NULL");
    if (g->device_state) return fail(ZERO_EINVAL, "graph recorded with device state: use zero_step_graph_launch_dev");
    StepCoef c;
    const int pst = prepare_adam(hp, &c);
    if (pst != ZERO_OK) return pst;
    if (hp->inv_loss_scale != g->inv_loss_scale)
        return fail(ZERO_EINVAL, "inv_loss_scale differs from the one the graph was recorded with");
    // the previous replay may still be reading the pinned coefficient block
    if (g->launched) {
        const hipError_t e = hipEventSynchronize(g->done);
        if (e != hipSuccess) return fail(ZERO_EHIP, "waiting for the previous replay: %s", hipGetErrorString(e));
    }
    std::memcpy(g->h_coef, &c, sizeof(c));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipGraphLaunch(g->exec, s);
    if (e == hipSuccess) e = hipEventRecord(g->done, s);
    if (e != hipSuccess) return fail(ZERO_EHIP, "graph launch: %s", hipGetErrorString(e));
    g->launched = true;
    return ZERO_OK;
}

int zero_step_graph_overflow(zero_step_graph* g, int32_t* overflow) {
    clear_error();
    if (g == nullptr || overflow == nullptr) return fail(ZERO_EINVAL, "NULL argument");
    if (g->device_state) return fail(ZERO_EINVAL, "graph recorded with device state: read the state instead");
    if (!g->launched) return fail(ZERO_EINVAL, "graph not launched yet");
    const hipError_t e = hipEventSynchronize(g->done);
    if (e != hipSuccess) return fail(ZERO_EHIP, "waiting for the replay: %s", hipGetErrorString(e));
    *overflow = *g->h_flag != 0 ? 1 : 0;
    return ZERO_OK;
}

int zero_step_graph_create_dev(zero_step_graph** out, float* master, float* exp_avg, float* exp_avg_sq,
                               const void* grad, int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                               const zero_adam_hyper* hp, zero_step_state* d_state, double* d_sqnorm,
                               int32_t* d_overflow, void* d_coef, void* d_workspace, size_t workspace_bytes) {
    clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "out is NULL");
    *out = nullptr;
    if (hp == nullptr) return fail(ZERO_EINVAL, "hp is NULL");
    int st = check_hyper(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm);
    if (st != ZERO_OK) return st;
    st = check_state(d_state);
    if (st != ZERO_OK) return st;
    if (d_coef == nullptr || ((uintptr_t)d_coef & 7u)) return fail(ZERO_EINVAL, "d_coef NULL or not 8-byte aligned");
    if (d_sqnorm == nullptr || d_overflow == nullptr || d_workspace == nullptr)
        return fail(ZERO_EINVAL, "NULL norm output or workspace");
    if (((uintptr_t)d_sqnorm & 7u) || ((uintptr_t)d_overflow & 3u) || !aligned16(d_workspace))
        return fail(ZERO_EALIGN, "norm outputs or workspace misaligned");
    if (workspace_bytes < zero_norm_workspace_bytes(n)) return fail(ZERO_ENOSPC, "workspace too small");
    st = check_step_args(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n, d_sqnorm,
                         d_overflow);
    if (st != ZERO_OK) return st;
    zero_step_graph* g = new zero_step_graph();
    g->device_state = true;
    hipStream_t cs = nullptr;
    hipError_t e = hipEventCreateWithFlags(&g->done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreate(&cs);
    if (e != hipSuccess) {
        if (cs) (void)hipStreamDestroy(cs);
        release_graph(g);
        return fail(ZERO_EHIP, "step graph resources: %s", hipGetErrorString(e));
    }
    // record: the norm pass with the decision in its last kernel, then the update
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        st = zero_shard_norm_decide_dev(grad, grad_dtype, n, hp, d_state, d_sqnorm, d_overflow, d_coef, d_workspace,
                                        workspace_bytes, cs);
        if (st == ZERO_OK)
            st = zero_shard_adam_step_coef(master, exp_avg, exp_avg_sq, grad, grad_dtype, param_out, param_dtype, n,
                                           d_coef, d_sqnorm, d_overflow, cs);
        e = hipStreamEndCapture(cs, &g->graph);
    }
    if (e == hipSuccess && st == ZERO_OK) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cs);
    if (e != hipSuccess || st != ZERO_OK) {
        release_graph(g);
        if (st != ZERO_OK) return st;
        return fail(ZERO_EHIP, "step graph capture: %s", hipGetErrorString(e));
    }
    *out = g;
    return ZERO_OK;
}

int zero_step_graph_launch_dev(zero_step_graph* g, void* hip_stream) {
    clear_error();
    if (g == nullptr) return fail(ZERO_EINVAL, "graph is NULL");
    if (!g->device_state) return fail(ZERO_EINVAL, "graph recorded with host coefficients: use zero_step_graph_launch");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipGraphLaunch(g->exec, s);
    if (e == hipSuccess) e = hipEventRecord(g->done, s);      // lets destroy wait for the last replay
    if (e != hipSuccess) return fail(ZERO_EHIP, "graph launch: %s", hipGetErrorString(e));
    g->launched = true;
    return ZERO_OK;
}

int zero_step_graph_destroy(zero_step_graph* g) {
    clear_error();
    if (g == nullptr) return ZERO_OK;
    if (g->launched && g->done != nullptr) (void)hipEventSynchronize(g->done);
    release_graph(g);
    return ZERO_OK;
}

}  // extern "C"
