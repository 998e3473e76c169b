// The local half of the all-reduce of the norm pass's two scalars.
//
// Each rank updates only its own partition (ZeRO method entry, description;
// explainer "Data Parallelism Without the Copies", Ch.02 "The Three Stages",
// what each stage shards), yet the clip coefficient and the skip depend on
// the gradient of the whole model: the ranks' sums of squares are added and
// their inf/NaN flags OR-ed.  With a direct exchange every rank writes its
// (sum of squares, flag) into slot r of two small arrays on every peer; once
// the slots have landed, each rank runs this kernel, which adds the slots in
// rank order in fp64 and ORs the flags, so every rank obtains the same bits
// whatever order the slots arrived in.
//
// One workgroup: the slots are staged through LDS 1024 at a time and one
// thread adds them in order (a sequential sum, the order a host loop over
// ranks would use); the flags are OR-ed by every thread.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "zero_shard.h"

namespace zero_shard {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kCombineStage = 1024;

__global__ __launch_bounds__(kCombineThreads) void combine_ranks(const double* __restrict__ slot_sq,
                                                                 const int32_t* __restrict__ slot_ovf, int n_ranks,
                                                                 double* __restrict__ d_sq,
                                                                 int32_t* __restrict__ d_ovf) {
    __shared__ double s_sq[kCombineStage];
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    double total = 0.0;
    int bad = 0;
    for (int base = 0; base < n_ranks; base += kCombineStage) {
        const int m = n_ranks - base < kCombineStage ? n_ranks - base : kCombineStage;
        __syncthreads();                                    // the previous stage has been added
        for (int i = threadIdx.x; i < m; i += kCombineThreads) {
            s_sq[i] = slot_sq[base + i];
            bad |= slot_ovf[base + i] != 0;
        }
        __syncthreads();
        if (threadIdx.x == 0)
            for (int i = 0; i < m; ++i) total += s_sq[i];
    }
    if (bad) atomicOr(&s_bad, 1);                           // LDS
    __syncthreads();
    if (threadIdx.x == 0) {
        *d_sq = total;
        *d_ovf = s_bad;
    }
}

bool spans_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" int zero_norm_combine_ranks(const double* slot_sqnorm, const int32_t* slot_overflow, int32_t n_ranks,
                                       double* d_global_sqnorm, int32_t* d_global_overflow, void* hip_stream) {
    clear_error();
    if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
        return fail(ZERO_EINVAL, "n_ranks must lie in [1, %d] (got %d)", ZERO_MAX_RANKS, n_ranks);
    if (!slot_sqnorm || !slot_overflow || !d_global_sqnorm || !d_global_overflow)
        return fail(ZERO_EINVAL, "NULL pointer");
    if (((uintptr_t)slot_sqnorm & 7u) || ((uintptr_t)d_global_sqnorm & 7u) || ((uintptr_t)slot_overflow & 3u) ||
        ((uintptr_t)d_global_overflow & 3u))
        return fail(ZERO_EALIGN, "sums of squares must be 8-byte and flags 4-byte aligned");
    const int64_t bsq = (int64_t)n_ranks * 8, bov = (int64_t)n_ranks * 4;
    if (spans_overlap(slot_sqnorm, bsq, slot_overflow, bov) ||
        spans_overlap(d_global_sqnorm, 8, slot_sqnorm, bsq) || spans_overlap(d_global_sqnorm, 8, slot_overflow, bov) ||
        spans_overlap(d_global_overflow, 4, slot_sqnorm, bsq) || spans_overlap(d_global_overflow, 4, slot_overflow, bov) ||
        spans_overlap(d_global_sqnorm, 8, d_global_overflow, 4))
        return fail(ZERO_EINVAL, "slot arrays and outputs must not overlap");
    hipLaunchKernelGGL(combine_ranks, dim3(1), dim3(kCombineThreads), 0, static_cast<hipStream_t>(hip_stream),
                       slot_sqnorm, slot_overflow, (int)n_ranks, d_global_sqnorm, d_global_overflow);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "combine_ranks launch: %s", hipGetErrorString(e));
    return ZERO_OK;
}
