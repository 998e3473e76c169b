// Reference device copy: the achievable streaming rate of one read stream
// plus one write stream on this GPU, against which the step's kernels are
// reported next to the nominal HBM peak.  It is a measurement aid, not a step
// of the method.
//
// Each lane moves one 16-byte vector; a wave's load and store instructions
// each cover one contiguous 1 KiB run.  One-shot grid of 256-thread
// workgroups in address order; non-temporal hints on both sides, as in the
// step's kernels.  A launch holds fewer than 2^32 work-items, so a copy past
// 2^24 - 1 workgroups' worth (just under 64 GiB) takes further turns of a
// grid-stride loop.
//
// The widening copy reads 8 bytes and writes 16 per lane (each 8-byte word
// twice), one-wave workgroups: the access pattern of the first micro-batch's
// gradient accumulation (2 bytes read, 4 written per element), whose
// achievable rate it measures.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"
#include "zero_shard.h"

namespace zero_shard {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kCopyThreads = 256;
// grid * kCopyThreads stays below 2^32 work-items per dispatch
constexpr int64_t kCopyMaxGrid = (int64_t(1) << 24) - 1;

__global__ __launch_bounds__(kCopyThreads) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       int64_t nvec) {
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
    for (int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < nvec; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kWidenThreads = 64;
constexpr int64_t kWidenMaxGrid = (int64_t(1) << 26) - 1;   // grid * 64 work-items < 2^32

__global__ __launch_bounds__(kWidenThreads) void copy8to16(const u32x2* __restrict__ src, u32x4* __restrict__ dst,
                                                           int64_t nwords) {
    const int64_t stride = (int64_t)gridDim.x * kWidenThreads;
    for (int64_t i = (int64_t)blockIdx.x * kWidenThreads + threadIdx.x; i < nwords; i += stride) {
        const u32x2 v = __builtin_nontemporal_load(src + i);
        const u32x4 o = {v[0], v[1], v[0], v[1]};
        __builtin_nontemporal_store(o, dst + i);
    }
}

}  // namespace
}  // namespace zero_shard

using namespace zero_shard;

extern "C" int zero_copy_reference(void* dst, const void* src, int64_t bytes, void* hip_stream) {
    clear_error();
    if (bytes < 0 || (bytes & 15)) return fail(ZERO_EINVAL, "bytes must be a non-negative multiple of 16");
    if (bytes == 0) return ZERO_OK;
    if (dst == nullptr || src == nullptr) return fail(ZERO_EINVAL, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u)
        return fail(ZERO_EALIGN, "dst and src must be 16-byte aligned");
    const int64_t nvec = bytes / 16;
    const int64_t grid = std::min<int64_t>((nvec + kCopyThreads - 1) / kCopyThreads, kCopyMaxGrid);
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) return fail(ZERO_EINVAL, "dst and src overlap");
    hipLaunchKernelGGL(copy16, dim3((unsigned)grid), dim3(kCopyThreads), 0, static_cast<hipStream_t>(hip_stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "copy16 launch: %s", hipGetErrorString(e));
    return ZERO_OK;
}

extern "C" int zero_copy_widen_reference(void* dst, const void* src, int64_t src_bytes, void* hip_stream) {
    clear_error();
    if (src_bytes < 0 || (src_bytes & 7)) return fail(ZERO_EINVAL, "src_bytes must be a non-negative multiple of 8");
    if (src_bytes == 0) return ZERO_OK;
    if (dst == nullptr || src == nullptr) return fail(ZERO_EINVAL, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u)
        return fail(ZERO_EALIGN, "dst and src must be 16-byte aligned");
    if (src_bytes > INT64_MAX / 2) return fail(ZERO_ERANGE, "src_bytes too large");
    const int64_t nwords = src_bytes / 8;
    const int64_t grid = std::min<int64_t>((nwords + kWidenThreads - 1) / kWidenThreads, kWidenMaxGrid);
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (d < s + (uintptr_t)src_bytes && s < d + 2 * (uintptr_t)src_bytes)
        return fail(ZERO_EINVAL, "dst and src overlap");
    hipLaunchKernelGGL(copy8to16, dim3((unsigned)grid), dim3(kWidenThreads), 0, static_cast<hipStream_t>(hip_stream),
                       static_cast<const u32x2*>(src), static_cast<u32x4*>(dst), nwords);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "copy8to16 launch: %s", hipGetErrorString(e));
    return ZERO_OK;
}
