// Physically contiguous HBM for a shard's streams.
//
// The fused AdamW pass keeps eight streams in flight (four reads, four
// writes).  Its rate depends on where the streams' pages land in HBM: with
// buffers from the default allocator it varied between processes on one
// MI355X from 75% to 82% of the 8 TB/s peak (16 processes: mean 79.5%,
// standard deviation 1.6 points), while the same buffers allocated
// physically contiguous ran at 78.8-83.5% (mean 81.6%, standard deviation
// 1.2 points).  The two-stream copy kernel shows no such spread.  These calls
// provide that memory; the step's calls themselves still allocate nothing.
//
// zero_pool_alloc / zero_pool_free have the signatures of a PyTorch
// pluggable allocator, so a torch memory pool can serve tensors from it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

#include "common.h"
#include "zero_shard.h"

using namespace zero_shard;

namespace {

// What zero_pool_alloc has handed out since the library was loaded: segments
// that are physically contiguous, and segments that fell back to ordinary
// device memory.  Read by zero_pool_counts, so a caller can tell which kind
// its tensors got.
std::atomic<int64_t> g_pool_contiguous{0};
std::atomic<int64_t> g_pool_fallback{0};

// Allocates on `device` (the current device if device < 0), restoring the
// caller's current device.
hipError_t alloc_on(void** ptr, size_t bytes, int device, bool contiguous) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    const bool switch_dev = device >= 0 && device != cur;
    if (switch_dev && (e = hipSetDevice(device)) != hipSuccess) return e;
    e = contiguous ? hipExtMallocWithFlags(ptr, bytes, hipDeviceMallocContiguous) : hipMalloc(ptr, bytes);
    if (switch_dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess && e2 != hipSuccess) {
            (void)hipFree(*ptr);
            *ptr = nullptr;
            e = e2;
        }
    }
    return e;
}

}  // namespace

extern "C" {

int zero_device_alloc_contiguous(void** ptr, size_t bytes) {
    clear_error();
    if (ptr == nullptr) return fail(ZERO_EINVAL, "ptr is NULL");
    *ptr = nullptr;
    if (bytes == 0) return ZERO_OK;
    const hipError_t e = alloc_on(ptr, bytes, -1, true);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *ptr = nullptr;
        return fail(ZERO_EHIP, "contiguous allocation of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    return ZERO_OK;
}

int zero_device_free(void* ptr) {
    clear_error();
    if (ptr == nullptr) return ZERO_OK;
    const hipError_t e = hipFree(ptr);
    if (e != hipSuccess) return fail(ZERO_EHIP, "hipFree: %s", hipGetErrorString(e));
    return ZERO_OK;
}

void* zero_pool_alloc(size_t bytes, int device, void* stream) {
    (void)stream;
    if (bytes == 0) return nullptr;
    void* p = nullptr;
    if (alloc_on(&p, bytes, device, true) == hipSuccess) {
        g_pool_contiguous.fetch_add(1, std::memory_order_relaxed);
        return p;
    }
    // no contiguous range of that size left: ordinary device memory
    (void)hipGetLastError();
    p = nullptr;
    if (alloc_on(&p, bytes, device, false) == hipSuccess) {
        g_pool_fallback.fetch_add(1, std::memory_order_relaxed);
        return p;
    }
    (void)hipGetLastError();
    return nullptr;
}

int zero_pool_counts(int64_t* contiguous, int64_t* fallback) {
    clear_error();
    if (contiguous == nullptr || fallback == nullptr) return fail(ZERO_EINVAL, "output pointer is NULL");
    *contiguous = g_pool_contiguous.load(std::memory_order_relaxed);
    *fallback = g_pool_fallback.load(std::memory_order_relaxed);
    return ZERO_OK;
}

void zero_pool_free(void* ptr, size_t bytes, int device, void* stream) {
    (void)bytes;
    (void)device;
    (void)stream;
    if (ptr != nullptr) (void)hipFree(ptr);
}

}  // extern "C"
