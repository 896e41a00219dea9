// pfs_noalloc.hip -- pfs_verify_noalloc: the verify step for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). The split partials live in a
// file-scope device array of fixed size instead of a caller workspace; the
// kernels are the ones pfs_verify launches.
//
// Each GPU the library runs on holds its own copy of the array (module
// memory, kept until the process ends). The call uses the copy of the GPU
// that runs its stream; that copy's device address is taken once per device
// with hipGetSymbolAddress while that device is current; host code
// only ever passes that address, never the array's name (on the host the name
// is a stand-in, not a device address). The verify workspace needs no
// initialization (every partial the combine reads is written earlier in the
// same call), so nothing is cleared between calls. Calls that overlap on one
// GPU (different streams, or host threads without stream order) share the
// array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "pfs_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[pfs::kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the copy of `scratch` on the GPU that runs `stream` (the
// current device for the NULL stream); nullptr on error. The first call for
// a device looks the address up with that device current, then restores the
// caller's current device.
void* device_scratch(hipStream_t stream, int* status) {
    int dev = -1;
    const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = PFS_ERR_LAUNCH;
        return nullptr;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) {
            *status = PFS_ERR_LAUNCH;
            return nullptr;
        }
        void* addr = nullptr;
        const hipError_t found = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) {
            *status = PFS_ERR_LAUNCH;
            return nullptr;
        }
        if (found != hipSuccess || !addr) {
            *status = PFS_ERR_LAUNCH;
            return nullptr;
        }
        g_scratch[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}

}  // namespace

extern "C" {

int64_t pfs_noalloc_scratch_bytes(void) { return pfs::kNoallocScratchBytes; }

int32_t pfs_verify_noalloc(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool, const uint8_t* v_pool,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           const int32_t* live_len, void* out_fp16, pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    if (plan->ws_bytes > pfs::kNoallocScratchBytes) return PFS_ERR_WORKSPACE;
    if (!q_fp16 || !k_pool || !v_pool || !k_scale || !v_scale || !block_table || !live_len || !out_fp16)
        return PFS_ERR_NULL;  // before any HIP call
    int32_t st = PFS_OK;
    void* ws = device_scratch(reinterpret_cast<hipStream_t>(stream), &st);
    if (!ws) return st;
    return pfs_verify(plan, q_fp16, k_pool, v_pool, k_scale, v_scale, block_table, live_len, out_fp16, ws,
                      pfs::kNoallocScratchBytes, stream);
}

}  // extern "C"
