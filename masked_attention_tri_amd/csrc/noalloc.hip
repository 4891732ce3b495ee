// tri_attn_bwd_noalloc: the backward for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It is tri_attn_bwd with its workspace (the per-row data)
// taken from a fixed device array of this library instead of from the
// caller: nothing is allocated or freed, and nothing but the kernels of
// tri_attn_bwd runs.
//
// The array (`scratch`) lives in every GPU that loads the library until the
// process ends.  Its address differs per device, so it is resolved with
// hipGetSymbolAddress on the first call on each device (that device
// current) and cached; host code never passes the symbol itself to a
// kernel.  Calls on one GPU share the array: calls that overlap in time on
// one GPU race (each stores its per-row data there and reads it back).
// Nothing in it needs clearing: a call's first pass writes every entry its
// later passes read.
#include <atomic>
#include <mutex>

#include "triattn_internal.h"

namespace {

// The workspace: TRIATTN_BWD_NOALLOC_BYTES (48 MiB).
constexpr int64_t kScratchFloats = TRIATTN_BWD_NOALLOC_BYTES / 4;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// This device's copy of `scratch`, or nullptr (with the HIP error) if its
// address cannot be obtained.
float* device_scratch(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    float* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        void* addr = nullptr;
        *err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        ptr = static_cast<float*>(addr);
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" {

triattn_status tri_attn_bwd_noalloc(const tri_attn_shape* shape, int32_t dtype, const void* q,
                                    const void* k, const void* v, const float* bias,
                                    const tri_attn_mask* mask, float scale, const void* out,
                                    const void* dout, const float* lse, const float* max,
                                    void* dq, void* dk, void* dv, float* dbias,
                                    hipStream_t stream) {
    // Everything tri_attn_bwd validates but the workspace, then the
    // scratch's capacity; nothing touches the device first.
    const triattn_status st =
        triattn::bwd_validate(shape, dtype, q, k, v, bias, mask, scale, out, dout, lse, max, dq,
                              dk, dv, dbias, nullptr, 0, false);
    if (st != TRIATTN_OK) return st;
    if (shape->B == 0 || shape->N == 0 || shape->H == 0 || shape->Q == 0) return TRIATTN_OK;
    // the per-row data must fit the scratch
    const int64_t slices = shape->B * shape->N * shape->H;  // validated: no overflow
    const int64_t need = triattn::bwd_rows_bytes(slices, shape->Q);
    if (need < 0 || need > TRIATTN_BWD_NOALLOC_BYTES) return TRIATTN_ERR_UNSUPPORTED;
    hipError_t err = hipSuccess;
    float* ws = device_scratch(&err);
    if (!ws) return TRIATTN_ERR_HIP;
    return tri_attn_bwd(shape, dtype, q, k, v, bias, mask, scale, out, dout, lse, max, dq, dk,
                        dv, dbias, ws, static_cast<size_t>(kScratchFloats) * sizeof(float), stream);
}

}  // extern "C"
