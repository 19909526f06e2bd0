// tq_attend_decode_static: decode attention with no allocation in the call.
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it), the split-K workspace of
// tq_attend_decode (prepared queries and per-chunk partial states) lives in
// a file-scope device array instead of a caller buffer.  Each GPU holds its
// own copy of the array until the process ends; its device address is
// looked up once per device (hipGetSymbolAddress) and only that address is
// ever handed to kernels.  The array keeps the last call's contents; the
// kernels write every entry they read (the merge reads only partial states
// written by the same call), so nothing needs clearing between calls.
#include <atomic>
#include <mutex>

#include "tq_internal.h"

namespace {

constexpr int64_t kScratchBytes = TQ_ATTEND_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (device must be current).
hipError_t scratch_for_device(int dev, void ** out) {
    void * p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" int32_t tq_attend_decode_static(const tq_ctx * k_ctx, const tq_ctx * v_ctx, const float * q,
                                           tq_planes k, tq_planes v, const int32_t * seq_lens, int32_t B,
                                           int32_t Hq, int32_t Hkv, int64_t t_max, float scale, float * out,
                                           void * hip_stream) {
    if (!k_ctx || !v_ctx) return tq::set_error(TQ_STATUS_INVALID_ARG, "k_ctx and v_ctx must be non-NULL");
    const int64_t need = tq_attend_decode_workspace(k_ctx, v_ctx, B, Hq, Hkv, t_max);
    if (need < 0) return tq::set_error(TQ_STATUS_INVALID_ARG, "invalid sizes");
    if (need > kScratchBytes)
        return tq::set_error(TQ_STATUS_UNSUPPORTED,
                             "tq_attend_decode_static: these sizes need %lld bytes of workspace, more than "
                             "its static %lld-byte buffer; use tq_attend_decode with a caller workspace",
                             (long long)need, (long long)kScratchBytes);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return tq::set_error(TQ_STATUS_DEVICE, "no usable current HIP device");
    if (dev != tq::ctx_device(k_ctx))
        return tq::set_error(TQ_STATUS_INVALID_ARG, "the current device is not the contexts' device");
    void * ws = nullptr;
    hipError_t e = scratch_for_device(dev, &ws);
    if (e != hipSuccess)
        return tq::set_error(TQ_STATUS_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    return tq_attend_decode(k_ctx, v_ctx, q, k, v, seq_lens, B, Hq, Hkv, t_max, scale, out, ws, kScratchBytes,
                            hip_stream);
}
