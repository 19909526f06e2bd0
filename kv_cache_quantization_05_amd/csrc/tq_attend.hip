// Decode attention dispatch: query prep, partial kernels, merge.
#include <atomic>

#include "tq_attend_v1.h"
#include "tq_internal.h"

namespace tq {

// The general launchers are instantiated in tq_attend_dims.hip, one object
// file per head dimension.
namespace v1 {
#define TQ_EXTERN_DIM(D)                                                                                  \
    extern template hipError_t launch_attend_d<D>(const dev_tables &, const dev_tables &, const attend_args &, \
                                                  hipStream_t);                                         \
    extern template hipError_t launch_prep_d<D>(const dev_tables &, const float *, int64_t, float *, int64_t, \
                                                hipStream_t);
TQ_EXTERN_DIM(32)
TQ_EXTERN_DIM(64)
TQ_EXTERN_DIM(128)
TQ_EXTERN_DIM(256)
#undef TQ_EXTERN_DIM
}  // namespace v1

// Compute units of the current device, queried once per device.
int current_cu_count() {
    static std::atomic<int> counts[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev >= 64) {
        hipDeviceProp_t prop;
        return hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
    }
    int n = counts[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        hipDeviceProp_t prop;
        n = hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
        counts[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tokens per split-K chunk.  Each (batch, KV head, chunk) is one block; the
// chunk is a multiple of 256 tokens chosen so that the number of blocks fills
// whole rounds of the resident block slots (no half-empty last round),
// preferring the fewest rounds (fewest partial states) that reach 90%.
int attend_chunk_tokens(const dev_tables & kt, const dev_tables & vt, int32_t B, int32_t Hq, int32_t Hkv,
                        int64_t t_max) {
    if (t_max <= 0 || B <= 0 || Hkv <= 0) return 256;
    const int cu_count = current_cu_count();
    const bool mfma = attend_mfma_shape_ok(kt, vt, Hq, Hkv);
    const int64_t slots = int64_t(cu_count) * (mfma ? attend_mfma_blocks_per_cu(kt, vt) : 2);
    const int64_t base = int64_t(B) * Hkv;
    int64_t best_chunk = 0;
    double best_eff = -1.0;
    for (int r = 1; r <= 32; ++r) {
        const int64_t per_bg = (r * slots + base - 1) / base;
        int64_t chunk = (t_max + per_bg - 1) / per_bg;
        chunk = (chunk + 255) / 256 * 256;
        const int64_t blocks = base * ((t_max + chunk - 1) / chunk);
        const double eff = double(blocks) / double(((blocks + slots - 1) / slots) * slots);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best_chunk = chunk;
        }
        if (eff >= 0.9 || chunk <= 256) break;
    }
    return static_cast<int>(best_chunk);
}

hipError_t launch_query_prep(const dev_tables & t, const float * q, int64_t n, float * qp,
                             int64_t qp_stride, hipStream_t s) {
    if (n == 0) return hipSuccess;
    switch (t.d) {
        case 32: return v1::launch_prep_d<32>(t, q, n, qp, qp_stride, s);
        case 64: return v1::launch_prep_d<64>(t, q, n, qp, qp_stride, s);
        case 128: return v1::launch_prep_d<128>(t, q, n, qp, qp_stride, s);
        case 256: return v1::launch_prep_d<256>(t, q, n, qp, qp_stride, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attend(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                         hipStream_t s) {
    switch (kt.d) {
        case 32: return v1::launch_attend_d<32>(kt, vt, a, s);
        case 64: return v1::launch_attend_d<64>(kt, vt, a, s);
        case 128: return v1::launch_attend_d<128>(kt, vt, a, s);
        case 256: return v1::launch_attend_d<256>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
