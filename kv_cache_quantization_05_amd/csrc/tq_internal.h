// Internal declarations shared by the host code and the kernel translation
// units of libtq.  Nothing here is part of the public ABI (include/tq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

// Size of the device array behind tq_attend_decode_static (16 MiB: the
// benchmark layers need about 1.2 MB).
#define TQ_ATTEND_STATIC_SCRATCH_BYTES (int64_t(16) << 20)

namespace tq {

constexpr int kMaxDim = 256;

// Records the thread-local error text and returns `status` (tq_host.cpp).
int32_t set_error(int32_t status, const char * fmt, ...) __attribute__((format(printf, 2, 3)));
// Device a ctx is bound to.
int ctx_device(const tq_ctx * ctx);

// Small per-config tables passed to kernels by value (kernel arguments).
// Sign masks: bit i of word i/32 set means the diagonal entry is -1.
struct dev_tables {
    uint32_t d1[kMaxDim / 32];
    uint32_t d2[kMaxDim / 32];
    float cb[16];        // codebook, ascending; entries >= 2^b unused
    float th[16];        // 2^b - 1 thresholds; th[2^b - 1 ..] = +inf
    const float * S;     // device, m x d row-major (QJL only)
    const uint16_t * S16;  // device, fp16 split of S: hi [m x d] then lo [m x d]
    const float * Q;     // device, d x d row-major dense rotation (Haar only), y = Q x
    const uint16_t * Q16;  // device, fp16 split of 16 Q: hi [d x d] then lo [d x d]
    int32_t d;
    int32_t bits;
    int32_t m;
    int32_t qjl;
    int32_t haar;        // rotation is the dense Q (else D1.H.D2)
    int32_t norm_group;  // 0: one norm per vector; 32: one per 32-code block
    int32_t norm_corr;   // stored norms carry the norm correction
};

// Norms per vector in the norms plane.
inline int norms_per_vector(const dev_tables & t) { return t.norm_group ? t.d / t.norm_group : 1; }

// Host-side table generation (tq_tables.cpp); independent of any device.
int build_tables(const tq_config & cfg, int8_t * d1, int8_t * d2, float * codebook,
                 float * thresholds, float * s_rowmajor);
int validate_config(const tq_config & cfg, const char ** why);
// Dense rotation R (d x d row-major float64): y = R x.
void build_rotation(const tq_config & cfg, double * r);
// hi = fp16(v), lo = fp16(v - hi), both round-to-nearest-even (v ~ hi + lo
// to ~2^-22 relative).
void split_fp16(const float * v, int64_t n, uint16_t * hi, uint16_t * lo);

// Launchers (kernel translation units).  Return hipError_t of the launch.
struct encode_args {
    const void * x;
    int32_t dtype;
    int64_t n0, n1, n2;
    int64_t xs0, xs1, xs2;      // element strides
    tq_planes out;
};
hipError_t launch_encode(const dev_tables & t, const encode_args & a, hipStream_t s);
// Haar rotation, block norms or norm correction (tq_encode_var.hip).
hipError_t launch_encode_variant(const dev_tables & t, const encode_args & a, hipStream_t s);
bool encode_grid_supported(const encode_args & a);  // n0*n1*n2 < 2^32
// QJL keys, bf16 input, d = 64 or 128: matrix-core rotation and sketch
// (tq_encode_qjl.hip).
bool encode_qjl_mfma_supported(const dev_tables & t, const encode_args & a);
hipError_t launch_encode_qjl_mfma(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s);

// Query preparation: qp[i] = [ R q_i (d floats) | S R q_i (m floats, qjl) ].
hipError_t launch_query_prep(const dev_tables & t, const float * q, int64_t n, float * qp,
                             int64_t qp_stride, hipStream_t s);

struct attend_args {
    const float * q;            // queries [B*Hq, d] as given
    float * qp;                 // prepared queries [B*Hq, qp_stride] (workspace)
    int64_t qp_stride;
    tq_planes k, v;
    const int32_t * seq_lens;
    int32_t B, Hq, Hkv;
    int64_t t_max;
    int32_t chunk;              // tokens per split-K chunk
    int32_t n_chunks;
    float scale;
    float * partial;            // [B*Hq, n_chunks, d + 2]
    float * out;
};
hipError_t launch_attend(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                         hipStream_t s);
// Matrix-core partial kernel for d = 128 with 4 query heads per KV head.
bool attend_mfma_supported(const dev_tables & kt, const dev_tables & vt, const attend_args & a);
bool attend_mfma_shape_ok(const dev_tables & kt, const dev_tables & vt, int32_t Hq, int32_t Hkv);
int attend_mfma_blocks_per_cu(const dev_tables & kt, const dev_tables & vt);
hipError_t launch_attend_mfma_partial(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                                      hipStream_t s);
// Compute units of the current device (queried once per device).
int current_cu_count();
int attend_chunk_tokens(const dev_tables & kt, const dev_tables & vt, int32_t B, int32_t Hq, int32_t Hkv,
                        int64_t t_max);

struct prefill_args {
    const float * q;            // queries [B*Hq*Tq, d] as given
    float * qp;                 // prepared queries [B*Hq*Tq, qp_stride] (workspace)
    int64_t qp_stride;
    tq_planes k, v;
    const int32_t * seq_lens;   // lengths including the Tq new positions
    int32_t B, Hq, Hkv;
    int64_t Tq;
    int64_t t_max;
    float scale;
    float * out_rot;            // rotated-domain outputs [B*Hq*Tq, d] (workspace)
    float * out;                // [B*Hq*Tq, d]
};
bool prefill_supported(const dev_tables & kt, const dev_tables & vt);
hipError_t launch_prefill(const dev_tables & kt, const dev_tables & vt, const prefill_args & a, hipStream_t s);

struct scores_args {
    const float * qp;
    int64_t qp_stride;
    int64_t n_q;
    tq_planes k;
    int64_t n_k;
    float scale;
    int32_t top_k;
    float * out_scores;
    int64_t * out_idx;
    float * cand_s;             // top-k candidates [n_ranges, n_q, top_k]
    int64_t * cand_i;
    int32_t n_ranges;
    int64_t keys_per_range;     // keys of one range (a multiple of 16 on the matrix-core path)
};
hipError_t launch_scores(const dev_tables & t, const scores_args & a, hipStream_t s);
// Split of the keys into ranges (one top-k list per query each) for head_dim d.
void scores_plan(int d, bool block_norms, int64_t n_q, int64_t n_k, int32_t top_k, int32_t & ranges,
                 int64_t & keys_per_range);
// 32 x 32-tile scorer (tq_scores32.hip): d = 128 or 256, one norm per vector,
// top_k <= 16; one wave per range, scores_tile32_waves() ranges per block.
bool scores_tile32_supported(int d, bool block_norms, int32_t top_k);
int scores_tile32_waves();
hipError_t launch_scores_tile32(const dev_tables & t, const scores_args & a, hipStream_t s);

}  // namespace tq
