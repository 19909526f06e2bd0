/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache encode and decode attention on
 * AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [TQ+ guide]    "TurboQuant+ 上游化实战指南：llama.cpp KV Cache 压缩分支的 4 阶段
 *                   PR 重构路线图"
 *   [Orión plan]   "Plan de Integración: TurboQuant en Orión"
 *   [TQ explainer] "Google TurboQuant 深度解析：KV Cache 压缩的技术革命"
 *
 * Conventions (taken from the public-API rules in [TQ+ guide] §2.4 and §9):
 * fixed-width integers, enum values prefixed with the enum name, snake_case
 * <class>_<action>_<noun> names, no typedef'd structs.
 *
 * Memory: every device buffer (inputs, outputs, workspaces) is allocated and
 * owned by the caller.  A tq_ctx owns only its small device tables.  No entry
 * point allocates device memory except tq_ctx_create.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a
 * failed check returns a non-zero tq_status and leaves the stream untouched.
 * tq_last_error() then describes it (thread-local).  A failed kernel launch
 * returns TQ_STATUS_DEVICE.  Faults inside a kernel surface at the caller's next
 * synchronisation.  NaN/Inf inputs are not checked; their outputs are
 * undefined.  No C++ exception crosses this interface.
 *
 * Streams: `hip_stream` is a hipStream_t (NULL = the default stream).  All
 * device work is asynchronous on it.  A ctx is immutable after creation, so
 * calls on several streams or threads may share one.
 *
 * Packed layout (the "planes"): vector v of a plane set occupies
 *   codes  + v * code_bytes   d*b/8 bytes: code i at bits b*i..b*i+b-1 of an
 *                             LSB-first bit stream (bit k is bit k%8 of byte
 *                             k/8); a 32-code block is 4*b bytes
 *   norms  + v * nn           fp16 bits of the norms (rounded once, RNE):
 *                             nn = 1 (||x||_2) or d/32 (block norms of R x)
 *   signs  + v * sign_bytes   QJL: m sign bits, bit l = bit l%8 of byte l/8
 *                             ([Orión plan] Fase 3, sign-bit sketch)
 *   rnorms + v                QJL: fp16 bits of the residual norm gamma
 * A plane set addresses a 3-D grid of vectors [n0, n1, n2]; vector (i0,i1,i2)
 * is v = i0*stride[0] + i1*stride[1] + i2*stride[2].  codes rows must be
 * 4-byte aligned (d*b/8 is a multiple of 4 for d >= 32).
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tq_status {
    TQ_STATUS_OK = 0,
    TQ_STATUS_INVALID_ARG = 1,
    TQ_STATUS_UNSUPPORTED = 2,
    TQ_STATUS_DEVICE = 3,
    TQ_STATUS_NO_MEMORY = 4,
};

enum tq_dtype {
    TQ_DTYPE_F32 = 0,
    TQ_DTYPE_BF16 = 1,
};

/* Rotation applied before quantisation ([TQ+ guide] §3, §4: the fast
 * structured D1.H.D2 rotation and the dense rotation from a seeded QR). */
enum tq_rotation {
    TQ_ROTATION_WHT = 0,   /* R = D1.H.D2 / sqrt(d), O(d log d) */
    TQ_ROTATION_HAAR = 1,  /* R = Q of a seeded Gaussian's QR, det +1, O(d^2) */
};

/*
 * Method configuration ([TQ+ guide] §5.1-§5.2: MSE-only codebook, block size
 * 32, rotation width decoupled from block size; [Orión plan] Fase 2 settings
 * block: separate key and value bit widths -> one config per K and per V).
 *   seed      seeds the rotation signs D1, D2 and the QJL matrix S
 *             ([TQ+ guide] §3: rotation generated from a seed, same seed ->
 *             same matrix)
 *   head_dim  d: 32, 64, 128 or 256
 *   bits      b: 2, 3 or 4 bits per coordinate
 *   block     32 (codes per packed block)
 *   qjl       1 adds the 1-bit QJL residual sketch ([TQ explainer] §2.2)
 *   qjl_dim   m, rows of S: 0 means m = d (the kernels support only m = d;
 *             another multiple of 32 up to 256 gives TQ_STATUS_UNSUPPORTED)
 *   rotation  enum tq_rotation.  TQ_ROTATION_HAAR: R = Q with G = Q R' the
 *             Householder QR of a d x d Gaussian G drawn from the seed (a
 *             third SplitMix64 stream, seed ^ 0x4841415200000000, Box-Muller
 *             pairs rounded to float, row-major), Q's columns multiplied by
 *             the signs of diag(R'), and column 0 negated if det(Q) = -1
 *             ([TQ+ guide] §3, the seeded QR rotation with det = +1)
 *   norm_group 0: one fp16 norm per vector (the norm of x); 32: one fp16 norm
 *             per 32-code block, the norm of that block of the rotated vector
 *             R x, with z = sqrt(32) (R x)_block / norm_block (the 3.5-bit
 *             turbo3 layout of [TQ+ guide] §1.2)
 *   norm_correction 1: the stored norm of each group of L coordinates (the
 *             vector, L = d, or the block, L = 32) is n sqrt(L) / ||c[code]||
 *             over the group, so that the reconstruction keeps the group's
 *             norm ([TQ+ guide] §11 names the method; this is the reading)
 * QJL contexts take rotation TQ_ROTATION_WHT, norm_group 0 and no correction
 * (TQ_STATUS_UNSUPPORTED otherwise); a Haar context takes norm_group 0.
 */
struct tq_config {
    uint64_t seed;
    int32_t head_dim;
    int32_t bits;
    int32_t block;
    int32_t qjl;
    int32_t qjl_dim;
    int32_t rotation;
    int32_t norm_group;
    int32_t norm_correction;
};

/* Opaque, immutable context: the config plus its device tables (D1/D2 sign
 * masks, fp16-exact Lloyd-Max codebook, thresholds, S).  Bound to the device
 * current at creation. */
struct tq_ctx;

/* Vector-grid view of caller-owned packed planes (see the layout above).
 * signs/rnorms are only used when the ctx has qjl = 1. */
struct tq_planes {
    uint8_t * codes;
    uint16_t * norms;
    uint8_t * signs;
    uint16_t * rnorms;
    int64_t stride[3];
};

/* Validate cfg, build its tables on the host and upload them to the current
 * device.  *out receives the ctx on success.  Errors: INVALID_ARG (bad cfg or
 * NULL), NO_MEMORY, DEVICE. */
int32_t tq_ctx_create(const struct tq_config * cfg, struct tq_ctx ** out);

/* Release a ctx and its device tables (NULL is ignored).  The caller must
 * ensure no queued work still uses it. */
void tq_ctx_free(struct tq_ctx * ctx);

/* Host-only (no device needed): write the tables cfg generates.  Any pointer
 * may be NULL to skip that table.  d1, d2: d entries of +-1.  codebook: 2^b
 * fp16-exact centroids, ascending.  thresholds: 2^b - 1 midpoints.
 * s_rowmajor: m*d entries (only when cfg->qjl).  Rotation: R = D1.H.D2/sqrt(d)
 * with H the Sylvester Hadamard matrix ([TQ+ guide] §4). */
int32_t tq_tables_export(const struct tq_config * cfg, int8_t * d1, int8_t * d2,
                         float * codebook, float * thresholds, float * s_rowmajor);

/* Bytes per vector in each plane for cfg (0 on an invalid cfg). */
int64_t tq_code_bytes(const struct tq_config * cfg);
int64_t tq_sign_bytes(const struct tq_config * cfg);
/* fp16 norms per vector for cfg: 1, or d/32 with norm_group = 32 (0 on an
 * invalid cfg). */
int64_t tq_norm_count(const struct tq_config * cfg);

/* Host-only (no device needed): the dense rotation R (d x d, row-major,
 * float64) that cfg applies, y = R x: D1.H.D2/sqrt(d) or the Haar Q
 * ([TQ+ guide] §4).  Errors: INVALID_ARG. */
int32_t tq_rotation_export(const struct tq_config * cfg, double * r_rowmajor);

/*
 * Encode a [n0, n1, n2] grid of d-vectors ([TQ+ guide] §4, §5.1-§5.2;
 * [Orión plan] Fase 3 sketches; [TQ explainer] §2.2):
 *   n = ||x||_2 (fp64 accumulation, stored fp16 RNE);
 *   z = sqrt(d) * R x / n;  code_i = #{k : tau_k < z_i};  pack;
 *   QJL: rho = (z - c[code]) / sqrt(d), gamma = ||rho|| (fp16), sign bits of
 *   S rho.
 * x: device pointer, dtype TQ_DTYPE_F32 or TQ_DTYPE_BF16; element (i0,i1,i2,k)
 * at x[i0*x_stride[0] + i1*x_stride[1] + i2*x_stride[2] + k] (strides in
 * elements; the d elements of a vector are contiguous and 16-byte aligned).
 * out: planes to write (caller-owned device memory).  n0*n1*n2 == 0 is a no-op;
 * more than 2^32 - 1 vectors in one call gives TQ_STATUS_UNSUPPORTED.
 * Precision: the norm is accumulated in double, so fp16 norms match a float64
 * evaluation except within ~1e-15 relative of an fp16 rounding midpoint.  For
 * an MSE-only ctx the rotation runs in fp32: a code can differ from a float64
 * evaluation only within ~1e-6 of a threshold.  For a qjl ctx the rotation,
 * residual and gamma run in double as well.
 */
int32_t tq_encode(const struct tq_ctx * ctx, const void * x, int32_t x_dtype,
                  int64_t n0, int64_t n1, int64_t n2, const int64_t x_stride[3],
                  struct tq_planes out, void * hip_stream);

/*
 * Rotated-query scores against packed keys, straight from the codes
 * ([TQ+ guide] §5.3 pre-rotate-queries: <q, R^T c> = <R q, c>; [TQ explainer]
 * §3.2 attention logits from 4-bit keys, §2.2.2 full-precision query):
 *   s[i, j] = scale * N_j * ( <R q_i, c[code_j]> / sqrt(d)
 *                             + gamma_j sqrt(pi/2)/m <S R q_i, sigma_j> )
 * (the second term only for a qjl ctx; sigma = +-1 from the sign bits).
 * q: device fp32 [n_q, d] dense.  Keys: the n_k vectors at plane offsets
 * j * k.stride[2] (stride[0], stride[1] unused).
 * top_k == 0: out_scores is device fp32 [n_q, n_k]; out_idx ignored.
 * top_k in 1..64: out_scores [n_q, top_k] fp32 and out_idx [n_q, top_k] int64,
 * best first, equal scores ordered by lower index; the full score matrix is
 * never stored.  workspace: device memory of tq_scores_workspace() bytes.
 * n_k is limited to 2^31 - 1 (TQ_STATUS_UNSUPPORTED beyond).
 */
int32_t tq_scores(const struct tq_ctx * k_ctx, const float * q, int64_t n_q, float scale,
                  struct tq_planes k, int64_t n_k, int32_t top_k,
                  float * out_scores, int64_t * out_idx,
                  void * workspace, int64_t workspace_bytes, void * hip_stream);

int64_t tq_scores_workspace(const struct tq_ctx * k_ctx, int64_t n_q, int64_t n_k, int32_t top_k);

/*
 * Fused decode attention over packed K and V ([TQ explainer] §4.3:
 * softmax(q K^T * scale) V; [TQ+ guide] §5.3 pre-rotated query, §6.1 output
 * rotated back to the original domain):
 *   out[b, h] = sum_{j < seq_lens[b]} p_j v_hat_j,  p = softmax_j(s_j),
 *   s_j = scale * <q_{b,h}, k_hat_j>  (QJL-corrected when k_ctx has qjl),
 * with query head h reading KV head h / (Hq / Hkv).
 * q: device fp32 [B, Hq, d] dense.  k, v: planes over the grid [B, Hkv, Tcap].
 * seq_lens: device int32 [B]; entries are clamped to [0, t_max]; a zero
 * length gives a zero output row.  t_max: host upper bound of seq_lens (sizes
 * the launch).  out: device fp32 [B, Hq, d] dense.  workspace: device memory
 * of tq_attend_decode_workspace() bytes.  k_ctx and v_ctx must share
 * head_dim and seed (the output rotation is v_ctx's); v_ctx must not be qjl.
 */
int32_t tq_attend_decode(const struct tq_ctx * k_ctx, const struct tq_ctx * v_ctx,
                         const float * q, struct tq_planes k, struct tq_planes v,
                         const int32_t * seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int64_t t_max, float scale, float * out,
                         void * workspace, int64_t workspace_bytes, void * hip_stream);

/* Workspace bytes tq_attend_decode needs for these contexts and sizes (the
 * split of the context into chunks depends on the device's occupancy); -1 on
 * invalid arguments. */
int64_t tq_attend_decode_workspace(const struct tq_ctx * k_ctx, const struct tq_ctx * v_ctx, int32_t B,
                                   int32_t Hq, int32_t Hkv, int64_t t_max);

/*
 * Causal prefill attention over packed K and V ([TQ explainer] §4.3
 * attention; [TQ+ guide] §1.2 prefill context scaling, §5.3 pre-rotated
 * queries and the flash-attention path): the last Tq positions of each
 * sequence attend to the cache up to and including themselves,
 *   out[b, h, i] = sum_{j <= p} p_j v_hat_j,  p = seq_lens[b] - Tq + i,
 *   p_j = softmax_j(scale * <q_{b,h,i}, k_hat_j>)  (QJL-corrected keys),
 * with query head h reading KV head h / (Hq / Hkv).  A query whose position
 * p is negative (a sequence shorter than Tq) gets a zero row.
 * q: device fp32 [B, Hq, Tq, d] dense, 16-byte aligned.  k, v: planes over
 * [B, Hkv, Tcap] already holding the Tq new positions (tq_encode them into
 * the cache first).  seq_lens: device int32 [B], clamped to [0, t_max].
 * out: device fp32 [B, Hq, Tq, d].  workspace: tq_attend_prefill_workspace()
 * bytes.  head_dim 64, 128 or 256, one norm per vector (block-norm contexts
 * give TQ_STATUS_UNSUPPORTED); K and V share head_dim and rotation.
 */
int32_t tq_attend_prefill(const struct tq_ctx * k_ctx, const struct tq_ctx * v_ctx,
                          const float * q, struct tq_planes k, struct tq_planes v,
                          const int32_t * seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                          int64_t Tq, int64_t t_max, float scale, float * out,
                          void * workspace, int64_t workspace_bytes, void * hip_stream);

/* Workspace bytes tq_attend_prefill needs; -1 on invalid arguments. */
int64_t tq_attend_prefill_workspace(const struct tq_ctx * k_ctx, const struct tq_ctx * v_ctx,
                                    int32_t B, int32_t Hq, int64_t Tq);

/*
 * tq_attend_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and results
 * as tq_attend_decode; the workspace is a fixed device buffer of
 * TQ_ATTEND_STATIC_SCRATCH_BYTES = 16 MiB held by the library on each GPU it
 * runs on until the process ends.  Sizes whose tq_attend_decode_workspace()
 * exceeds it give TQ_STATUS_UNSUPPORTED.  The call allocates nothing.  Every
 * call on one GPU shares that GPU's buffer: calls that overlap on one GPU
 * (on different streams or host threads without ordering) race and give
 * undefined outputs.  The current device must be the contexts' device.
 */
int32_t tq_attend_decode_static(const struct tq_ctx * k_ctx, const struct tq_ctx * v_ctx,
                                const float * q, struct tq_planes k, struct tq_planes v,
                                const int32_t * seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                int64_t t_max, float scale, float * out, void * hip_stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char * tq_last_error(void);

/* Library version string. */
const char * tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
