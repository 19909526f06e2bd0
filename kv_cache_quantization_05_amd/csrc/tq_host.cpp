// libtq host side: contexts, argument validation, workspace sizing, launches.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tq_internal.h"

struct tq_ctx {
    tq_config cfg;
    int device;
    tq::dev_tables tab;
    float * S_dev;
    float * Q_dev;
};

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char * fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t status, const char * fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int32_t ok() {
    g_last_error.clear();
    return TQ_STATUS_OK;
}

}  // namespace

int32_t tq::set_error(int32_t status, const char * fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int tq::ctx_device(const tq_ctx * ctx) { return ctx->device; }

namespace {

int32_t device_status(hipError_t e, const char * what) {
    if (e == hipSuccess) return ok();
    return fail(TQ_STATUS_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int64_t m_of(const tq_config & c) { return c.qjl_dim ? c.qjl_dim : c.head_dim; }

bool aligned(const void * p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks a plane set for `ctx` against a vector grid; returns a message or NULL.
const char * check_planes(const tq_ctx * ctx, const tq_planes & p, bool need_qjl) {
    if (!p.codes || !p.norms) return "codes and norms planes must be non-NULL";
    if (!aligned(p.codes, 4)) return "codes plane must be 4-byte aligned";
    if (!aligned(p.norms, 2)) return "norms plane must be 2-byte aligned";
    if (need_qjl) {
        if (!p.signs || !p.rnorms) return "QJL signs and rnorms planes must be non-NULL";
        if (!aligned(p.signs, 4)) return "signs plane must be 4-byte aligned";
        if (!aligned(p.rnorms, 2)) return "rnorms plane must be 2-byte aligned";
    }
    for (int i = 0; i < 3; ++i)
        if (p.stride[i] < 0) return "plane strides must be non-negative";
    (void)ctx;
    return nullptr;
}

constexpr int64_t kAlign = 256;
int64_t round_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

}  // namespace

extern "C" {

const char * tq_last_error(void) { return g_last_error.c_str(); }

const char * tq_version(void) { return "libtq 0.1 (gfx950)"; }

int64_t tq_code_bytes(const tq_config * cfg) {
    const char * why;
    if (!cfg || tq::validate_config(*cfg, &why) == TQ_STATUS_INVALID_ARG) return 0;
    return static_cast<int64_t>(cfg->head_dim) * cfg->bits / 8;
}

int64_t tq_sign_bytes(const tq_config * cfg) {
    const char * why;
    if (!cfg || tq::validate_config(*cfg, &why) == TQ_STATUS_INVALID_ARG) return 0;
    return cfg->qjl ? m_of(*cfg) / 8 : 0;
}

int64_t tq_norm_count(const tq_config * cfg) {
    const char * why;
    if (!cfg || tq::validate_config(*cfg, &why) == TQ_STATUS_INVALID_ARG) return 0;
    return cfg->norm_group ? cfg->head_dim / cfg->norm_group : 1;
}

int32_t tq_rotation_export(const tq_config * cfg, double * r_rowmajor) {
    if (!cfg || !r_rowmajor) return fail(TQ_STATUS_INVALID_ARG, "cfg and r_rowmajor must be non-NULL");
    const char * why = "";
    int32_t st = tq::validate_config(*cfg, &why);
    if (st == TQ_STATUS_INVALID_ARG) return fail(st, "invalid config: %s", why);
    tq::build_rotation(*cfg, r_rowmajor);
    return ok();
}

int32_t tq_tables_export(const tq_config * cfg, int8_t * d1, int8_t * d2, float * codebook,
                         float * thresholds, float * s_rowmajor) {
    if (!cfg) return fail(TQ_STATUS_INVALID_ARG, "cfg is NULL");
    const char * why = "";
    int32_t st = tq::validate_config(*cfg, &why);
    if (st == TQ_STATUS_INVALID_ARG) return fail(st, "invalid config: %s", why);
    tq::build_tables(*cfg, d1, d2, codebook, thresholds, s_rowmajor);
    return ok();
}

int32_t tq_ctx_create(const tq_config * cfg, tq_ctx ** out) {
    if (!cfg || !out) return fail(TQ_STATUS_INVALID_ARG, "cfg and out must be non-NULL");
    *out = nullptr;
    const char * why = "";
    int32_t st = tq::validate_config(*cfg, &why);
    if (st != TQ_STATUS_OK) return fail(st, "config: %s", why);
    const int d = cfg->head_dim;
    const int64_t m = m_of(*cfg);
    std::vector<int8_t> d1(d), d2(d);
    std::vector<float> cb(16, 0.0f), th(16, INFINITY);
    std::vector<float> S(cfg->qjl ? m * d : 0);
    tq::build_tables(*cfg, d1.data(), d2.data(), cb.data(), th.data(), cfg->qjl ? S.data() : nullptr);
    th[(1 << cfg->bits) - 1] = INFINITY;

    tq_ctx * c = new (std::nothrow) tq_ctx();
    if (!c) return fail(TQ_STATUS_NO_MEMORY, "host allocation failed");
    c->cfg = *cfg;
    c->S_dev = nullptr;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        return fail(TQ_STATUS_DEVICE, "no HIP device available");
    }
    std::memset(&c->tab, 0, sizeof c->tab);
    for (int i = 0; i < d; ++i) {
        if (d1[i] < 0) c->tab.d1[i / 32] |= 1u << (i % 32);
        if (d2[i] < 0) c->tab.d2[i / 32] |= 1u << (i % 32);
    }
    for (int k = 0; k < 16; ++k) {
        c->tab.cb[k] = cb[k];
        c->tab.th[k] = th[k];
    }
    c->tab.d = d;
    c->tab.bits = cfg->bits;
    c->tab.m = static_cast<int32_t>(m);
    c->tab.qjl = cfg->qjl;
    c->tab.haar = cfg->rotation == TQ_ROTATION_HAAR;
    c->tab.norm_group = cfg->norm_group;
    c->tab.norm_corr = cfg->norm_correction;
    c->tab.S = nullptr;
    c->tab.Q = nullptr;
    c->Q_dev = nullptr;
    if (c->tab.haar) {
        // one allocation: Q (fp32), then the fp16 split of 16 Q (hi, lo):
        // the scale keeps the low parts of the small entries normal in fp16
        const size_t n = size_t(d) * d;
        std::vector<double> qd(n);
        tq::build_rotation(*cfg, qd.data());
        std::vector<float> qf(n), q16(n);
        for (size_t i = 0; i < n; ++i) {
            qf[i] = static_cast<float>(qd[i]);
            q16[i] = static_cast<float>(16.0 * qd[i]);
        }
        std::vector<uint16_t> h16(2 * n);
        tq::split_fp16(q16.data(), static_cast<int64_t>(n), h16.data(), h16.data() + n);
        const size_t bytes = n * sizeof(float) + 2 * n * sizeof(uint16_t);
        hipError_t e = hipMalloc(&c->Q_dev, bytes);
        if (e != hipSuccess) {
            delete c;
            return fail(TQ_STATUS_NO_MEMORY, "hipMalloc of the rotation failed: %s", hipGetErrorString(e));
        }
        e = hipMemcpy(c->Q_dev, qf.data(), n * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess)
            e = hipMemcpy(c->Q_dev + n, h16.data(), 2 * n * sizeof(uint16_t), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            hipFree(c->Q_dev);
            delete c;
            return device_status(e, "upload of the rotation");
        }
        c->tab.Q = c->Q_dev;
        c->tab.Q16 = reinterpret_cast<const uint16_t *>(c->Q_dev + n);
    }
    if (cfg->qjl) {
        // one allocation: S (fp32), then its fp16 split hi and lo
        const size_t n = S.size();
        std::vector<uint16_t> s16(2 * n);
        tq::split_fp16(S.data(), static_cast<int64_t>(n), s16.data(), s16.data() + n);
        const size_t bytes = n * sizeof(float) + 2 * n * sizeof(uint16_t);
        hipError_t e = hipMalloc(&c->S_dev, bytes);
        if (e != hipSuccess) {
            if (c->Q_dev) hipFree(c->Q_dev);
            delete c;
            return fail(TQ_STATUS_NO_MEMORY, "hipMalloc of S failed: %s", hipGetErrorString(e));
        }
        e = hipMemcpy(c->S_dev, S.data(), n * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess)
            e = hipMemcpy(c->S_dev + n, s16.data(), 2 * n * sizeof(uint16_t), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            hipFree(c->S_dev);
            if (c->Q_dev) hipFree(c->Q_dev);
            delete c;
            return device_status(e, "upload of S");
        }
        c->tab.S = c->S_dev;
        c->tab.S16 = reinterpret_cast<const uint16_t *>(c->S_dev + n);
    }
    *out = c;
    return ok();
}

void tq_ctx_free(tq_ctx * ctx) {
    if (!ctx) return;
    if (ctx->S_dev) hipFree(ctx->S_dev);
    if (ctx->Q_dev) hipFree(ctx->Q_dev);
    delete ctx;
}

int32_t tq_encode(const tq_ctx * ctx, const void * x, int32_t x_dtype, int64_t n0, int64_t n1,
                  int64_t n2, const int64_t x_stride[3], tq_planes out, void * hip_stream) {
    if (!ctx) return fail(TQ_STATUS_INVALID_ARG, "ctx is NULL");
    if (n0 < 0 || n1 < 0 || n2 < 0) return fail(TQ_STATUS_INVALID_ARG, "negative grid size");
    if (n0 == 0 || n1 == 0 || n2 == 0) return ok();
    if (!x || !x_stride) return fail(TQ_STATUS_INVALID_ARG, "x and x_stride must be non-NULL");
    if (x_dtype != TQ_DTYPE_F32 && x_dtype != TQ_DTYPE_BF16)
        return fail(TQ_STATUS_INVALID_ARG, "x_dtype must be TQ_DTYPE_F32 or TQ_DTYPE_BF16");
    const int64_t esz = x_dtype == TQ_DTYPE_F32 ? 4 : 2;
    if (!aligned(x, 16)) return fail(TQ_STATUS_INVALID_ARG, "x must be 16-byte aligned");
    for (int i = 0; i < 3; ++i)
        if (x_stride[i] < 0 || (x_stride[i] * esz) % 16 != 0)
            return fail(TQ_STATUS_INVALID_ARG, "x strides must be non-negative multiples of 16 bytes");
    if (const char * why = check_planes(ctx, out, ctx->cfg.qjl != 0))
        return fail(TQ_STATUS_INVALID_ARG, "%s", why);
    tq::encode_args a{x, x_dtype, n0, n1, n2, x_stride[0], x_stride[1], x_stride[2], out};
    if (!tq::encode_grid_supported(a))
        return fail(TQ_STATUS_UNSUPPORTED, "encode grids are limited to 2^32 - 1 vectors per call");
    return device_status(tq::launch_encode(ctx->tab, a, static_cast<hipStream_t>(hip_stream)),
                         "encode launch");
}

int64_t tq_scores_workspace(const tq_ctx * k_ctx, int64_t n_q, int64_t n_k, int32_t top_k) {
    if (!k_ctx || n_q < 0 || n_k < 0 || top_k < 0) return -1;
    const int64_t qp = round_up(n_q * (k_ctx->tab.d + k_ctx->tab.m) * 4);
    if (top_k == 0) return qp;
    int32_t ranges = 1;
    int64_t per = 0;
    tq::scores_plan(k_ctx->tab.d, k_ctx->tab.norm_group != 0, n_q, n_k, top_k, ranges, per);
    return qp + round_up(int64_t(ranges) * n_q * top_k * 4) + round_up(int64_t(ranges) * n_q * top_k * 8);
}

int32_t tq_scores(const tq_ctx * k_ctx, const float * q, int64_t n_q, float scale, tq_planes k,
                  int64_t n_k, int32_t top_k, float * out_scores, int64_t * out_idx,
                  void * workspace, int64_t workspace_bytes, void * hip_stream) {
    if (!k_ctx) return fail(TQ_STATUS_INVALID_ARG, "k_ctx is NULL");
    if (n_q < 0 || n_k < 0) return fail(TQ_STATUS_INVALID_ARG, "negative n_q or n_k");
    if (top_k < 0 || top_k > 64) return fail(TQ_STATUS_INVALID_ARG, "top_k must be in 0..64");
    if (top_k > 0 && top_k > n_k) return fail(TQ_STATUS_INVALID_ARG, "top_k exceeds n_k");
    if (n_k > (int64_t(1) << 31) - 1) return fail(TQ_STATUS_UNSUPPORTED, "n_k is limited to 2^31 - 1");
    if (n_q == 0 || n_k == 0) return ok();
    if (!q || !out_scores) return fail(TQ_STATUS_INVALID_ARG, "q and out_scores must be non-NULL");
    if (top_k > 0 && !out_idx) return fail(TQ_STATUS_INVALID_ARG, "out_idx must be non-NULL when top_k > 0");
    if (const char * why = check_planes(k_ctx, k, k_ctx->cfg.qjl != 0))
        return fail(TQ_STATUS_INVALID_ARG, "%s", why);
    const int64_t need = tq_scores_workspace(k_ctx, n_q, n_k, top_k);
    if (!workspace || workspace_bytes < need)
        return fail(TQ_STATUS_INVALID_ARG, "workspace too small: need %lld bytes", (long long)need);
    if (!aligned(workspace, 256)) return fail(TQ_STATUS_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    char * ws = static_cast<char *>(workspace);
    float * qp = reinterpret_cast<float *>(ws);
    const int64_t qp_stride = k_ctx->tab.d + k_ctx->tab.m;
    hipError_t e = tq::launch_query_prep(k_ctx->tab, q, n_q, qp, qp_stride, s);
    if (e != hipSuccess) return device_status(e, "query prep launch");
    tq::scores_args a{};
    a.qp = qp;
    a.qp_stride = qp_stride;
    a.n_q = n_q;
    a.k = k;
    a.n_k = n_k;
    a.scale = scale;
    a.top_k = top_k;
    a.out_scores = out_scores;
    a.out_idx = out_idx;
    tq::scores_plan(k_ctx->tab.d, k_ctx->tab.norm_group != 0, n_q, n_k, top_k, a.n_ranges, a.keys_per_range);
    if (top_k > 0) {
        char * p = ws + round_up(n_q * qp_stride * 4);
        a.cand_s = reinterpret_cast<float *>(p);
        a.cand_i = reinterpret_cast<int64_t *>(p + round_up(a.n_ranges * n_q * top_k * 4));
    }
    return device_status(tq::launch_scores(k_ctx->tab, a, s), "scores launch");
}

int64_t tq_attend_decode_workspace(const tq_ctx * k_ctx, const tq_ctx * v_ctx, int32_t B, int32_t Hq,
                                   int32_t Hkv, int64_t t_max) {
    if (!k_ctx || !v_ctx || B < 0 || Hq < 0 || Hkv <= 0 || t_max < 0) return -1;
    const int d = k_ctx->tab.d;
    const int64_t chunk = tq::attend_chunk_tokens(k_ctx->tab, v_ctx->tab, B, Hq, Hkv, t_max);
    const int64_t n_chunks = t_max > 0 ? (t_max + chunk - 1) / chunk : 1;
    const int64_t qp = round_up(int64_t(B) * Hq * (d + k_ctx->tab.m) * 4);
    const int64_t part = round_up(int64_t(B) * Hq * n_chunks * (d + 2) * 4);
    return qp + part;
}

int32_t tq_attend_decode(const tq_ctx * k_ctx, const tq_ctx * v_ctx, const float * q, tq_planes k,
                         tq_planes v, const int32_t * seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int64_t t_max, float scale, float * out, void * workspace,
                         int64_t workspace_bytes, void * hip_stream) {
    if (!k_ctx || !v_ctx) return fail(TQ_STATUS_INVALID_ARG, "k_ctx and v_ctx must be non-NULL");
    if (k_ctx->tab.d != v_ctx->tab.d)
        return fail(TQ_STATUS_INVALID_ARG, "k_ctx and v_ctx must share head_dim");
    if (k_ctx->cfg.seed != v_ctx->cfg.seed || k_ctx->cfg.rotation != v_ctx->cfg.rotation)
        return fail(TQ_STATUS_UNSUPPORTED, "k_ctx and v_ctx must share the rotation (seed and kind)");
    if (v_ctx->cfg.qjl) return fail(TQ_STATUS_INVALID_ARG, "v_ctx must not use QJL");
    if (k_ctx->device != v_ctx->device) return fail(TQ_STATUS_INVALID_ARG, "contexts on different devices");
    if (B < 0 || Hq < 0 || Hkv <= 0 || t_max < 0) return fail(TQ_STATUS_INVALID_ARG, "negative sizes");
    if (Hq % Hkv != 0) return fail(TQ_STATUS_INVALID_ARG, "Hq must be a multiple of Hkv");
    const int group = Hkv ? Hq / Hkv : 0;
    if (B == 0 || Hq == 0) return ok();
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(TQ_STATUS_UNSUPPORTED, "Hq / Hkv must be 1, 2, 4 or 8");
    if (!q || !out || !seq_lens) return fail(TQ_STATUS_INVALID_ARG, "q, out and seq_lens must be non-NULL");
    if (t_max > (int64_t(1) << 31) - 1) return fail(TQ_STATUS_INVALID_ARG, "t_max too large");
    if (const char * why = check_planes(k_ctx, k, k_ctx->cfg.qjl != 0))
        return fail(TQ_STATUS_INVALID_ARG, "k: %s", why);
    if (const char * why = check_planes(v_ctx, v, false)) return fail(TQ_STATUS_INVALID_ARG, "v: %s", why);
    const int64_t need = tq_attend_decode_workspace(k_ctx, v_ctx, B, Hq, Hkv, t_max);
    if (!workspace || workspace_bytes < need)
        return fail(TQ_STATUS_INVALID_ARG, "workspace too small: need %lld bytes", (long long)need);
    if (!aligned(workspace, 256)) return fail(TQ_STATUS_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int d = k_ctx->tab.d;
    const int64_t qp_stride = d + k_ctx->tab.m;
    char * ws = static_cast<char *>(workspace);
    float * qp = reinterpret_cast<float *>(ws);
    tq::attend_args a{};
    a.q = q;
    a.qp = qp;
    a.qp_stride = qp_stride;
    a.k = k;
    a.v = v;
    a.seq_lens = seq_lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.t_max = t_max;
    a.chunk = tq::attend_chunk_tokens(k_ctx->tab, v_ctx->tab, B, Hq, Hkv, t_max);
    a.n_chunks = t_max > 0 ? static_cast<int32_t>((t_max + a.chunk - 1) / a.chunk) : 1;
    a.scale = scale;
    a.partial = reinterpret_cast<float *>(ws + round_up(int64_t(B) * Hq * qp_stride * 4));
    a.out = out;
    return device_status(tq::launch_attend(k_ctx->tab, v_ctx->tab, a, s), "attend launch");
}

int64_t tq_attend_prefill_workspace(const tq_ctx * k_ctx, const tq_ctx * v_ctx, int32_t B, int32_t Hq,
                                    int64_t Tq) {
    if (!k_ctx || !v_ctx || B < 0 || Hq < 0 || Tq < 0) return -1;
    const int64_t rows = int64_t(B) * Hq * Tq;
    return round_up(rows * (k_ctx->tab.d + k_ctx->tab.m) * 4) + round_up(rows * k_ctx->tab.d * 4);
}

int32_t tq_attend_prefill(const tq_ctx * k_ctx, const tq_ctx * v_ctx, const float * q, tq_planes k, tq_planes v,
                          const int32_t * seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int64_t Tq, int64_t t_max,
                          float scale, float * out, void * workspace, int64_t workspace_bytes, void * hip_stream) {
    if (!k_ctx || !v_ctx) return fail(TQ_STATUS_INVALID_ARG, "k_ctx and v_ctx must be non-NULL");
    if (k_ctx->tab.d != v_ctx->tab.d)
        return fail(TQ_STATUS_INVALID_ARG, "k_ctx and v_ctx must share head_dim");
    if (k_ctx->cfg.seed != v_ctx->cfg.seed || k_ctx->cfg.rotation != v_ctx->cfg.rotation)
        return fail(TQ_STATUS_UNSUPPORTED, "k_ctx and v_ctx must share the rotation (seed and kind)");
    if (v_ctx->cfg.qjl) return fail(TQ_STATUS_INVALID_ARG, "v_ctx must not use QJL");
    if (k_ctx->device != v_ctx->device) return fail(TQ_STATUS_INVALID_ARG, "contexts on different devices");
    if (B < 0 || Hq < 0 || Hkv <= 0 || Tq < 0 || t_max < 0) return fail(TQ_STATUS_INVALID_ARG, "negative sizes");
    if (Hq % Hkv != 0) return fail(TQ_STATUS_INVALID_ARG, "Hq must be a multiple of Hkv");
    if (B == 0 || Hq == 0 || Tq == 0) return ok();
    const int group = Hq / Hkv;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(TQ_STATUS_UNSUPPORTED, "Hq / Hkv must be 1, 2, 4 or 8");
    if (!tq::prefill_supported(k_ctx->tab, v_ctx->tab))
        return fail(TQ_STATUS_UNSUPPORTED, "prefill takes head_dim 64, 128 or 256 and one norm per vector");
    if (!q || !out || !seq_lens) return fail(TQ_STATUS_INVALID_ARG, "q, out and seq_lens must be non-NULL");
    if (t_max > (int64_t(1) << 31) - 1 || Tq > (int64_t(1) << 31) - 1 ||
        int64_t(B) * Hq * Tq > (int64_t(1) << 31) - 1)
        return fail(TQ_STATUS_UNSUPPORTED, "t_max, Tq and B * Hq * Tq are limited to 2^31 - 1");
    if (const char * why = check_planes(k_ctx, k, k_ctx->cfg.qjl != 0))
        return fail(TQ_STATUS_INVALID_ARG, "k: %s", why);
    if (const char * why = check_planes(v_ctx, v, false)) return fail(TQ_STATUS_INVALID_ARG, "v: %s", why);
    const int64_t need = tq_attend_prefill_workspace(k_ctx, v_ctx, B, Hq, Tq);
    if (!workspace || workspace_bytes < need)
        return fail(TQ_STATUS_INVALID_ARG, "workspace too small: need %lld bytes", (long long)need);
    if (!aligned(workspace, 256)) return fail(TQ_STATUS_INVALID_ARG, "workspace must be 256-byte aligned");
    if (!aligned(q, 16)) return fail(TQ_STATUS_INVALID_ARG, "q must be 16-byte aligned");
    const int64_t rows = int64_t(B) * Hq * Tq;
    char * ws = static_cast<char *>(workspace);
    tq::prefill_args a{};
    a.q = q;
    a.qp = reinterpret_cast<float *>(ws);
    a.qp_stride = k_ctx->tab.d + k_ctx->tab.m;
    a.k = k;
    a.v = v;
    a.seq_lens = seq_lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.t_max = t_max;
    a.scale = scale;
    a.out_rot = reinterpret_cast<float *>(ws + round_up(rows * a.qp_stride * 4));
    a.out = out;
    return device_status(tq::launch_prefill(k_ctx->tab, v_ctx->tab, a, static_cast<hipStream_t>(hip_stream)),
                         "prefill launch");
}

}  // extern "C"
