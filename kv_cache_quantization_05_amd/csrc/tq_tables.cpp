// Host-side table generation for libtq: rotation signs, JL matrix, codebook.
//
// Rotation data is generated from the seed at context creation rather than
// shipped as a static table, and one seed always yields one matrix
// ([TQ+ guide] §3, Codex finding 6).  Readings where the pages are silent:
//   * generator: SplitMix64 (Steele, Lea, Flood 2014); it is counter based,
//     output k of a stream seeded with s is mix(s + (k+1) * golden_gamma);
//   * D1 = outputs 0..d-1, D2 = outputs d..2d-1 of the stream seeded with the
//     config seed; the entry is -1 when the output's top bit is set;
//   * S (m x d, row-major) from the stream seeded with seed ^ 0x514A4C00...;
//     consecutive output pairs -> Box-Muller (double) -> two float entries;
//   * the dense Haar rotation from a third stream (seed ^ 0x48414152...),
//     the same Box-Muller fill, and a Householder QR with the sign and
//     determinant fixes ([TQ+ guide] §3: QR of a seeded matrix, det = +1);
//   * codebook: Lloyd-Max quantiser of N(0,1) with 2^b levels (Max 1960),
//     each centroid rounded once from double to fp16 (RNE); thresholds are
//     midpoints of neighbouring fp16 centroids (exact in float).
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kSStream = 0x514A4C0000000000ull;
constexpr uint64_t kHaarStream = 0x4841415200000000ull;

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Output k (0-based) of the SplitMix64 stream seeded with `seed`.
uint64_t splitmix_at(uint64_t seed, uint64_t k) { return mix64(seed + (k + 1) * kGamma); }

// Round a double to the nearest fp16 (ties to even) in one step.
uint16_t half_bits_from_double(double v) {
    uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (std::isnan(v)) return 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;
    if (a < std::ldexp(1.0, -14)) {
        double q = std::nearbyint(std::ldexp(a, 24));  // exact scaling, RNE
        return sign | static_cast<uint16_t>(q);       // q == 1024 is the min normal
    }
    int e2;
    std::frexp(a, &e2);                                // a = f * 2^e2, f in [0.5, 1)
    int e = e2 - 1;
    double q = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31) return sign | 0x7C00;
    return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(q) - 1024));
}

// Outputs k, k + 1 of the stream seeded with `stream` -> two Gaussians
// (Box-Muller in double, each rounded to float).
void box_muller(uint64_t stream, int64_t k, float & g0, float & g1) {
    const uint64_t z1 = splitmix_at(stream, k);
    const uint64_t z2 = splitmix_at(stream, k + 1);
    const double u1 = std::ldexp(static_cast<double>((z1 >> 11) + 1), -53);
    const double u2 = std::ldexp(static_cast<double>(z2 >> 11), -53);
    const double r = std::sqrt(-2.0 * std::log(u1));
    g0 = static_cast<float>(r * std::cos(2.0 * M_PI * u2));
    g1 = static_cast<float>(r * std::sin(2.0 * M_PI * u2));
}

double half_bits_to_double(uint16_t h) {
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v = e == 0 ? std::ldexp(static_cast<double>(f), -24)
                      : std::ldexp(static_cast<double>(f + 1024), e - 25);
    return (h & 0x8000) ? -v : v;
}

double gauss_pdf(double t) {
    return std::isinf(t) ? 0.0 : std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI);
}

// P(a < X <= b), X ~ N(0,1), using the tail that keeps relative precision.
double gauss_mass(double a, double b) {
    const double r2 = std::sqrt(2.0);
    if (a >= 0.0) return 0.5 * (std::erfc(a / r2) - std::erfc(b / r2));
    if (b <= 0.0) return 0.5 * (std::erfc(-b / r2) - std::erfc(-a / r2));
    return 1.0 - 0.5 * std::erfc(-a / r2) - 0.5 * std::erfc(b / r2);
}

// Lloyd's iteration for the minimum-MSE quantiser of N(0,1).
std::vector<double> lloyd_max(int bits) {
    const int L = 1 << bits;
    std::vector<double> c(L), t(L + 1), nc(L);
    for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
    for (int it = 0; it < 100000; ++it) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        double moved = 0.0;
        for (int k = 0; k < L; ++k) {
            nc[k] = (gauss_pdf(t[k]) - gauss_pdf(t[k + 1])) / gauss_mass(t[k], t[k + 1]);
            moved = std::fmax(moved, std::fabs(nc[k] - c[k]));
        }
        c.swap(nc);
        if (moved < 1e-15) break;
    }
    return c;
}

}  // namespace

void split_fp16(const float * v, int64_t n, uint16_t * hi, uint16_t * lo) {
    for (int64_t i = 0; i < n; ++i) {
        hi[i] = half_bits_from_double(v[i]);
        lo[i] = half_bits_from_double(static_cast<double>(v[i]) - half_bits_to_double(hi[i]));
    }
}

int validate_config(const tq_config & cfg, const char ** why) {
    const int d = cfg.head_dim;
    if (d != 32 && d != 64 && d != 128 && d != 256) {
        *why = "head_dim must be 32, 64, 128 or 256";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.bits < 2 || cfg.bits > 4) {
        *why = "bits must be 2, 3 or 4";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.block != 32) {
        *why = "block must be 32";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.qjl != 0 && cfg.qjl != 1) {
        *why = "qjl must be 0 or 1";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.qjl_dim < 0 || (cfg.qjl_dim > 0 && (cfg.qjl_dim % 32 != 0 || cfg.qjl_dim > 256))) {
        *why = "qjl_dim must be 0 or a multiple of 32 up to 256";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.rotation != TQ_ROTATION_WHT && cfg.rotation != TQ_ROTATION_HAAR) {
        *why = "rotation must be TQ_ROTATION_WHT or TQ_ROTATION_HAAR";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.norm_group != 0 && cfg.norm_group != 32) {
        *why = "norm_group must be 0 (one norm per vector) or 32 (one per 32-code block)";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.norm_correction != 0 && cfg.norm_correction != 1) {
        *why = "norm_correction must be 0 or 1";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.qjl && (cfg.norm_group != 0 || cfg.norm_correction != 0)) {
        *why = "QJL keys take one plain norm per vector (norm_group 0, no correction)";
        return TQ_STATUS_INVALID_ARG;
    }
    if (cfg.qjl && cfg.qjl_dim != 0 && cfg.qjl_dim != d) {
        *why = "qjl_dim other than head_dim is not supported by the kernels";
        return TQ_STATUS_UNSUPPORTED;
    }
    if (cfg.qjl && cfg.rotation == TQ_ROTATION_HAAR) {
        *why = "QJL keys with the Haar rotation are not supported by the kernels";
        return TQ_STATUS_UNSUPPORTED;
    }
    if (cfg.rotation == TQ_ROTATION_HAAR && cfg.norm_group != 0) {
        *why = "block norms with the Haar rotation are not supported by the kernels";
        return TQ_STATUS_UNSUPPORTED;
    }
    return TQ_STATUS_OK;
}

// Dense rotation R (d x d, row-major) applied as y = R x.
//  * WHT: R = D1 H D2 / sqrt(d), H the Sylvester matrix (+-1 / sqrt(d)).
//  * Haar: Householder QR of the seeded Gaussian G (stream seed ^ "HAAR",
//    Box-Muller pairs as for S, entries rounded to float), then Q's columns
//    times the signs of R's diagonal (the unique factor with a positive
//    diagonal), then column 0 negated if det(Q) = -1.
void build_rotation(const tq_config & cfg, double * r) {
    const int d = cfg.head_dim;
    if (cfg.rotation != TQ_ROTATION_HAAR) {
        std::vector<int8_t> d1(d), d2(d);
        build_tables(cfg, d1.data(), d2.data(), nullptr, nullptr, nullptr);
        const double s = 1.0 / std::sqrt(static_cast<double>(d));
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j)
                r[int64_t(i) * d + j] = ((__builtin_popcount(i & j) & 1) ? -s : s) * d1[i] * d2[j];
        return;
    }
    std::vector<double> a(int64_t(d) * d);
    {
        const uint64_t gs = cfg.seed ^ kHaarStream;
        for (int64_t k = 0; k < int64_t(d) * d; k += 2) {
            float g0, g1;
            box_muller(gs, k, g0, g1);
            a[k] = g0;
            a[k + 1] = g1;
        }
    }
    // Householder: column k's reflector v_k (unit) maps a[k:, k] to
    // alpha_k e_1 with alpha_k = -sign(a_kk) ||a[k:, k]||.
    std::vector<double> vs(int64_t(d) * d, 0.0), diag(d);
    int reflections = 0;
    for (int k = 0; k < d; ++k) {
        double nrm = 0.0;
        for (int i = k; i < d; ++i) nrm += a[int64_t(i) * d + k] * a[int64_t(i) * d + k];
        nrm = std::sqrt(nrm);
        const double akk = a[int64_t(k) * d + k];
        const double alpha = akk > 0 ? -nrm : nrm;
        double * v = &vs[int64_t(k) * d];
        for (int i = k; i < d; ++i) v[i] = a[int64_t(i) * d + k];
        v[k] -= alpha;
        double vn = 0.0;
        for (int i = k; i < d; ++i) vn += v[i] * v[i];
        if (k == d - 1 || vn == 0.0) {   // nothing below the diagonal: no reflection
            for (int i = k; i < d; ++i) v[i] = 0.0;
            diag[k] = akk;
            continue;
        }
        vn = std::sqrt(vn);
        for (int i = k; i < d; ++i) v[i] /= vn;
        ++reflections;
        for (int j = k; j < d; ++j) {
            double dot = 0.0;
            for (int i = k; i < d; ++i) dot += v[i] * a[int64_t(i) * d + j];
            for (int i = k; i < d; ++i) a[int64_t(i) * d + j] -= 2.0 * v[i] * dot;
        }
        diag[k] = a[int64_t(k) * d + k];
    }
    // Q = H_0 H_1 ... applied to the identity from the last reflector back
    std::vector<double> q(int64_t(d) * d, 0.0);
    for (int i = 0; i < d; ++i) q[int64_t(i) * d + i] = 1.0;
    for (int k = d - 1; k >= 0; --k) {
        const double * v = &vs[int64_t(k) * d];
        bool any = false;
        for (int i = k; i < d; ++i) any = any || v[i] != 0.0;
        if (!any) continue;
        for (int j = 0; j < d; ++j) {
            double dot = 0.0;
            for (int i = k; i < d; ++i) dot += v[i] * q[int64_t(i) * d + j];
            for (int i = k; i < d; ++i) q[int64_t(i) * d + j] -= 2.0 * v[i] * dot;
        }
    }
    // det(H_k) = -1 for each reflection; the sign fix multiplies by the
    // product of the diagonal's signs
    int neg = reflections;
    for (int j = 0; j < d; ++j) {
        if (diag[j] < 0) {
            ++neg;
            for (int i = 0; i < d; ++i) q[int64_t(i) * d + j] = -q[int64_t(i) * d + j];
        }
    }
    if (neg & 1)
        for (int i = 0; i < d; ++i) q[int64_t(i) * d] = -q[int64_t(i) * d];
    for (int64_t i = 0; i < int64_t(d) * d; ++i) r[i] = q[i];
}

int build_tables(const tq_config & cfg, int8_t * d1, int8_t * d2, float * codebook,
                 float * thresholds, float * s_rowmajor) {
    const int d = cfg.head_dim;
    const int m = cfg.qjl_dim ? cfg.qjl_dim : d;
    for (int i = 0; i < d; ++i) {
        if (d1) d1[i] = (splitmix_at(cfg.seed, i) >> 63) ? -1 : 1;
        if (d2) d2[i] = (splitmix_at(cfg.seed, d + i) >> 63) ? -1 : 1;
    }
    const int L = 1 << cfg.bits;
    std::vector<double> c = lloyd_max(cfg.bits);
    std::vector<double> c16(L);
    for (int k = 0; k < L; ++k) c16[k] = half_bits_to_double(half_bits_from_double(c[k]));
    // Lloyd's iteration keeps the centroids ascending; rounding preserves order.
    if (codebook)
        for (int k = 0; k < L; ++k) codebook[k] = static_cast<float>(c16[k]);
    if (thresholds)
        for (int k = 0; k + 1 < L; ++k) thresholds[k] = static_cast<float>(0.5 * (c16[k] + c16[k + 1]));
    if (cfg.qjl && s_rowmajor) {
        const uint64_t s_seed = cfg.seed ^ kSStream;
        const int64_t total = static_cast<int64_t>(m) * d;
        for (int64_t k = 0; k < total; k += 2) box_muller(s_seed, k, s_rowmajor[k], s_rowmajor[k + 1]);
    }
    return TQ_STATUS_OK;
}

}  // namespace tq
