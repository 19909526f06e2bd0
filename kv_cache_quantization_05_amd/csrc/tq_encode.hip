// Encode kernels: norm -> rotation -> scalar codebook -> packing -> QJL.
//
// Steps as the pages order them: per-vector norm extraction ([TQ+ guide]
// §5.1), structured rotation D1.H.D2 by a fast Walsh-Hadamard transform
// ([TQ+ guide] §4), MSE-only centroid quantisation in blocks of 32 with the
// rotation width decoupled from the block size ([TQ+ guide] §5.1-§5.2, §6.1),
// bit packing, and the optional 1-bit QJL sketch of the residual
// ([Orión plan] Fase 3 sign-bit sketch; [TQ explainer] §2.2).
//
// Work mapping: a vector of d coordinates is owned by d/32 consecutive lanes;
// lane `blk` holds coordinates 32*blk .. 32*blk+31, which is exactly one
// packed 32-code block, so each lane writes its own block.  The first five
// butterfly stages run inside a lane's registers, the remaining log2(d/32)
// stages exchange with partner lanes (DPP quad permutes / ds_swizzle).
//
// Two precisions:
//  * MSE-only ctx (encode_kernel): the norm is accumulated in double (fp16
//    norms must round exactly as a float64 evaluation does), the rotation in
//    fp32.  A code can then differ from a float64 evaluation only within
//    ~1e-6 of a threshold, far inside the 1e-5 boundary window.  The
//    quantiser uses the symmetry of the Lloyd-Max codebook (c[2^b-1-k] =
//    -c[k], thresholds likewise, with 0 in the middle): code(z) is the count
//    of positive thresholds below |z| XOR a constant chosen by the sign of
//    z, and the sign flips of D1 become one XOR with 2^b-1 per affected code
//    on the packed words.  Comparing |y| against thresholds pre-multiplied
//    by the norm avoids a per-coordinate division.
//  * QJL ctx (encode_qjl_kernel): everything after the load in double, so
//    that the fp16 residual norm also rounds exactly as float64 does.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

// Unsigned 32-bit division by a runtime divisor through a multiply-high
// (Granlund and Montgomery 1994, round-up method): q = (t + ((n - t) >> s1))
// >> s2 with t = umulhi(m, n).  Exact for every 32-bit n.
struct fastdiv {
    uint32_t d, m, s1, s2;
};

fastdiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return fastdiv{d, static_cast<uint32_t>(m), l < 1 ? l : 1u, l > 1 ? l - 1 : 0u};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const fastdiv & f) {
    const uint32_t t = __umulhi(f.m, n);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

struct grid_index {
    fastdiv n2, n1;
};

// Offsets of vector v of the [n0, n1, n2] grid: input element offset and
// output plane index.  v < 2^32 (checked on the host).
__device__ __forceinline__ void vector_offsets(uint32_t v, const encode_args & a, const grid_index & gi,
                                               int64_t & xoff, int64_t & pv) {
    const uint32_t r = fdiv(v, gi.n2);
    const uint32_t i2 = v - r * gi.n2.d;
    const uint32_t i0 = fdiv(r, gi.n1);
    const uint32_t i1 = r - i0 * gi.n1.d;
    xoff = int64_t(i0) * a.xs0 + int64_t(i1) * a.xs1 + int64_t(i2) * a.xs2;
    pv = int64_t(i0) * a.out.stride[0] + int64_t(i1) * a.out.stride[1] + int64_t(i2) * a.out.stride[2];
}

__device__ __forceinline__ float fma_t(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_t(double a, double b, double c) { return __builtin_fma(a, b, c); }

// Butterflies across the lanes of one vector (lane index bits = the high
// coordinate bits).  The lower-index partner keeps a + b, the other a - b.
template <int LPV, typename T>
__device__ __forceinline__ void cross_lane_fwht(T (&x)[32], int blk) {
    if constexpr (LPV >= 2) {
        const T sg = (blk & 1) ? T(-1) : T(1);
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = fma_t(sg, x[e], lane_xor<1>(x[e]));
    }
    if constexpr (LPV >= 4) {
        const T sg = (blk & 2) ? T(-1) : T(1);
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = fma_t(sg, x[e], lane_xor<2>(x[e]));
    }
    if constexpr (LPV >= 8) {
        const T sg = (blk & 4) ? T(-1) : T(1);
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = fma_t(sg, x[e], lane_xor<4>(x[e]));
    }
}

// Unnormalised 32-point Hadamard transform of a lane's coordinates.
template <typename T>
__device__ __forceinline__ void lane_fwht(T (&x)[32]) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            if ((e & h) == 0) {
                const T p0 = x[e], p1 = x[e + h];
                x[e] = p0 + p1;
                x[e + h] = p0 - p1;
            }
        }
    }
}

// Loads the lane's 32 coordinates of one vector as floats.
template <bool BF16>
__device__ __forceinline__ void load_block(const encode_args & a, int64_t xoff, float (&x)[32]) {
    if constexpr (BF16) {
        const uint4 * p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + xoff);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 w = p[c];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[8 * c + 2 * j] = bf16_lo(ws[j]);
                x[8 * c + 2 * j + 1] = bf16_hi(ws[j]);
            }
        }
    } else {
        const float4 * p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + xoff);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float4 f = p[c];
            x[4 * c] = f.x;
            x[4 * c + 1] = f.y;
            x[4 * c + 2] = f.z;
            x[4 * c + 3] = f.w;
        }
    }
}

// #{j : p[j] < a} for the 2^(b-1) - 1 ascending positive thresholds p.
template <int BITS>
__device__ __forceinline__ uint32_t count_below(float a, const float (&p)[8]) {
    // binary search over the sorted thresholds (same count as a linear scan)
    if constexpr (BITS == 4) {
        const bool t1 = a > p[3];
        const float q2 = t1 ? p[5] : p[1];
        const float hi3 = t1 ? p[6] : p[2];
        const float lo3 = t1 ? p[4] : p[0];
        const bool t2 = a > q2;
        const float q3 = t2 ? hi3 : lo3;
        const bool t3 = a > q3;
        return (t1 ? 4u : 0u) + (t3 ? 1u : 0u) + (t2 ? 2u : 0u);
    } else if constexpr (BITS == 3) {
        const bool t1 = a > p[1];
        const bool t2 = a > (t1 ? p[2] : p[0]);
        return (t1 ? 2u : 0u) + (t2 ? 1u : 0u);
    } else {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < (1 << (BITS - 1)) - 1; ++j) c += a > p[j] ? 1u : 0u;
        return c;
    }
}

template <int D, int BITS, bool BF16>
__global__ __launch_bounds__(256) void encode_kernel(const dev_tables t, const encode_args a, const grid_index gi,
                                                     const uint32_t nvec) {
    constexpr int LPV = D / 32;
    constexpr int VPB = 256 / LPV;
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    constexpr uint32_t kAll = (1u << BITS) - 1;
    const int tid = threadIdx.x;
    const int blk = tid % LPV;
    const uint32_t d1w = t.d1[blk];
    const uint32_t d2w = t.d2[blk];
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = j < int(kHalf) - 1 ? t.th[kHalf + j] : 0.f;
    // D1 as an XOR of the packed words: all BITS bits of code e when d1_e = -1
    // (also folds in the constant XOR 2^(b-1) of every code)
    uint32_t xm[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) xm[k] = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const uint32_t f = (((d1w >> e) & 1) ? kAll : 0u) ^ kHalf;
        const int bit = BITS * e;
        xm[bit >> 5] |= f << (bit & 31);
        if ((bit & 31) + BITS > 32) xm[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
    }

    // pack(2^(b-1) - 1): the code of every coordinate of a zero vector
    uint32_t zero_code[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) zero_code[k] = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int bit = BITS * e;
        zero_code[bit >> 5] |= (kHalf - 1) << (bit & 31);
        if ((bit & 31) + BITS > 32) zero_code[(bit >> 5) + 1] |= (kHalf - 1) >> (32 - (bit & 31));
    }
    // D2 as sign-bit XORs on the loaded bf16 pairs (bit 15: even, bit 31: odd)
    uint32_t m2[BF16 ? 16 : 1];
    if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) m2[j] = (((d2w >> (2 * j)) & 1) << 15) | (((d2w >> (2 * j + 1)) & 1) << 31);
    }

    for (uint32_t base = blockIdx.x * VPB; base < nvec; base += gridDim.x * VPB) {
        const uint32_t v = base + tid / LPV;
        const bool valid = v < nvec;
        int64_t xoff, pv;
        vector_offsets(valid ? v : nvec - 1, a, gi, xoff, pv);

        float x[32];
        bool flipped = false;
        if constexpr (BF16) {
            const uint4 * src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + xoff + blk * 32);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 q = src[c];
                const uint32_t ws[4] = {q.x ^ m2[4 * c], q.y ^ m2[4 * c + 1], q.z ^ m2[4 * c + 2], q.w ^ m2[4 * c + 3]};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[8 * c + 2 * j] = bf16_lo(ws[j]);
                    x[8 * c + 2 * j + 1] = bf16_hi(ws[j]);
                }
            }
            flipped = true;
        } else {
            load_block<BF16>(a, xoff + blk * 32, x);
        }

        // norm of the input vector, float64 accumulation
        double nsq = 0.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) nsq = fma(double(x[e]), double(x[e]), nsq);
        nsq = group_sum<LPV>(nsq);
        const double n = sqrt(nsq);
        if (valid && blk == 0) a.out.norms[pv] = half_bits_rne(n);

        // keep the fp32 transform in range: scale by a power of two (exact)
        float nf = static_cast<float>(n);
        if (n > 0.0 && !(n >= 0x1p-60 && n <= 0x1p60)) {
            const int e = ilogb(n);
            const float sc = ldexpf(1.f, -e);
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] *= sc;
            nf = static_cast<float>(ldexp(n, -e));
        }

        // y = H . D2 . x (unnormalised Hadamard);  z = D1 . y / n
        if (!flipped) {
#pragma unroll
            for (int e = 0; e < 32; ++e)
                if ((d2w >> e) & 1) x[e] = -x[e];
        }
        lane_fwht(x);
        cross_lane_fwht<LPV>(x, blk);

        // code(y/n) = count_below(|y|/n) XOR 2^(b-1) XOR (y < 0 ? 2^b - 1 : 0):
        // the counts and the sign fields are packed separately, then XORed
        float T[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) T[j] = p[j] * nf;
        uint32_t w[BITS], ng[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = ng[k] = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const uint32_t c = count_below<BITS>(fabsf(x[e]), T);
            const uint32_t neg = static_cast<uint32_t>(__float_as_int(x[e]) >> 31);  // all ones if y < 0
            const int bit = BITS * e;
            w[bit >> 5] |= c << (bit & 31);
            ng[bit >> 5] = ((neg & (kAll << (bit & 31))) | (ng[bit >> 5] & ~(kAll << (bit & 31))));
            if ((bit & 31) + BITS > 32) {
                w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
                const uint32_t m = kAll >> (32 - (bit & 31));
                ng[(bit >> 5) + 1] = (neg & m) | (ng[(bit >> 5) + 1] & ~m);
            }
        }
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = n > 0.0 ? w[k] ^ ng[k] ^ xm[k] : zero_code[k];
        if (valid) {
            uint32_t * dst = reinterpret_cast<uint32_t *>(a.out.codes + pv * (D * BITS / 8)) + blk * BITS;
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[k] = w[k];
        }
    }
}

template <int D, int BITS, bool BF16>
__global__ __launch_bounds__(256) void encode_qjl_kernel(const dev_tables t, const encode_args a,
                                                         const grid_index gi, const uint32_t nvec) {
    constexpr int LPV = D / 32;
    constexpr int VPB = 256 / LPV;
    constexpr int NT = (1 << BITS) - 1;
    const int tid = threadIdx.x;
    const int blk = tid % LPV;
    const uint32_t d1w = t.d1[blk];
    const uint32_t d2w = t.d2[blk];
    float th[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) th[k] = t.th[k];

    for (uint32_t base = blockIdx.x * VPB; base < nvec; base += gridDim.x * VPB) {
        const uint32_t v = base + tid / LPV;
        const bool valid = v < nvec;
        int64_t xoff, pv;
        vector_offsets(valid ? v : nvec - 1, a, gi, xoff, pv);

        float xf[32];
        load_block<BF16>(a, xoff + blk * 32, xf);
        double x[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = xf[e];

        // norm of the input vector, float64 accumulation
        double nsq = 0.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) nsq = fma(x[e], x[e], nsq);
        nsq = group_sum<LPV>(nsq);
        const double n = sqrt(nsq);
        if (valid && blk == 0) a.out.norms[pv] = half_bits_rne(n);

        // y = H . D2 . x  (unnormalised Hadamard)
#pragma unroll
        for (int e = 0; e < 32; ++e)
            if ((d2w >> e) & 1) x[e] = -x[e];
        lane_fwht(x);
        cross_lane_fwht<LPV>(x, blk);

        // z = sqrt(d) * R x / n = D1 . y / n ;  code = #{k : th_k < z}
        const double inv_n = n > 0.0 ? 1.0 / n : 0.0;
        uint32_t w[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = 0;
        uint32_t codes[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            double z = x[e] * inv_n;
            if ((d1w >> e) & 1) z = -z;
            x[e] = z;
            uint32_t c = 0;
#pragma unroll
            for (int k = 0; k < NT; ++k) c += (z > static_cast<double>(th[k])) ? 1u : 0u;
            codes[e] = c;
            const int bit = BITS * e;
            w[bit >> 5] |= c << (bit & 31);
            if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
        }
        if (valid) {
            uint32_t * dst = reinterpret_cast<uint32_t *>(a.out.codes + pv * (D * BITS / 8)) + blk * BITS;
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[k] = w[k];
        }

        // rho = (z - c[code]) / sqrt(d); gamma = ||rho||; signs of S rho
        const double rs = 1.0 / sqrt(static_cast<double>(D));
        float rho[32];
        double gsq = 0.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const double rr = (x[e] - static_cast<double>(t.cb[codes[e]])) * rs;
            gsq = fma(rr, rr, gsq);
            rho[e] = static_cast<float>(rr);
        }
        gsq = group_sum<LPV>(gsq);
        if (valid && blk == 0) a.out.rnorms[pv] = half_bits_rne(sqrt(gsq));
        // m == d rows: lane blk owns rows 32*blk .. 32*blk+31
        uint32_t bits = 0;
        for (int l = 0; l < D; ++l) {
            const float4 * srow = reinterpret_cast<const float4 *>(t.S + int64_t(l) * D + blk * 32);
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 s4 = srow[c];
                acc = fmaf(s4.x, rho[4 * c], acc);
                acc = fmaf(s4.y, rho[4 * c + 1], acc);
                acc = fmaf(s4.z, rho[4 * c + 2], acc);
                acc = fmaf(s4.w, rho[4 * c + 3], acc);
            }
            acc = group_sum<LPV>(acc);
            if ((l >> 5) == blk && acc > 0.f) bits |= 1u << (l & 31);
        }
        if (valid) reinterpret_cast<uint32_t *>(a.out.signs + pv * (D / 8))[blk] = bits;
    }
}

template <int D, int BITS, bool QJL>
hipError_t launch_encode_dtype(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    constexpr int VPB = 256 / (D / 32);
    int64_t blocks = (int64_t(nvec) + VPB - 1) / VPB;
    if (blocks > 256 * 16) blocks = 256 * 16;
    const grid_index gi{make_fastdiv(static_cast<uint32_t>(a.n2)), make_fastdiv(static_cast<uint32_t>(a.n1))};
    const bool bf16 = a.dtype == TQ_DTYPE_BF16;
    if constexpr (QJL) {
        if (bf16)
            hipLaunchKernelGGL((encode_qjl_kernel<D, BITS, true>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
        else
            hipLaunchKernelGGL((encode_qjl_kernel<D, BITS, false>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    } else {
        if (bf16)
            hipLaunchKernelGGL((encode_kernel<D, BITS, true>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
        else
            hipLaunchKernelGGL((encode_kernel<D, BITS, false>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_encode_d(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    switch (t.bits * 2 + (t.qjl ? 1 : 0)) {
        case 4: return launch_encode_dtype<D, 2, false>(t, a, nvec, s);
        case 5: return launch_encode_dtype<D, 2, true>(t, a, nvec, s);
        case 6: return launch_encode_dtype<D, 3, false>(t, a, nvec, s);
        case 7: return launch_encode_dtype<D, 3, true>(t, a, nvec, s);
        case 8: return launch_encode_dtype<D, 4, false>(t, a, nvec, s);
        case 9: return launch_encode_dtype<D, 4, true>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool encode_grid_supported(const encode_args & a) {
    const int64_t nvec = a.n0 * a.n1 * a.n2;
    return nvec < (int64_t(1) << 32) && a.n1 < (int64_t(1) << 32) && a.n2 < (int64_t(1) << 32);
}

hipError_t launch_encode(const dev_tables & t, const encode_args & a, hipStream_t s) {
    const uint32_t nvec = static_cast<uint32_t>(a.n0 * a.n1 * a.n2);
    switch (t.d) {
        case 32: return launch_encode_d<32>(t, a, nvec, s);
        case 64: return launch_encode_d<64>(t, a, nvec, s);
        case 128: return launch_encode_d<128>(t, a, nvec, s);
        case 256: return launch_encode_d<256>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
