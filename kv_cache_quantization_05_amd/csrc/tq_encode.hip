// Encode kernel: norm -> rotation -> scalar codebook -> packing -> QJL.
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
// The rotation and z are evaluated in double (full-rate on CDNA4 vector
// ALUs), so codes and fp16 norms agree with a float64 evaluation except
// within ~1e-15 of a threshold or an fp16 rounding midpoint.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

template <int LPV>
__device__ __forceinline__ void cross_lane_fwht(double (&x)[32], int blk) {
    // Butterflies across the lanes of one vector (lane index bits = the high
    // coordinate bits).  The lower-index partner keeps a + b, the other a - b.
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if constexpr (LPV >= 2) {
            double o = lane_xor<1>(x[e]);
            x[e] = (blk & 1) ? o - x[e] : x[e] + o;
        }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if constexpr (LPV >= 4) {
            double o = lane_xor<2>(x[e]);
            x[e] = (blk & 2) ? o - x[e] : x[e] + o;
        }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if constexpr (LPV >= 8) {
            double o = lane_xor<4>(x[e]);
            x[e] = (blk & 4) ? o - x[e] : x[e] + o;
        }
    }
}

template <int D, int BITS, bool QJL, bool BF16>
__global__ __launch_bounds__(256) void encode_kernel(const dev_tables t, const encode_args a,
                                                     const int64_t nvec) {
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

    for (int64_t base = int64_t(blockIdx.x) * VPB; base < nvec; base += int64_t(gridDim.x) * VPB) {
        const int64_t v = base + tid / LPV;
        const bool valid = v < nvec;
        const int64_t vv = valid ? v : nvec - 1;
        const int64_t i2 = vv % a.n2;
        const int64_t r = vv / a.n2;
        const int64_t i1 = r % a.n1;
        const int64_t i0 = r / a.n1;
        const int64_t xoff = i0 * a.xs0 + i1 * a.xs1 + i2 * a.xs2 + blk * 32;
        const int64_t pv = i0 * a.out.stride[0] + i1 * a.out.stride[1] + i2 * a.out.stride[2];

        double x[32];
        if constexpr (BF16) {
            const uint4 * p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + xoff);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint4 w = p[c];
                uint32_t ws[4] = {w.x, w.y, w.z, w.w};
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
                float4 f = p[c];
                x[4 * c] = f.x;
                x[4 * c + 1] = f.y;
                x[4 * c + 2] = f.z;
                x[4 * c + 3] = f.w;
            }
        }

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
#pragma unroll
        for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                if ((e & h) == 0) {
                    double p0 = x[e], p1 = x[e + h];
                    x[e] = p0 + p1;
                    x[e + h] = p0 - p1;
                }
            }
        }
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

        if constexpr (QJL) {
            // rho = (z - c[code]) / sqrt(d); gamma = ||rho||; signs of S rho
            const double rs = 1.0 / sqrt(static_cast<double>(D));
            float rho[32];
            double gsq = 0.0;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                double rr = (x[e] - static_cast<double>(t.cb[codes[e]])) * rs;
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
                    float4 s4 = srow[c];
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
}

template <int D, int BITS, bool QJL>
hipError_t launch_encode_dtype(const dev_tables & t, const encode_args & a, int64_t nvec,
                               hipStream_t s) {
    constexpr int VPB = 256 / (D / 32);
    int64_t blocks = (nvec + VPB - 1) / VPB;
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (a.dtype == TQ_DTYPE_BF16)
        hipLaunchKernelGGL((encode_kernel<D, BITS, QJL, true>), dim3(blocks), dim3(256), 0, s, t, a, nvec);
    else
        hipLaunchKernelGGL((encode_kernel<D, BITS, QJL, false>), dim3(blocks), dim3(256), 0, s, t, a, nvec);
    return hipGetLastError();
}

template <int D>
hipError_t launch_encode_d(const dev_tables & t, const encode_args & a, int64_t nvec, hipStream_t s) {
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

hipError_t launch_encode(const dev_tables & t, const encode_args & a, hipStream_t s) {
    const int64_t nvec = a.n0 * a.n1 * a.n2;
    switch (t.d) {
        case 32: return launch_encode_d<32>(t, a, nvec, s);
        case 64: return launch_encode_d<64>(t, a, nvec, s);
        case 128: return launch_encode_d<128>(t, a, nvec, s);
        case 256: return launch_encode_d<256>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
