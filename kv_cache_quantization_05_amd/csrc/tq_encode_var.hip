// Encode kernels for the layout and rotation variants.
//
//  * encode_var_kernel: the structured rotation D1.H.D2 with one fp16 norm
//    per 32-code block of the rotated vector (the 3.5-bit turbo3 layout,
//    [TQ+ guide] §1.2) and/or the norm correction named in [TQ+ guide] §11.
//    Lane per 32-coordinate block, the rotation in double: a block norm is a
//    norm of rotated coordinates, and it must round to the same fp16 as a
//    float64 evaluation does, so the rotation cannot be fp32 here.  A lane
//    owns exactly one block, so its block norm is lane-local.
//  * encode_haar_kernel: the dense rotation y = Q x ([TQ+ guide] §3-§4: the
//    O(d^2) rotation from a seeded QR) as a real dense contraction on the
//    16x16x32 fp16 matrix cores: A = 16 Q split into fp16 hi + lo (staged in
//    LDS for d <= 128), B = the inputs scaled by a power of two so that the
//    largest coordinate lies in [2^14, 2^15) and split into fp16 hi (+ lo
//    for fp32 inputs; bf16 values are exact in fp16 after the scaling),
//    fp32 accumulation: about 22 bits, so z is within ~1e-6 of its float64
//    value.  One norm per vector (of x, accumulated in double).
#include "tq_device.h"
#include "tq_encode_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Structured rotation, block norms and/or norm correction (float64).

template <int D, int BITS, bool BF16, bool BLOCKN, bool CORR>
__global__ __launch_bounds__(256) void encode_var_kernel(const dev_tables t, const encode_args a,
                                                         const grid_index gi, const uint32_t nvec) {
    constexpr int LPV = D / 32;
    constexpr int VPB = 256 / LPV;
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    constexpr int NN = BLOCKN ? D / 32 : 1;          // norms per vector
    constexpr double kGroupLen = BLOCKN ? 32.0 : double(D);
    __shared__ double cpos[8];                         // positive centroids
    const int tid = threadIdx.x;
    const int blk = tid % LPV;
    const uint32_t d1w = t.d1[blk];
    const uint32_t d2w = t.d2[blk];
    float pth[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pth[j] = j < int(kHalf) - 1 ? t.th[kHalf + j] : 0.f;
    if (tid < int(kHalf)) cpos[tid] = static_cast<double>(t.cb[kHalf + tid]);
    __syncthreads();
    const double sqrt_len = sqrt(kGroupLen);

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
        double n = 0.0;
        if constexpr (!BLOCKN) {
            double nsq = 0.0;
#pragma unroll
            for (int e = 0; e < 32; ++e) nsq = fma(x[e], x[e], nsq);
            n = sqrt(group_sum<LPV>(nsq));               // ||x||
        }
        // x <- H D2 x (unnormalised); the rotated vector is y = D1 x / sqrt(d)
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = flip_sign(x[e], d2w, e);
        lane_fwht(x);
        cross_lane_fwht<LPV>(x, blk);
        double inv;
        if constexpr (BLOCKN) {
            double ysq = 0.0;                            // d ||y_block||^2
#pragma unroll
            for (int e = 0; e < 32; ++e) ysq = fma(x[e], x[e], ysq);
            n = sqrt(ysq / double(D));                   // ||y_block|| (D a power of two: exact scaling)
            inv = ysq > 0.0 ? sqrt(32.0) / sqrt(ysq) : 0.0;   // z = sqrt(32) y / n_block
        } else {
            inv = n > 0.0 ? 1.0 / n : 0.0;               // z = sqrt(d) y / n = D1 x / n
        }
        uint32_t w[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = 0;
        double csq = 0.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            // code = #{k : th_k < z}, decided on fp32(z) through the
            // codebook's symmetry (as in the QJL kernel)
            const float zf = static_cast<float>(flip_sign(x[e] * inv, d1w, e));
            const uint32_t kk = count_below<BITS>(fabsf(zf), pth);
            const bool zneg = !(zf > 0.f);
            const uint32_t c = zneg ? kHalf - 1 - kk : kHalf + kk;
            const int bit = BITS * e;
            w[bit >> 5] |= c << (bit & 31);
            if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
            if constexpr (CORR) csq = fma(cpos[kk], cpos[kk], csq);  // c^2 is exact in double
        }
        double stored = n;
        if constexpr (CORR) {
            if constexpr (!BLOCKN) csq = group_sum<LPV>(csq);     // exact: < 53 significant bits
            stored = n * sqrt_len / sqrt(csq);
        }
        if (valid) {
            uint32_t * dst = reinterpret_cast<uint32_t *>(a.out.codes + pv * (D * BITS / 8)) + blk * BITS;
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[k] = w[k];
            if (BLOCKN || blk == 0) a.out.norms[pv * NN + (BLOCKN ? blk : 0)] = half_bits_rne(stored);
        }
    }
}

// ---------------------------------------------------------------------------
// Dense Haar rotation on matrix cores.
//
// A wave takes 32 vectors (two 16-vector column tiles) per iteration.  For
// the 16x16x32 MFMA, lane l supplies row/column l % 16 at k-slots
// 8 (l / 16) .. + 7: as the B operand it loads coordinates 32 ks + 8 g .. + 7
// (g = l / 16) of vector l % 16 of each column tile, and as the result it
// holds rows 16 rt + 4 g + i (i = 0..3) of that vector.  Two row tiles make
// one 32-code block: lane g owns codes 4 g .. 4 g + 3 and 16 + 4 g .. + 3 of
// it, packs them at their bit offsets and the four lanes of the vector OR
// their parts together.

__device__ __forceinline__ f16x8 ld_f16x8(const uint16_t * p) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    f16x8 r;
    __builtin_memcpy(&r, &w, 16);
    return r;
}

// OR `v` (fewer than 17 bits) into the 128-bit value (lo, hi) at bit `shift`.
__device__ __forceinline__ void or_bits(uint64_t & lo, uint64_t & hi, uint64_t v, int shift) {
    if (shift < 64) {
        lo |= v << shift;
        if (shift > 48) hi |= v >> (64 - shift);
    } else {
        hi |= v << (shift - 64);
    }
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
    return (uint64_t(hi) << 32) | lo;
}

template <int D, int BITS, bool BF16, bool CORR, bool LDSQ>
__global__ __launch_bounds__(256) void encode_haar_kernel(const dev_tables t, const encode_args a,
                                                          const grid_index gi, const uint32_t nvec) {
    constexpr int KS = D / 32;                 // k-steps
    constexpr int RT = D / 16;                 // row tiles
    constexpr int CT = 2;                      // column tiles (16 vectors each) per wave
    constexpr int VPW = 16 * CT;               // vectors per wave iteration
    constexpr int RS = D + 8;                  // LDS row stride (halves): rows 16 B apart in the banks
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    __shared__ __align__(16) uint16_t qs[LDSQ ? 2 * D * RS : 8];   // [2][D][RS]: 16 Q hi, lo
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const uint16_t * qhi;
    const uint16_t * qlo;
    int qstride;
    if constexpr (LDSQ) {
        for (int i = tid; i < 2 * D * (D / 8); i += 256) {
            const int part = i / (D * (D / 8)), r = (i / (D / 8)) % D, c8 = i % (D / 8);
            *reinterpret_cast<uint4 *>(&qs[(part * D + r) * RS + 8 * c8]) =
                *reinterpret_cast<const uint4 *>(t.Q16 + int64_t(part) * D * D + int64_t(r) * D + 8 * c8);
        }
        __syncthreads();
        qhi = qs;
        qlo = qs + D * RS;
        qstride = RS;
    } else {
        qhi = t.Q16;
        qlo = t.Q16 + D * D;
        qstride = D;
    }
    float pth[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pth[j] = j < int(kHalf) - 1 ? t.th[kHalf + j] : 0.f;
    double cpos2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cpos2[j] = j < int(kHalf) ? double(t.cb[kHalf + j]) * double(t.cb[kHalf + j]) : 0.0;
    const double sqrt_d = sqrt(double(D));

    for (uint32_t base = (blockIdx.x * 4 + wave) * VPW; base < nvec; base += gridDim.x * 4 * VPW) {
        // ---- load this lane's coordinates of its vector in each column tile
        f16x8 xh[CT][KS], xl[BF16 ? 1 : CT][BF16 ? 1 : KS];
        float inv[CT];
        double nrm[CT];
        int64_t pvs[CT];
        bool valid[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint32_t v = base + 16 * ct + n16;
            valid[ct] = v < nvec;
            int64_t xoff;
            vector_offsets(valid[ct] ? v : nvec - 1, a, gi, xoff, pvs[ct]);
            float xv[KS][8];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int64_t off = xoff + 32 * ks + 8 * g;
                if constexpr (BF16) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + off);
                    const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xv[ks][2 * j] = bf16_lo(ws[j]);
                        xv[ks][2 * j + 1] = bf16_hi(ws[j]);
                    }
                } else {
                    const float4 * p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off);
                    const float4 f0 = p[0], f1 = p[1];
                    xv[ks][0] = f0.x; xv[ks][1] = f0.y; xv[ks][2] = f0.z; xv[ks][3] = f0.w;
                    xv[ks][4] = f1.x; xv[ks][5] = f1.y; xv[ks][6] = f1.z; xv[ks][7] = f1.w;
                }
            }
            // the vector's norm (double) and largest magnitude, over its 4 lanes
            double nsq = 0.0;
            float mx = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    nsq = fma(double(xv[ks][j]), double(xv[ks][j]), nsq);
                    mx = fmaxf(mx, fabsf(xv[ks][j]));
                }
            nsq += __shfl_xor(nsq, 16);
            nsq += __shfl_xor(nsq, 32);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            nrm[ct] = sqrt(nsq);
            // scale by 2^(14 - E), E = exponent of the largest magnitude, so it
            // lies in [2^14, 2^15): exact, and every coordinate fits fp16
            const int sh = mx > 0.f ? 14 - ilogbf(mx) : 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float s = ldexpf(xv[ks][j], sh);
                    const _Float16 h = static_cast<_Float16>(s);
                    xh[ct][ks][j] = h;
                    if constexpr (!BF16) xl[ct][ks][j] = static_cast<_Float16>(s - static_cast<float>(h));
                }
            // y_scaled = 16 2^sh y, z = sqrt(d) y / n
            inv[ct] = nrm[ct] > 0.0 ? static_cast<float>(sqrt_d / ldexp(nrm[ct], 4 + sh)) : 0.f;
        }

        double csq[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) csq[ct] = 0.0;
#pragma unroll 1
        for (int rp = 0; rp < RT / 2; ++rp) {        // row-tile pairs = 32-code blocks
            f32x4 acc[2][CT];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[h][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 16 * (2 * rp + h) + n16;
                    const f16x8 ah = ld_f16x8(qhi + row * qstride + 32 * ks + 8 * g);
                    const f16x8 al = ld_f16x8(qlo + row * qstride + 32 * ks + 8 * g);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, xh[ct][ks], acc[h][ct], 0, 0, 0);
                        acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, xh[ct][ks], acc[h][ct], 0, 0, 0);
                        if constexpr (!BF16)
                            acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, xl[ct][ks], acc[h][ct], 0, 0, 0);
                    }
                }
            }
            // quantise: lane g holds codes 4 g + i (h = 0) and 16 + 4 g + i (h = 1)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                uint64_t lo = 0, hi = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t chunk = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float z = acc[h][ct][i] * inv[ct];
                        const uint32_t kk = count_below<BITS>(fabsf(z), pth);
                        const uint32_t c = z > 0.f ? kHalf + kk : kHalf - 1 - kk;
                        chunk |= c << (BITS * i);
                        if constexpr (CORR) csq[ct] += cpos2[kk];
                    }
                    or_bits(lo, hi, chunk, BITS * (16 * h + 4 * g));
                }
                lo |= shfl_xor64(lo, 16);
                hi |= shfl_xor64(hi, 16);
                lo |= shfl_xor64(lo, 32);
                hi |= shfl_xor64(hi, 32);
                if (g == 0 && valid[ct]) {
                    uint32_t * dst = reinterpret_cast<uint32_t *>(a.out.codes + pvs[ct] * (D * BITS / 8)) + rp * BITS;
                    dst[0] = static_cast<uint32_t>(lo);
                    if constexpr (BITS >= 2) dst[1] = static_cast<uint32_t>(lo >> 32);
                    if constexpr (BITS >= 3) dst[2] = static_cast<uint32_t>(hi);
                    if constexpr (BITS >= 4) dst[3] = static_cast<uint32_t>(hi >> 32);
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            double stored = nrm[ct];
            if constexpr (CORR) {
                double c = csq[ct];
                c += __shfl_xor(c, 16);
                c += __shfl_xor(c, 32);
                stored = nrm[ct] * sqrt_d / sqrt(c);
            }
            if (g == 0 && valid[ct]) a.out.norms[pvs[ct]] = half_bits_rne(stored);
        }
    }
}

template <int D, int BITS, bool BF16>
hipError_t launch_var_b(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    const grid_index gi{make_fastdiv(static_cast<uint32_t>(a.n2)), make_fastdiv(static_cast<uint32_t>(a.n1))};
    if (t.haar) {
        constexpr bool LDSQ = D <= 128;
        const size_t lds = 0;
        int64_t blocks = (int64_t(nvec) + 127) / 128;            // 4 waves x 32 vectors
        const int64_t cap = int64_t(current_cu_count()) * (LDSQ && D == 128 ? 2 : 4);
        if (blocks > cap) blocks = cap;
        if (t.norm_corr)
            hipLaunchKernelGGL((encode_haar_kernel<D, BITS, BF16, true, LDSQ>), dim3(blocks), dim3(256), lds, s, t, a, gi, nvec);
        else
            hipLaunchKernelGGL((encode_haar_kernel<D, BITS, BF16, false, LDSQ>), dim3(blocks), dim3(256), lds, s, t, a, gi, nvec);
        return hipGetLastError();
    }
    constexpr int VPB = 256 / (D / 32);
    int64_t blocks = (int64_t(nvec) + VPB - 1) / VPB;
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (t.norm_group && t.norm_corr)
        hipLaunchKernelGGL((encode_var_kernel<D, BITS, BF16, true, true>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    else if (t.norm_group)
        hipLaunchKernelGGL((encode_var_kernel<D, BITS, BF16, true, false>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    else
        hipLaunchKernelGGL((encode_var_kernel<D, BITS, BF16, false, true>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    return hipGetLastError();
}

template <int D>
hipError_t launch_var_d(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    const bool bf16 = a.dtype == TQ_DTYPE_BF16;
    switch (t.bits) {
        case 2: return bf16 ? launch_var_b<D, 2, true>(t, a, nvec, s) : launch_var_b<D, 2, false>(t, a, nvec, s);
        case 3: return bf16 ? launch_var_b<D, 3, true>(t, a, nvec, s) : launch_var_b<D, 3, false>(t, a, nvec, s);
        case 4: return bf16 ? launch_var_b<D, 4, true>(t, a, nvec, s) : launch_var_b<D, 4, false>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Encode for contexts with the Haar rotation, block norms or norm correction.
hipError_t launch_encode_variant(const dev_tables & t, const encode_args & a, hipStream_t s) {
    const uint32_t nvec = static_cast<uint32_t>(a.n0 * a.n1 * a.n2);
    switch (t.d) {
        case 32: return launch_var_d<32>(t, a, nvec, s);
        case 64: return launch_var_d<64>(t, a, nvec, s);
        case 128: return launch_var_d<128>(t, a, nvec, s);
        case 256: return launch_var_d<256>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
