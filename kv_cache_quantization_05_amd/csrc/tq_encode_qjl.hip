// Encode kernel for QJL keys with bf16 input and d = 64 or 128: the
// rotation and the residual sketch both on matrix cores.  Steps as the pages
// order them: the norm and the structured rotation D1.H.D2 ([TQ+ guide]
// §4, §5.1), the scalar codebook and packing ([TQ+ guide] §5.1-§5.2), and the
// 1-bit sketch of the residual with its norm ([Orión plan] Fase 3;
// [TQ explainer] §2.2).
//
// Accuracy.  Besides the codes, a QJL key stores gamma = ||z - c[code]|| /
// sqrt(d) as fp16, which must round as a float64 evaluation does, and the
// residual feeds the sketch; z = H D2 x / n (D1 aside) is needed well beyond
// fp32.  The rotation is made exact on bf16 matrix cores by splitting each
// vector's coordinates into three exponent bands relative to E, the
// exponent of its largest |x| (the elements are masked, never changed, so
// each band is an exact bf16 operand with its own fp32 accumulation):
//   band 1, |x| in [2^(E-9), 2^(E+1)): multiples of 2^(E-16); every partial
//     sum of up to 128 of them is a multiple of 2^(E-16) below 2^(E+8), i.e.
//     fewer than 2^24 units, so it is exact in fp32 in any order;
//   band 2, |x| in [2^(E-19), 2^(E-9)): multiples of 2^(E-26) below
//     2^(E-9), exact the same way;
//   band 3, the rest (below 2^(E-19), rare): rounded, at most
//     127 * 2^-23 * sum|x_j| <= 2^(E-28) per output (2^-23 also covers
//     truncating adders).  Its products are skipped for a wave without such
//     elements.
// y = y1 + y2 + y3 is summed in float64 (y1 + y2 exactly).  The norm comes
// from ||y||^2 = d ||x||^2, and z, the residual and gamma^2 are formed in
// float64.  With band-3 elements both the norm and gamma are known to within
// 2^-27 (relative, resp. absolute, as ||z|| = sqrt(d)), otherwise to within
// float64 rounding.  The fp16 of each is taken from the computed value when
// no fp16 rounding midpoint lies within that bound; otherwise, and outside
// fp16's normal range, the wave recomputes it from the input by float64
// butterflies (rare: about one vector in 10^4 with band-3 elements).
// Vectors whose largest |x| lies outside [2^-60, 2^101) are first rescaled
// by a power of two, which changes neither z, the codes, gamma nor the
// signs.
//
// Layout.  As in the MSE matrix-core kernel, a wave takes 16 vectors; lane l
// loads coordinates 8 g .. 8 g + 7 (g = l / 16) of each 32-block of vector
// n = l % 16 and, through the row order of the +-1 A operand, receives the
// same output coordinates, 32 b + 8 g + j (j < 8).  The codes are decided on
// fp32(z) by the wave-mask quantiser; D1 enters as an XOR of the packed
// codes and as a sign on S's columns, so the residual r' = z' - c' stays in
// the H D2 frame (z' = D1 z) and S D1 r' = S r.  Those coordinates are the
// k-slots 8 g .. 8 g + 7 of k-step b of the sketch's B operand, so the
// residual (fp16 hi + lo) goes to the sketch from registers.  S D1 is
// staged in LDS once per workgroup as fp16 hi + lo A fragments whose rows
// are permuted so that each lane receives d/4 consecutive sketch rows: its
// sign bits are one contiguous piece of the sign plane.
#include <atomic>

#include "tq_device.h"
#include "tq_encode_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 0xFFFF in each 16-bit half of a that is below the same half of t (both
// halves of both in [0, 0x7FFF])
__device__ __forceinline__ uint32_t below_mask(uint32_t a, uint32_t t) {
    i16x2 x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &t, 4);
    const i16x2 m = (x - y) >> 15;
    uint32_t r;
    __builtin_memcpy(&r, &m, 4);
    return r;
}

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    u16x2 x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    const u16x2 m = __builtin_elementwise_max(x, y);
    uint32_t r;
    __builtin_memcpy(&r, &m, 4);
    return r;
}

// fp16 (round to nearest, ties to even) of a value known as v to within err
// (err far below half an fp16 ulp).  Returns false when v is outside fp16's
// normal range or an fp16 rounding midpoint lies within err of v; otherwise
// sets bits to the rounding of every value within err of v.
__device__ __forceinline__ bool fp16_of_bracketed(double v, double err, uint16_t & bits) {
    const float vf = static_cast<float>(v);
    if (!(vf >= 0x1p-14f && vf < 65504.f)) return false;
    const uint32_t base = __float_as_uint(vf) & ~0x1FFFu;  // the fp16 value at or below vf
    const double mid = static_cast<double>(__uint_as_float(base | 0x1000u));
    const uint16_t lo = __builtin_bit_cast(unsigned short, static_cast<_Float16>(__uint_as_float(base)));
    bits = v < mid ? lo : static_cast<uint16_t>(lo + 1);
    return fabs(v - mid) > err;
}

// r - (fp16 half of hp, low or high) in one mixed-precision FMA (plain ALU;
// the compiler forms it only with fp32 denormals flushed)
__device__ __forceinline__ float sub_half_lo(float r, uint32_t hp) {
    float d;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(hp), "v"(r));
    return d;
}
__device__ __forceinline__ float sub_half_hi(float r, uint32_t hp) {
    float d;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(hp), "v"(r));
    return d;
}

// fp16 hi + lo pairs of (a, b): hi truncated, lo the truncated remainder
// (a ~ hi + lo to about 2^-20 relative)
__device__ __forceinline__ void split_pair(float a, float b, uint32_t & hi, uint32_t & lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sub_half_lo(a, hi), sub_half_hi(b, hi)));
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const int64_t b = __double_as_longlong(v);
    const int lo = __shfl_xor(static_cast<int>(b), m);
    const int hi = __shfl_xor(static_cast<int>(b >> 32), m);
    return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Sum over the 4 lanes of a vector (lanes n, n + 16, n + 32, n + 48), the
// same bits in each.
__device__ __forceinline__ double vec_sum(double v) {
    v += shfl_xor_f64(v, 16);
    return v + shfl_xor_f64(v, 32);
}

// Two waves per SIMD: the 64 KB of S fragments allow two workgroups per CU.
template <int D, int BITS, bool FLAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void encode_qjl_mfma_kernel(const dev_tables t, const encode_args a,
                                                              const grid_index gi, const uint32_t nvec) {
    constexpr int NB = D / 32;
    constexpr int RT = D / 16;              // 16-row tiles of S (m = d)
    constexpr int NF = RT * NB * 2 * 64;    // 16-byte LDS entries of the S fragments
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    constexpr uint32_t kAll = (1u << BITS) - 1;
    static_assert(NB == 2 || NB == 4, "d = 64 or 128");
    __shared__ uint4 sfrag[NF];
    __shared__ double cpos[8];
    __shared__ double cneg[16];  // by code field [sign, k]: -(sign ? -c_pos[k] : c_pos[k])
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;

    // S D1 as A fragments: entry ((rt NB + ks) 2 + part) 64 + l holds columns
    // 32 ks + 8 (l / 16) .. +7 of row 4 RT (m / 4) + 4 rt + m % 4, m = l % 16,
    // of the fp16 hi (part 0) or lo (part 1) half; D1 flips column signs.
    // The product's lane (n, g) then holds rows 4 RT g + 4 rt + i of vector n.
    for (int f = tid; f < NF; f += 256) {
        const int l = f & 63, part = (f >> 6) & 1, rk = f >> 7;
        const int ks = rk % NB, rt = rk / NB;
        const int m = l & 15, gg = l >> 4;
        const int row = 4 * RT * (m >> 2) + 4 * rt + (m & 3);
        const int col = 32 * ks + 8 * gg;
        uint4 v = *reinterpret_cast<const uint4 *>(t.S16 + int64_t(part) * D * D + row * D + col);
        const uint32_t d1b = t.d1[ks] >> (8 * gg);
        v.x ^= ((d1b & 1u) << 15) | (((d1b >> 1) & 1u) << 31);
        v.y ^= (((d1b >> 2) & 1u) << 15) | (((d1b >> 3) & 1u) << 31);
        v.z ^= (((d1b >> 4) & 1u) << 15) | (((d1b >> 5) & 1u) << 31);
        v.w ^= (((d1b >> 6) & 1u) << 15) | (((d1b >> 7) & 1u) << 31);
        sfrag[f] = v;
    }
    if (tid < int(kHalf)) cpos[tid] = static_cast<double>(t.cb[kHalf + tid]);
    if (tid < int(2 * kHalf)) {
        const double cm = static_cast<double>(t.cb[kHalf + (tid & (kHalf - 1))]);
        cneg[tid] = (tid & kHalf) ? cm : -cm;
    }

    // A operand of output half tt: row m holds H_32 row 8 (m / 4) + 4 tt + m % 4;
    // this lane supplies row n, columns 8 g .. 8 g + 7; [1]: the negation
    bf16x8 hA[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int row = 8 * (n >> 2) + 4 * tt + (n & 3);
        uint32_t p[4], q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 8 * g + 2 * j;
            const uint32_t lo = (__builtin_popcount(row & c0) & 1) ? 0xBF80u : 0x3F80u;  // -1 / +1
            const uint32_t hi = (__builtin_popcount(row & (c0 + 1)) & 1) ? 0xBF80u : 0x3F80u;
            p[j] = lo | (hi << 16);
            q[j] = p[j] ^ 0x80008000u;
        }
        hA[tt][0] = as_bf16x8(p);
        hA[tt][1] = as_bf16x8(q);
    }
    // D2's signs for the lane's input columns (bit 15: even, bit 31: odd)
    uint32_t m2[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 8 * g + 2 * j;
            m2[b][j] = (((t.d2[b] >> e) & 1) << 15) | (((t.d2[b] >> (e + 1)) & 1) << 31);
        }
    // D1 (all bits of a code whose z changes sign) as XORs of the lane's
    // 8-code chunks; and the chunk of a zero vector
    uint32_t xm[NB], zero_chunk = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        xm[b] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) xm[b] |= (((t.d1[b] >> (8 * g + j)) & 1) ? kAll : 0u) << (BITS * j);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) zero_chunk |= (kHalf - 1) << (BITS * j);
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = j < int(kHalf) - 1 ? t.th[kHalf + j] : 0.f;
    __syncthreads();

    // each wave takes 16 vectors per iteration, the next iteration's inputs
    // loaded while the current ones are processed (lanes past the end load
    // the last vector again)
    const uint32_t stride = gridDim.x * 64;
    uint32_t wn[NB][4];
    int64_t pv_next = 0;
    bool valid_next = false;
    auto load_inputs = [&](uint64_t bs) {
        const uint64_t v = bs + n;
        valid_next = v < nvec;
        int64_t xoff;
        vector_offsets<FLAT>(valid_next ? static_cast<uint32_t>(v) : nvec - 1, a, gi, xoff, pv_next);
        const uint16_t * src = static_cast<const uint16_t *>(a.x) + xoff + 8 * g;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint4 q = *reinterpret_cast<const uint4 *>(src + 32 * b);
            wn[b][0] = q.x;
            wn[b][1] = q.y;
            wn[b][2] = q.z;
            wn[b][3] = q.w;
        }
    };
    uint64_t base = blockIdx.x * 64 + wave * 16;
    if (base < nvec) load_inputs(base);
    for (; base < nvec; base += stride) {
        const bool valid = valid_next;
        const int64_t pv = pv_next;
        // D2 x: sign flips of the loaded bf16 pairs
        uint32_t w[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[b][j] = wn[b][j] ^ m2[b][j];
        load_inputs(base + stride);

        // exponent field of the vector's largest |x|
        auto max_field = [&]() {
            uint32_t mx = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) mx = max_u16x2(mx, w[b][j] & 0x7FFF7FFFu);
            uint32_t m1 = max(mx & 0xFFFFu, mx >> 16);
            m1 = max(m1, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m1), 16)));
            m1 = max(m1, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m1), 32)));
            return m1 >> 7;
        };
        uint32_t ef = max_field();
        // largest |x| outside [2^-60, 2^101) (or only subnormal coordinates):
        // rescale by 2^-e, exact for bf16 apart from coordinates below 2^-126
        // of the new scale
        int e = 0;
        const bool far = ef < 67u || ef > 227u;
        if (__any(far)) {
            if (far) {
                e = ef == 0 ? -133 : int(ef) - 127;
                const float s1 = ldexpf(1.f, -(e / 2)), s2 = ldexpf(1.f, -(e - e / 2));
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wj = opaque(w[b][j]);
                        const uint32_t lo = __float_as_uint(bf16_lo(wj) * s1 * s2) >> 16;
                        const uint32_t hi = __float_as_uint(bf16_hi(wj) * s1 * s2) & 0xFFFF0000u;
                        w[b][j] = lo | hi;
                    }
            }
            ef = max_field();
        }

        // the three bands as bf16 operands
        const uint32_t t1 = ((ef - 9u) << 7) * 0x10001u;
        const uint32_t t2 = ((ef - 19u) << 7) * 0x10001u;
        bf16x8 xb1[NB], xb2[NB], xb3[NB];
        uint32_t any3 = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint32_t p1[4], p2[4], p3[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t aw = w[b][j] & 0x7FFF7FFFu;
                const uint32_t l1 = below_mask(aw, t1), l2 = below_mask(aw, t2);
                p1[j] = w[b][j] & ~l1;
                p3[j] = w[b][j] & l2;
                p2[j] = (w[b][j] & l1) ^ p3[j];
                any3 |= aw & l2;
            }
            xb1[b] = as_bf16x8(p1);
            xb2[b] = as_bf16x8(p2);
            xb3[b] = as_bf16x8(p3);
        }
        const bool band3 = __any(any3 != 0);

        // y = H D2 x: output block bo = sum over input blocks bi of
        // (-1)^popcount(bo & bi) H_32 x_bi, per band; lane gets coordinates
        // 32 bo + 8 g + j, j = 4 tt + i
        double y[NB][8];
#pragma unroll
        for (int bo = 0; bo < NB; ++bo) {
            f32x4 u1[2], u2[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bi = 0; bi < NB; ++bi) {
                    const int sg = __builtin_popcount(bo & bi) & 1;
                    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hA[tt][sg], xb1[bi], c1, 0, 0, 0);
                    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hA[tt][sg], xb2[bi], c2, 0, 0, 0);
                }
                u1[tt] = c1;
                u2[tt] = c2;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                y[bo][j] = static_cast<double>(u1[j >> 2][j & 3]) + static_cast<double>(u2[j >> 2][j & 3]);
        }
        if (band3) {
            // (the sums pass through an empty asm so that they stay inside
            // the branch: otherwise the compiler adds -0.0 to every y when the
            // band is absent)
#pragma unroll
            for (int bo = 0; bo < NB; ++bo)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    f32x4 c3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int bi = 0; bi < NB; ++bi)
                        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hA[tt][__builtin_popcount(bo & bi) & 1], xb3[bi], c3, 0,
                                                                     0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        double v = y[bo][4 * tt + i] + static_cast<double>(c3[i]);
                        asm volatile("" : "+v"(v));
                        y[bo][4 * tt + i] = v;
                    }
                }
        }
        double nsqb[NB];  // one partial sum per block (short dependency chains)
#pragma unroll
        for (int bo = 0; bo < NB; ++bo) {
            double a0 = y[bo][0] * y[bo][0], a1 = y[bo][1] * y[bo][1];
#pragma unroll
            for (int j = 2; j < 8; j += 2) {
                a0 = fma(y[bo][j], y[bo][j], a0);
                a1 = fma(y[bo][j + 1], y[bo][j + 1], a1);
            }
            nsqb[bo] = a0 + a1;
        }
        double nsq = nsqb[0];
#pragma unroll
        for (int bo = 1; bo < NB; ++bo) nsq += nsqb[bo];
        nsq = vec_sum(nsq);
        const double nv = sqrt(nsq * (1.0 / D));  // ||x|| of the (rescaled) vector
        const double inv_n = nv > 0.0 ? 1.0 / nv : 0.0;
        uint16_t nbits = 0;
        bool n_ok = true;
        if (nv > 0.0) {
            const double ns = ldexp(nv, e);
            n_ok = fp16_of_bracketed(ns, ns * (band3 ? 0x1p-27 : 0x1p-44), nbits);
        }

        // codes and the residual r' = z' - c' (z' = D1 z), one output block
        // at a time; codes decided on |fp32(y)| against fp32(threshold * n)
        const float nf = static_cast<float>(nv);
        float T[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) T[j] = p[j] * nf;
        uint32_t cpre[NB];  // [sign, magnitude] code fields before the XORs
        double gsqb[NB];  // one partial sum per block
        uint32_t rh[NB][4], rl[NB][4];  // the residual as fp16 hi + lo pairs
        const bool any_zero = __any(nv == 0.0);
        uint8_t * const crow = a.out.codes + pv * (D * BITS / 8);
        // each 8-code chunk is built bit-serially from the top: the sign bit,
        // then each magnitude decision as a wave mask shifted in by one
        // add-with-carry (the blocks' chunks interleaved: independent chains)
#pragma unroll
        for (int bo = 0; bo < NB; ++bo) cpre[bo] = 0;
#pragma unroll
        for (int j = 7; j >= 0; --j)
#pragma unroll
            for (int bo = 0; bo < NB; ++bo) {
                uint32_t c = cpre[bo];
                const float yf = static_cast<float>(y[bo][j]);
                const float ya = fabsf(yf);
                c = __builtin_amdgcn_alignbit(c, __float_as_uint(yf), 31);
                if constexpr (BITS == 4) {
                    const bool b1 = ya > T[3];
                    const float q2 = b1 ? T[5] : T[1];
                    const float hi3 = b1 ? T[6] : T[2];
                    const float lo3 = b1 ? T[4] : T[0];
                    const bool b2 = ya > q2;
                    const bool b3 = ya > (b2 ? hi3 : lo3);
                    c = shift_in(c, __ballot(b1));
                    c = shift_in(c, __ballot(b2));
                    c = shift_in(c, __ballot(b3));
                } else if constexpr (BITS == 3) {
                    const bool b1 = ya > T[1];
                    const bool b2 = ya > (b1 ? T[2] : T[0]);
                    c = shift_in(c, __ballot(b1));
                    c = shift_in(c, __ballot(b2));
                } else {
                    c = shift_in(c, __ballot(ya > T[0]));
                }
                cpre[bo] = c;
            }
#pragma unroll
        for (int bo = 0; bo < NB; ++bo) {
            uint32_t c = cpre[bo];
            // r' = y / n - sign(y) c_pos[k] (the sign field is y's sign bit)
            float rf[8];
            double g0 = 0.0, g1 = 0.0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double r = fma(y[bo][j], inv_n, cneg[(c >> (BITS * j)) & kAll]);
                if (j & 1)
                    g1 = fma(r, r, g1);
                else
                    g0 = fma(r, r, g0);
                rf[j] = static_cast<float>(r);
            }
            gsqb[bo] = g0 + g1;
#pragma unroll
            for (int k = 0; k < 4; ++k) split_pair(rf[2 * k], rf[2 * k + 1], rh[bo][k], rl[bo][k]);
            // a zero vector: every z is 0, its code 2^(b-1) - 1 and r = +c_pos[0]
            // in every coordinate, i.e. r' = D1 c_pos[0] here
            if (any_zero) {
                if (nv == 0.0) {
                    const uint32_t c0 = __builtin_bit_cast(unsigned short, static_cast<_Float16>(t.cb[kHalf]));
                    const uint32_t d1b = opaque(t.d1[bo] >> (8 * g));
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        rh[bo][k] = (c0 ^ (((d1b >> (2 * k)) & 1u) << 15)) | ((c0 ^ (((d1b >> (2 * k + 1)) & 1u) << 15)) << 16);
                        rl[bo][k] = 0;
                    }
                }
            }
            {
                // fields are [sign, magnitude bits]: flip the magnitude bits of
                // negative coordinates and every sign bit, then D1
                constexpr uint32_t low = BITS == 2 ? 0x5555u : BITS == 3 ? 0x249249u : 0x11111111u;
                const uint32_t m = (c >> (BITS - 1)) & low;
                const uint32_t spread = m * ((1u << (BITS - 1)) - 1);
                c = nv > 0.0 ? c ^ spread ^ (xm[bo] ^ (low << (BITS - 1))) : zero_chunk;
            }
            if constexpr (BITS == 4) {
                if (valid) reinterpret_cast<uint32_t *>(crow + 16 * bo)[g] = c;
            } else if constexpr (BITS == 3) {
                // block dword g = bits 32g..32g+31 = chunk g (24 bits at 24 g) and chunk g+1
                const uint32_t nx = __shfl_down(c, 16);
                const uint32_t dw = (c >> (8 * g)) | (nx << (24 - 8 * g));
                if (valid && g < 3) reinterpret_cast<uint32_t *>(crow + 12 * bo)[g] = dw;
            } else {
                const uint32_t nx = __shfl_down(c, 16);
                if (valid && (g & 1) == 0) reinterpret_cast<uint32_t *>(crow + 8 * bo)[g >> 1] = c | (nx << 16);
            }
        }
        double gsq = gsqb[0];
#pragma unroll
        for (int bo = 1; bo < NB; ++bo) gsq += gsqb[bo];
        gsq = vec_sum(gsq);
        const double gam = sqrt(gsq * (1.0 / D));
        uint16_t gbits = 0;
        const bool g_ok = fp16_of_bracketed(gam, (band3 ? 0x1p-26 : 0.0) + 0x1p-40 * (1.0 + gam), gbits);

        // (rare) the norm or gamma not decided: float64 butterflies of D2 x in
        // this lane layout (coordinate bits 0-2: j, 3-4: g across lanes,
        // 5..: the block), then the same codes
        if (__any(!n_ok || !g_ok)) {
            double v[NB][8];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t wj = opaque(w[b][j >> 1]);
                    v[b][j] = (j & 1) ? bf16_hi(wj) : bf16_lo(wj);
                }
#pragma unroll
            for (int h = 1; h < 8; h <<= 1)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if ((j & h) == 0) {
                            const double p0 = v[b][j], p1 = v[b][j + h];
                            v[b][j] = p0 + p1;
                            v[b][j + h] = p0 - p1;
                        }
#pragma unroll
            for (int h = 1; h < NB; h <<= 1)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if ((b & h) == 0)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const double p0 = v[b][j], p1 = v[b + h][j];
                            v[b][j] = p0 + p1;
                            v[b + h][j] = p0 - p1;
                        }
            const double s16 = (g & 1) ? -1.0 : 1.0, s32 = (g & 2) ? -1.0 : 1.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v[b][j] = fma(s16, v[b][j], shfl_xor_f64(v[b][j], 16));
                    v[b][j] = fma(s32, v[b][j], shfl_xor_f64(v[b][j], 32));
                }
            double s2 = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 8; ++j) s2 = fma(v[b][j], v[b][j], s2);
            const double nx = sqrt(vec_sum(s2) * (1.0 / D));
            const double inv = nx > 0.0 ? 1.0 / nx : 0.0;
            double gs = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t kk = (cpre[b] >> (BITS * j)) & (kHalf - 1);
                    const bool neg = (cpre[b] >> (BITS * j + BITS - 1)) & 1u;
                    const double r = v[b][j] * inv - (neg ? -cpos[kk] : cpos[kk]);
                    gs = fma(r, r, gs);
                }
            gs = vec_sum(gs);
            if (!n_ok) nbits = half_bits_rne(ldexp(nx, e));
            if (!g_ok) gbits = half_bits_rne(sqrt(gs * (1.0 / D)));
        }

        // sketch h = S D1 r': three fp16 products per row tile and k-step (hi
        // hi, hi lo, lo hi), the A fragments loaded kPipe steps ahead of their
        // products (the scheduling barrier keeps the compiler from sinking each
        // load to just before its use, which exposes the LDS latency)
        constexpr int NS = NB * RT, kPipe = 4;
        f32x4 hacc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) hacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto frag = [&](int st, int part) {
            return as_f16x8(sfrag[(((st % RT) * NB + st / RT) * 2 + part) * 64 + lane]);
        };
        f16x8 fh[kPipe], fl[kPipe];
#pragma unroll
        for (int st = 0; st < kPipe; ++st) {
            fh[st] = frag(st, 0);
            fl[st] = frag(st, 1);
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int ks = st / RT, rt = st % RT;
            const f16x8 ah = fh[st % kPipe], al = fl[st % kPipe];
            if (st + kPipe < NS) {
                fh[st % kPipe] = frag(st + kPipe, 0);
                fl[st % kPipe] = frag(st + kPipe, 1);
            }
            const f16x8 bh = as_f16x8(uint4{rh[ks][0], rh[ks][1], rh[ks][2], rh[ks][3]});
            const f16x8 bl = as_f16x8(uint4{rl[ks][0], rl[ks][1], rl[ks][2], rl[ks][3]});
            hacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, hacc[rt], 0, 0, 0);
            hacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, hacc[rt], 0, 0, 0);
            hacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, hacc[rt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane (n, g) holds rows 4 RT g + 4 rt + i: bit 4 rt + i of its sign word
        // (the sign bit of h, inverted: set for h >= +0)
        uint32_t sgn = 0;
#pragma unroll
        for (int rt = RT - 1; rt >= 0; --rt)
#pragma unroll
            for (int i = 3; i >= 0; --i) sgn = __builtin_amdgcn_alignbit(sgn, __float_as_uint(hacc[rt][i]), 31);
        sgn = ~sgn;
        if (valid) {
            if (g == 0) {
                a.out.norms[pv] = nbits;
                a.out.rnorms[pv] = gbits;
            }
            if constexpr (D == 128)
                reinterpret_cast<uint32_t *>(a.out.signs + pv * 16)[g] = sgn;
            else
                reinterpret_cast<uint16_t *>(a.out.signs + pv * 8)[g] = static_cast<uint16_t>(sgn);
        }
    }
}

template <int D, int BITS>
hipError_t launch_d(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    // one round of resident workgroups striding over the vectors
    static std::atomic<int> per_cu_cache{0};  // same on every gfx950 device
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, encode_qjl_mfma_kernel<D, BITS, false>, 256, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 2;
        per_cu_cache.store(per_cu, std::memory_order_relaxed);
    }
    const int64_t cap = int64_t(current_cu_count()) * per_cu;
    const int64_t need = (int64_t(nvec) + 63) / 64;
    const int64_t blocks = need < cap ? need : cap;
    const grid_index gi{make_fastdiv(static_cast<uint32_t>(a.n2)), make_fastdiv(static_cast<uint32_t>(a.n1))};
    encode_args f;
    if (fold_flat(a, f))
        hipLaunchKernelGGL((encode_qjl_mfma_kernel<D, BITS, true>), dim3(blocks), dim3(256), 0, s, t, f, gi, nvec);
    else
        hipLaunchKernelGGL((encode_qjl_mfma_kernel<D, BITS, false>), dim3(blocks), dim3(256), 0, s, t, a, gi, nvec);
    return hipGetLastError();
}

}  // namespace

bool encode_qjl_mfma_supported(const dev_tables & t, const encode_args & a) {
    return t.qjl && !t.haar && !t.norm_group && !t.norm_corr && t.m == t.d && (t.d == 64 || t.d == 128) &&
           a.dtype == TQ_DTYPE_BF16;
}

hipError_t launch_encode_qjl_mfma(const dev_tables & t, const encode_args & a, uint32_t nvec, hipStream_t s) {
    switch (t.d * 8 + t.bits) {
        case 64 * 8 + 2: return launch_d<64, 2>(t, a, nvec, s);
        case 64 * 8 + 3: return launch_d<64, 3>(t, a, nvec, s);
        case 64 * 8 + 4: return launch_d<64, 4>(t, a, nvec, s);
        case 128 * 8 + 2: return launch_d<128, 2>(t, a, nvec, s);
        case 128 * 8 + 3: return launch_d<128, 3>(t, a, nvec, s);
        case 128 * 8 + 4: return launch_d<128, 4>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
