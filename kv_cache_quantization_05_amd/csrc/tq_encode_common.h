// Helpers shared by the encode kernels: grid indexing, lane-per-block
// Walsh-Hadamard butterflies, input loads, the symmetric quantiser,
// matrix-core operand casts and the host-side grid folding.
#pragma once

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
// output plane index.  v < 2^32 (checked on the host).  FLAT: the host has
// folded the grid into its last dimension (n0 = n1 = 1) with both strides
// in [0, 2^32), so each offset is one 32 x 32 -> 64-bit product.
template <bool FLAT = false>
__device__ __forceinline__ void vector_offsets(uint32_t v, const encode_args & a, const grid_index & gi,
                                               int64_t & xoff, int64_t & pv) {
    if constexpr (FLAT) {
        xoff = static_cast<int64_t>(uint64_t(v) * static_cast<uint32_t>(a.xs2));
        pv = static_cast<int64_t>(uint64_t(v) * static_cast<uint32_t>(a.out.stride[2]));
        return;
    }
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

// v with its sign flipped when bit e of w is set, as a bit XOR on the high word
__device__ __forceinline__ double flip_sign(double v, uint32_t w, int e) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t m = static_cast<uint64_t>((w << (31 - e)) & 0x80000000u) << 32;
    return __longlong_as_double(static_cast<long long>(b ^ m));
}

// Matrix-core operand types and bit-casts.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8 as_f16x8(uint4 w) {
    f16x8 r;
    __builtin_memcpy(&r, &w, 16);
    return r;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
    bf16x2 r;
    __builtin_memcpy(&r, &w, 4);
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    bf16x8 r;
    __builtin_memcpy(&r, w, 16);
    return r;
}

// The value unchanged, but opaque to the optimiser: what is computed from it
// inside a rarely taken branch stays there instead of being hoisted into the
// common path.  (An empty asm: no instruction is emitted.)
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// 2c + bit with the bits of all lanes given as a wave mask (a compare result,
// possibly combined with others by scalar logic): one v_addc whose carry-in
// is the mask, where the compiler would turn each bit into a select and a
// shift-or.  (A plain ALU instruction: no memory access in the asm.)
__device__ __forceinline__ uint32_t shift_in(uint32_t c, uint64_t bits) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(c), "s"(bits));
    return r;
}

// The grid folded into one dimension when its vectors are evenly spaced in
// both the input and the planes (size-1 dimensions dropped, each remaining
// dimension's strides equal to the folded inner block's extent), with both
// strides in [0, 2^32).  Returns false, leaving f unset, otherwise.
inline bool fold_flat(const encode_args & a, encode_args & f) {
    const int64_t n[3] = {a.n0, a.n1, a.n2}, xs[3] = {a.xs0, a.xs1, a.xs2};
    const int64_t ps[3] = {a.out.stride[0], a.out.stride[1], a.out.stride[2]};
    constexpr int64_t kLim = int64_t(1) << 32;
    int64_t cn = 1, cx = 0, cp = 0;  // cn < 2^32: the host has checked n0 n1 n2 < 2^32
    bool any = false;
    for (int i = 2; i >= 0; --i) {
        if (n[i] == 1) continue;
        if (!any) {
            if (xs[i] < 0 || xs[i] >= kLim || ps[i] < 0 || ps[i] >= kLim) return false;
            cn = n[i];
            cx = xs[i];
            cp = ps[i];
            any = true;
        } else {
            // cn, cx, cp < 2^32: the products fit in 64 unsigned bits
            if (xs[i] < 0 || ps[i] < 0 || uint64_t(xs[i]) != uint64_t(cn) * uint64_t(cx) ||
                uint64_t(ps[i]) != uint64_t(cn) * uint64_t(cp))
                return false;
            cn *= n[i];
        }
    }
    f = a;
    f.n0 = f.n1 = 1;
    f.n2 = cn;
    f.xs0 = f.xs1 = 0;
    f.xs2 = cx;
    f.out.stride[0] = f.out.stride[1] = 0;
    f.out.stride[2] = cp;
    return true;
}

}  // namespace
}  // namespace tq
