// Device helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tq {

// ---------------------------------------------------------------------------
// Cross-lane exchange within small lane groups.  xor 1 and xor 2 use DPP
// quad permutes; larger masks use ds_swizzle in bit-mask mode (within 32
// lanes: source = lane ^ mask).

template <int MASK>
__device__ __forceinline__ int lane_xor_i32(int v) {
    static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8 || MASK == 16, "mask");
    if constexpr (MASK == 1) {
        return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (MASK == 2) {
        return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else {
        return __builtin_amdgcn_ds_swizzle(v, (MASK << 10) | 0x1F);
    }
}

template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
    return __int_as_float(lane_xor_i32<MASK>(__float_as_int(v)));
}

template <int MASK>
__device__ __forceinline__ double lane_xor(double v) {
    int64_t b = __double_as_longlong(v);
    int lo = lane_xor_i32<MASK>(static_cast<int>(b));
    int hi = lane_xor_i32<MASK>(static_cast<int>(b >> 32));
    return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Sum over aligned groups of N lanes (N a power of two <= 32); every lane of
// a group receives the identical value (the same pairwise tree in each lane).
template <int N, typename T>
__device__ __forceinline__ T group_sum(T v) {
    if constexpr (N >= 2) v += lane_xor<1>(v);
    if constexpr (N >= 4) v += lane_xor<2>(v);
    if constexpr (N >= 8) v += lane_xor<4>(v);
    if constexpr (N >= 16) v += lane_xor<8>(v);
    if constexpr (N >= 32) v += lane_xor<16>(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Maximum over the wave, returned wave-uniform.  Floats are mapped to
// integers of the same order (negative values get their magnitude bits
// flipped), so the row reductions are plain integer DPP maxima (quad swaps,
// then half-row and row mirrors); the four row results are combined in
// scalars.
__device__ __forceinline__ int float_order_key(int b) { return b ^ ((b >> 31) & 0x7FFFFFFF); }

__device__ __forceinline__ float wave_max_uniform(float v) {
    auto dpp_max = [](int x, auto ctrl) {
        return max(x, __builtin_amdgcn_update_dpp(x, x, decltype(ctrl)::value, 0xF, 0xF, true));
    };
    int k = float_order_key(__float_as_int(v));
    k = dpp_max(k, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    k = dpp_max(k, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    k = dpp_max(k, std::integral_constant<int, 0x141>{});  // row_half_mirror
    k = dpp_max(k, std::integral_constant<int, 0x140>{});  // row_mirror
    const int m = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
                      max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
    return __int_as_float(float_order_key(m));
}

// x + (the same register of lane l ^ 32) and of lane l ^ 16, with the
// cross-row permlane swaps of gfx950 (no LDS traffic).
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Sum over the wave, in every lane: DPP adds within rows of 16, then the
// two cross-row permlane swaps.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    auto dpp_add = [](float x, auto ctrl) {
        return x + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x),
                                                              decltype(ctrl)::value, 0xF, 0xF, true));
    };
    v = dpp_add(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    v = dpp_add(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    v = dpp_add(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    v = dpp_add(v, std::integral_constant<int, 0x140>{});  // row_mirror
    return add_xor32(add_xor16(v));
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------------------
// Half precision.

// Round a double to fp16 in one step, ties to even (no detour through float).
__device__ __forceinline__ uint16_t half_bits_rne(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
    const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    if (a >= 0x7FF0000000000000ull) return sign | (a > 0x7FF0000000000000ull ? 0x7E00 : 0x7C00);
    const int e = static_cast<int>(a >> 52) - 1023;
    if (e > 15) return sign | 0x7C00;
    if (e < -25 || a == 0) return sign;  // below half the smallest subnormal
    const uint64_t mant = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    const int shift = e >= -14 ? 42 : 42 + (-14 - e);  // bits dropped
    uint64_t q = mant >> shift;
    const uint64_t rem = mant & ((1ull << shift) - 1);
    const uint64_t halfway = 1ull << (shift - 1);
    if (rem > halfway || (rem == halfway && (q & 1))) ++q;
    if (e >= -14) {
        int ee = e;
        if (q == 2048) {
            q = 1024;
            ++ee;
        }
        if (ee > 15) return sign | 0x7C00;
        return sign | static_cast<uint16_t>(((ee + 15) << 10) | (q - 1024));
    }
    return sign | static_cast<uint16_t>(q);  // subnormal; q == 1024 encodes 2^-14
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return static_cast<float>(v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Code i (0 <= i < 32) of a 32-code block held in BITS consecutive dwords.
template <int BITS>
__device__ __forceinline__ uint32_t block_code(const uint32_t * w, int i) {
    const int bit = BITS * i;
    const int wi = bit >> 5, off = bit & 31;
    uint32_t c = w[wi] >> off;
    if (off + BITS > 32) c |= w[wi + 1] << (32 - off);
    return c & ((1u << BITS) - 1);
}

}  // namespace tq
