// Packed-code -> fp16 unpacking for MFMA operands (gfx950).
//
// A lane turns one 32-code block (4*BITS bytes) into 32 fp16 centroid values,
// i.e. 16 dwords of fp16 pairs, with v_perm byte look-ups into the centroid
// table (the fp16 centroid LUT idea of [TQ+ guide] §5.3, done with byte
// permutes instead of memory).  Codes come out in a fixed permuted order;
// block_code_of_pos<BITS>(pos) gives the code index (0..31) whose value sits
// in half `pos` of the output, so a contraction over the block can permute
// its other operand to match.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// fp16 centroid table split into byte planes for v_perm look-ups.
struct lut16 {
    uint32_t lo[4];  // low bytes of entries 0..15, 4 per dword
    uint32_t hi[4];  // high bytes
};

__device__ __forceinline__ uint16_t f16_bits(float v) {
    _Float16 h = static_cast<_Float16>(v);
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

__device__ __forceinline__ lut16 make_lut(const float * cb) {
    lut16 t;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = f16_bits(cb[4 * d + k]);
            lo |= (b & 0xFFu) << (8 * k);
            hi |= (b >> 8) << (8 * k);
        }
        t.lo[d] = lo;
        t.hi[d] = hi;
    }
    return t;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Four codes in the bytes of `sel` (values < 2^BITS) -> two dwords of fp16
// pairs: x = (v(sel.b0), v(sel.b1)), y = (v(sel.b2), v(sel.b3)).
template <int BITS>
__device__ __forceinline__ void lut4(const lut16 & t, uint32_t sel, uint32_t & x, uint32_t & y) {
    uint32_t lo, hi;
    if constexpr (BITS == 2) {
        lo = perm_b32(t.lo[0], t.lo[0], sel);
        hi = perm_b32(t.hi[0], t.hi[0], sel);
    } else if constexpr (BITS == 3) {
        lo = perm_b32(t.lo[1], t.lo[0], sel);
        hi = perm_b32(t.hi[1], t.hi[0], sel);
    } else {
        // 16 entries: look up in both halves, pick by bit 3 of each code
        const uint32_t s7 = sel & 0x07070707u;
        const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
        const uint32_t lo_a = perm_b32(t.lo[1], t.lo[0], s7), lo_b = perm_b32(t.lo[3], t.lo[2], s7);
        const uint32_t hi_a = perm_b32(t.hi[1], t.hi[0], s7), hi_b = perm_b32(t.hi[3], t.hi[2], s7);
        lo = (lo_b & m) | (lo_a & ~m);
        hi = (hi_b & m) | (hi_a & ~m);
    }
    x = perm_b32(hi, lo, 0x05010400u);
    y = perm_b32(hi, lo, 0x07030602u);
}

// fp16 bits of centroid idx (< 2^BITS), from the byte planes.
template <int BITS>
__device__ __forceinline__ uint32_t lut_bits(const lut16 & t, uint32_t idx) {
    uint32_t x, y;
    lut4<BITS>(t, idx, x, y);
    return x & 0xFFFFu;
}

// Code index inside the block of output half `pos` (0..31).
template <int BITS>
__host__ __device__ constexpr int block_code_of_pos(int pos) {
    if (BITS == 2) {  // pos = 16d + 4r + m  <->  code 16d + 4m + r
        return (pos & 16) + 4 * (pos & 3) + ((pos >> 2) & 3);
    } else if (BITS == 3) {  // pos = 4r + m  <->  code 8m + r
        return 8 * (pos & 3) + (pos >> 2);
    } else {  // pos = 8d + 4e + m  <->  code 8d + 2m + e
        return (pos & 24) + 2 * (pos & 3) + ((pos >> 2) & 1);
    }
}

// One block (BITS dwords, LSB-first codes) -> 16 dwords of fp16 pairs.
template <int BITS>
__device__ __forceinline__ void unpack_block(const lut16 & t, const uint32_t * w, uint32_t * out) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t s = (w[d] >> (2 * r)) & 0x03030303u;
                lut4<2>(t, s, out[8 * d + 2 * r], out[8 * d + 2 * r + 1]);
            }
        }
    } else if constexpr (BITS == 3) {
        // gather bytes 3m+0, 3m+1, 3m+2 (m = 0..3) of the 12-byte block
        const uint32_t ta = perm_b32(w[1], w[0], 0x00060300u);
        const uint32_t A = perm_b32(w[2], ta, 0x05020100u);
        const uint32_t tb = perm_b32(w[1], w[0], 0x00070401u);
        const uint32_t Bg = perm_b32(w[2], tb, 0x06020100u);
        const uint32_t tc = perm_b32(w[1], w[0], 0x00000502u);
        const uint32_t C = perm_b32(w[2], tc, 0x07040100u);
        const uint32_t M7 = 0x07070707u;
        uint32_t s[8];
        s[0] = A & M7;
        s[1] = (A >> 3) & M7;
        s[2] = ((A >> 6) & 0x03030303u) | ((Bg & 0x01010101u) << 2);
        s[3] = (Bg >> 1) & M7;
        s[4] = (Bg >> 4) & M7;
        s[5] = ((Bg >> 7) & 0x01010101u) | ((C & 0x03030303u) << 1);
        s[6] = (C >> 2) & M7;
        s[7] = (C >> 5) & M7;
#pragma unroll
        for (int r = 0; r < 8; ++r) lut4<3>(t, s[r], out[2 * r], out[2 * r + 1]);
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            lut4<4>(t, w[d] & 0x0F0F0F0Fu, out[4 * d], out[4 * d + 1]);
            lut4<4>(t, (w[d] >> 4) & 0x0F0F0F0Fu, out[4 * d + 2], out[4 * d + 3]);
        }
    }
}

// 32 QJL sign bits -> 16 dwords of fp16 +-1 pairs; pair k = (bit k, bit k+16).
__device__ __forceinline__ void unpack_signs(uint32_t bits, uint32_t * out) {
    const uint32_t nb = ~bits;  // a clear bit means -1: set the fp16 sign
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t sh = k <= 15 ? (nb << (15 - k)) : nb;
        out[k] = (sh & 0x80008000u) | 0x3C003C00u;
    }
}

// Bit index inside the 32-bit sign word of output half `pos`.
__host__ __device__ constexpr int sign_bit_of_pos(int pos) { return (pos >> 1) + 16 * (pos & 1); }

// 32 sign bits -> 16 dwords of fp16 pairs in the same order, as b in {0, 1}
// instead of +-1: pair k = (bit k, bit k + 16) as b 2^(k' - 24), k' = k for
// k < 10 and k - 6 above (exact fp16 denormals, one AND each: the bits stay
// in place).  A product against them uses sigma = 2 b - 1: the other operand
// carries 2^(24 - k') times a common power of two, and the sum of that operand
// is subtracted.
__device__ __forceinline__ void expand_signs(uint32_t bits, uint32_t * out) {
    const uint32_t b6 = bits >> 6;
#pragma unroll
    for (int k = 0; k < 16; ++k) out[k] = k < 10 ? (bits & (0x00010001u << k)) : (b6 & (0x00010001u << (k - 6)));
}

// Position k' of the sign bit behind fp16 half `pos` of expand_signs' output.
__host__ __device__ constexpr int sign_shift_of_pos(int pos) { return (pos >> 1) < 10 ? (pos >> 1) : (pos >> 1) - 6; }

// 3- and 4-bit codes can instead be decoded through an LDS
// table indexed by two consecutive codes (2 BITS bits of the row's bit
// stream): entry e holds the fp16 centroids of codes e & (2^BITS - 1) and
// e >> BITS.  The table is stored 32 times, copy c in bank c (entry e of copy
// c at byte 128 e + 4 c), and lane l reads copy l % 32, so the 32 lanes served
// together never share a bank whatever codes they hold.  A lookup costs a
// shift, a mask-or and one ds_read_b32 per two codes, and yields the pair in
// code order.  Sizes: 8 KB (3 bits), 32 KB (4 bits).
template <int BITS>
constexpr bool pair_table() { return BITS == 3 || BITS == 4; }
constexpr int kPairCopies = 32;
template <int BITS>
constexpr int pair_tab_bytes() { return pair_table<BITS>() ? (1 << (2 * BITS)) * kPairCopies * 4 : 0; }

// Code index inside a 32-code block of output half `pos` as the decoder lays
// the block out: pair-table look-ups keep code order, byte-permute unpacking
// permutes it.
template <int BITS>
__host__ __device__ constexpr int decoded_code_of_pos(int pos) {
    return pair_table<BITS>() ? pos : block_code_of_pos<BITS>(pos);
}

// LDS byte offset of pair p (codes 2p, 2p+1) of the code row held in w, in
// the copy whose offset is lane_off.
template <int BITS>
__device__ __forceinline__ uint32_t pair_offset(const uint32_t * w, int p, uint32_t lane_off) {
    constexpr int P = 2 * BITS;
    const int s = P * p, wi = s >> 5, o = s & 31;
    uint32_t t;
    if (o > 32 - P)
        t = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], o - 7);
    else if (o >= 7)
        t = w[wi] >> (o - 7);
    else
        t = w[wi] << (7 - o);
    return (t & (((1u << P) - 1) << 7)) | lane_off;
}

// 4-bit codes: the pair of codes 2p, 2p+1 is byte p of the row, so the LDS
// address of its table entry comes from one byte permute: entry e sits at
// byte 256 e, copy c of a key table at +4 c and of a value table at
// +128 + 4 c (one 64 KB region serves both).  base_byte is the lane's copy
// offset plus 128 for the value half (< 256).
constexpr int kByteTabBytes = 256 * 256;
__device__ __forceinline__ uint32_t byte_pair_offset(const uint32_t * w, int p, uint32_t base_byte) {
    return __builtin_amdgcn_perm(w[p >> 2], base_byte, 0x0C0C0000u | ((4u + uint32_t(p & 3)) << 8));
}

// 3-bit codes use the same 256-entry byte tables: the pair of codes 2p,
// 2p + 1 of a 32-code block (3 dwords) starts at bit 6p, so in the block
// shifted right by 6p mod 8 (0, 2, 4 or 6 bits) it starts at a byte
// boundary; that byte (both codes plus two bits of the next code) indexes
// the table, whose entries ignore their top two index bits.  shifted[k]
// holds the block shifted right by 2k bits (shifted[0] = the block).
struct block3_shifts {
    uint32_t w[4][3];
};

__device__ __forceinline__ block3_shifts shift_block3(const uint32_t * w) {
    block3_shifts s;
#pragma unroll
    for (int i = 0; i < 3; ++i) s.w[0][i] = w[i];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        s.w[k][0] = __builtin_amdgcn_alignbit(w[1], w[0], 2 * k);
        s.w[k][1] = __builtin_amdgcn_alignbit(w[2], w[1], 2 * k);
        s.w[k][2] = w[2] >> (2 * k);
    }
    return s;
}

__device__ __forceinline__ uint32_t byte3_pair_offset(const block3_shifts & s, int p, uint32_t base_byte) {
    const int o = 6 * p, sh = o & 7, bi = (o - sh) >> 3;
    return byte_pair_offset(s.w[sh >> 1], bi, base_byte);
}

}  // namespace tq
