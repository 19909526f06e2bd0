// Encode kernels: norm -> rotation -> scalar codebook -> packing -> QJL.
//
// Steps as the pages order them: per-vector norm extraction ([TQ+ guide]
// §5.1), structured rotation D1.H.D2 by a fast Walsh-Hadamard transform
// ([TQ+ guide] §4), MSE-only centroid quantisation in blocks of 32 with the
// rotation width decoupled from the block size ([TQ+ guide] §5.1-§5.2, §6.1),
// bit packing, and the optional 1-bit QJL sketch of the residual
// ([Orión plan] Fase 3 sign-bit sketch; [TQ explainer] §2.2).
//
// Three kernels:
//  * encode_mfma_kernel (bf16 inputs, d = 64 or 128, MSE-only): the rotation
//    as exact-product bf16 matrix-core tiles and a wave-mask quantiser; its
//    own comment below gives the lane layout.
//  * encode_kernel (other MSE-only inputs) and encode_qjl_kernel: a vector of
//    d coordinates is owned by d/32 consecutive lanes; lane `blk` holds
//    coordinates 32*blk .. 32*blk+31, which is exactly one packed 32-code
//    block, so each lane writes its own block.  The first five butterfly
//    stages run inside a lane's registers, the remaining log2(d/32) stages
//    exchange with partner lanes (DPP quad permutes / ds_swizzle).
//
// Precision of the lane-per-block kernels:
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
//  * QJL ctx (encode_qjl_kernel): the rotation, codes and residual in
//    double, so that the fp16 residual norm also rounds exactly as float64
//    does; the sketch S r on matrix cores (fp16 hi/lo split, ~22 bits).
#include <atomic>

#include "tq_device.h"
#include "tq_encode_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

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

// QJL ctx.  Phase A (per lane, one 32-coordinate block of one vector): the
// rotation, z, codes, residual r = z - c[code] and gamma = ||r|| / sqrt(d) in
// double (so gamma's fp16 rounding matches float64); r goes to LDS as an
// fp16 hi + lo pair.  Phase B (per wave, a quarter of S's rows): the sketch
// h = S r for the workgroup's vectors on matrix cores, 16x16x32 fp16 MFMAs
// over S = S_hi + S_lo and r = r_hi + r_lo (three products; ~22 bits), and
// the sign bits of h ([Orión plan] Fase 3; [TQ explainer] §2.2).  The sign
// of S rho equals the sign of S r, rho = r / sqrt(d).
template <int D, int BITS, bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void encode_qjl_kernel(const dev_tables t, const encode_args a,
                                                         const grid_index gi, const uint32_t nvec) {
    constexpr int LPV = D / 32;
    // vectors per workgroup iteration: NR rounds of phase A (256 / LPV
    // vectors each), so that every S fragment a k-step loads feeds at least
    // four 16-vector column tiles of phase B
    constexpr int NR = D == 256 ? 2 : 1;
    constexpr int VPB = NR * 256 / LPV;
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    constexpr int RS = D + 8;        // LDS row stride (halves): rows start 16 B apart in the banks
    constexpr int RT = D / 16;       // 16-row tiles of S (m = d)
    constexpr int KS = D / 32;       // 32-wide k-steps
    constexpr int CT = VPB / 16;     // 16-vector column tiles
    __shared__ __align__(16) uint16_t rl[2][VPB * RS];
    __shared__ int64_t pvs[VPB];  // plane index of each vector of the batch (-1: none)
    __shared__ float cpos[8];  // positive centroids cb[2^(b-1) + k]
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int blk = tid % LPV;
    const uint32_t d1w = t.d1[blk];
    const uint32_t d2w = t.d2[blk];
    // positive thresholds th[2^(b-1) + j]; the codebook is exactly symmetric
    float pth[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pth[j] = j < int(kHalf) - 1 ? t.th[kHalf + j] : 0.f;
    if (tid < int(kHalf)) cpos[tid] = t.cb[kHalf + tid];
    __syncthreads();
    const uint16_t * const s_hi = t.S16;
    const uint16_t * const s_lo = t.S16 + D * D;

    for (uint32_t base = blockIdx.x * VPB; base < nvec; base += gridDim.x * VPB) {
#pragma unroll 1
      for (int rd = 0; rd < NR; ++rd) {
        const int vl = tid / LPV + rd * (256 / LPV);   // vector within the workgroup's batch
        const uint32_t v = base + vl;
        const bool valid = v < nvec;
        int64_t xoff, pv;
        vector_offsets(valid ? v : nvec - 1, a, gi, xoff, pv);

        // ---------------- phase A
        float xf[32];
        load_block<BF16>(a, xoff + blk * 32, xf);
        double x[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = xf[e];
        double nsq = 0.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) nsq = fma(x[e], x[e], nsq);
        nsq = group_sum<LPV>(nsq);
        const double n = sqrt(nsq);
        if (valid && blk == 0) a.out.norms[pv] = half_bits_rne(n);
        if (blk == 0) pvs[vl] = valid ? pv : int64_t(-1);
        // D2 as sign-bit XORs (a per-element select would be hoisted into 32
        // scalar lane masks, more than the scalar registers hold)
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = flip_sign(x[e], d2w, e);
        lane_fwht(x);
        cross_lane_fwht<LPV>(x, blk);
        // z = sqrt(d) R x / n = D1 y / n;  code = #{k : th_k < z}, decided on
        // fp32(z) (it differs from the float64 decision only within an fp32
        // ulp of a threshold) through the codebook's symmetry:
        // code = 2^(b-1) + k for z > 0, 2^(b-1) - 1 - k for z <= 0, with
        // k = #{positive thresholds < |z|}; the residual stays in float64
        const double inv_n = n > 0.0 ? 1.0 / n : 0.0;
        uint32_t w[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = 0;
        double gsq = 0.0;
        uint32_t rh[16], rlo[16];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const double z = flip_sign(x[e] * inv_n, d1w, e);
            const float zf = static_cast<float>(z);
            const uint32_t kk = count_below<BITS>(fabsf(zf), pth);
            const bool zneg = !(zf > 0.f);  // z = 0 (zero vectors) counts no threshold: 2^(b-1) - 1
            const uint32_t c = zneg ? kHalf - 1 - kk : kHalf + kk;
            const int bit = BITS * e;
            w[bit >> 5] |= c << (bit & 31);
            if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
            const double cm = static_cast<double>(cpos[kk]);
            const double r = zneg ? z + cm : z - cm;
            gsq = fma(r, r, gsq);
            const float rf = valid ? static_cast<float>(r) : 0.f;
            const _Float16 h = static_cast<_Float16>(rf);
            const _Float16 l = static_cast<_Float16>(rf - static_cast<float>(h));
            const uint32_t hb = __builtin_bit_cast(unsigned short, h), lb = __builtin_bit_cast(unsigned short, l);
            if (e & 1) {
                rh[e >> 1] |= hb << 16;
                rlo[e >> 1] |= lb << 16;
            } else {
                rh[e >> 1] = hb;
                rlo[e >> 1] = lb;
            }
        }
        if (valid) {
            uint32_t * dst = reinterpret_cast<uint32_t *>(a.out.codes + pv * (D * BITS / 8)) + blk * BITS;
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[k] = w[k];
        }
        gsq = group_sum<LPV>(gsq);
        if (valid && blk == 0) a.out.rnorms[pv] = half_bits_rne(sqrt(gsq) / sqrt(static_cast<double>(D)));
        {
            uint4 * dh = reinterpret_cast<uint4 *>(&rl[0][vl * RS + 32 * blk]);
            uint4 * dl = reinterpret_cast<uint4 *>(&rl[1][vl * RS + 32 * blk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                dh[q] = uint4{rh[4 * q], rh[4 * q + 1], rh[4 * q + 2], rh[4 * q + 3]};
                dl[q] = uint4{rlo[4 * q], rlo[4 * q + 1], rlo[4 * q + 2], rlo[4 * q + 3]};
            }
        }
      }
        __syncthreads();

        // ---------------- phase B: rows 16 rt .. +15 of h for 16 vectors per
        // tile; wave w takes row tiles w, w + 4, ..., and every residual tile
        // read from LDS feeds all of them
        const int n16 = lane & 15, g4 = lane >> 4;
        constexpr int RW = (RT + 3) / 4;  // row tiles per wave (waves >= RT have none at d = 32)
        // the row tiles in groups of at most two, so that the accumulators of
        // a group (two row tiles x CT column tiles) and its S fragments fit
        // the registers with phase A's state; each group re-reads the
        // residual tiles from LDS
        constexpr int RG = RW < 2 ? RW : 2;
#pragma unroll 1
        for (int r0 = 0; r0 < RW; r0 += RG) {
            f32x4 acc[RG][CT];
#pragma unroll
            for (int rw = 0; rw < RG; ++rw)
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[rw][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            // one k-step at a time (a full unroll hoists every load and spills)
#pragma unroll 1
            for (int ks = 0; ks < KS; ++ks) {
                f16x8 ah[RG], al[RG];
#pragma unroll
                for (int rw = 0; rw < RG; ++rw) {
                    const int rt = wave + 4 * (r0 + rw) < RT ? wave + 4 * (r0 + rw) : 0;
                    const int64_t so = int64_t(16 * rt + n16) * D + 32 * ks + 8 * g4;
                    ah[rw] = as_f16x8(*reinterpret_cast<const uint4 *>(s_hi + so));
                    al[rw] = as_f16x8(*reinterpret_cast<const uint4 *>(s_lo + so));
                }
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const int ro = (16 * c + n16) * RS + 32 * ks + 8 * g4;
                    const f16x8 bh = as_f16x8(*reinterpret_cast<const uint4 *>(&rl[0][ro]));
                    const f16x8 bl = as_f16x8(*reinterpret_cast<const uint4 *>(&rl[1][ro]));
#pragma unroll
                    for (int rw = 0; rw < RG; ++rw) {
                        acc[rw][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rw], bh, acc[rw][c], 0, 0, 0);
                        acc[rw][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rw], bl, acc[rw][c], 0, 0, 0);
                        acc[rw][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rw], bh, acc[rw][c], 0, 0, 0);
                    }
                }
            }
            // lane holds rows 16 rt + 4 g4 + i of vector 16 c + n16
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const int64_t pvv = pvs[16 * c + n16];
#pragma unroll
                for (int rw = 0; rw < RG; ++rw) {
                    uint32_t bits = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) bits |= (acc[rw][c][i] > 0.f ? 1u : 0u) << (4 * g4 + i);
                    bits |= __shfl_xor(bits, 16);
                    bits |= __shfl_xor(bits, 32);
                    const int rt = wave + 4 * (r0 + rw);
                    if (g4 == 0 && pvv >= 0 && rt < RT)
                        reinterpret_cast<uint16_t *>(a.out.signs + pvv * (D / 8))[rt] = static_cast<uint16_t>(bits);
                }
            }
        }
        __syncthreads();  // the residual tile is rewritten by the next iteration
    }
}

// ---------------------------------------------------------------------------
// bf16 input, MSE-only, d = 64 or 128: the rotation on matrix cores.
//
// H_d = H_(d/32) (x) H_32 (Sylvester order: the block index is the high bits
// of the coordinate), so output block b' of H_d D2 x is the sum over input
// blocks b of (-1)^popcount(b' & b) H_32 (D2 x)_b.  Each term is a 16x16x32
// bf16 MFMA per 16-row half, accumulated over b in fp32: the B operand is
// the input with D2's sign flips (bf16, exact), the A operand the +-1
// entries of +-H_32, so the products are exact.  A wave takes 16 vectors;
// lane l loads coordinates 8(l/16)..+7 of each block of vector l%16.  The A
// rows are permuted so that the same lane receives output coordinates
// 8(l/16)..+7 of each block: the quantiser and the packing of 8 codes stay
// in the lane.
// At most 128 VGPRs (4 waves per SIMD; no spills): at 130 the prefetching
// kernel would drop to 3 waves and to the slower non-prefetching launch plan.
template <int D, int BITS, bool PREFETCH, bool FLAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void encode_mfma_kernel(const dev_tables t, const encode_args a,
                                                          const grid_index gi, const uint32_t nvec) {
    constexpr int NB = D / 32;
    constexpr uint32_t kHalf = 1u << (BITS - 1);
    constexpr uint32_t kAll = (1u << BITS) - 1;
    static_assert(NB == 2 || NB == 4, "d = 64 or 128");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;

    // A operand of output half tt: row m holds H_32 row 8(m/4) + 4 tt + m%4;
    // this lane supplies row n, columns 8g..8g+7
    uint32_t hw[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int row = 8 * (n >> 2) + 4 * tt + (n & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c0 = 8 * g + 2 * j;
            const uint32_t lo = (__builtin_popcount(row & c0) & 1) ? 0xBF80u : 0x3F80u;       // -1 / +1
            const uint32_t hi = (__builtin_popcount(row & (c0 + 1)) & 1) ? 0xBF80u : 0x3F80u;
            hw[tt][j] = lo | (hi << 16);
        }
    }
    // the cross-block transform's signs go into the A operand: +-H_32 tiles
    uint32_t hwn[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) hwn[tt][j] = hw[tt][j] ^ 0x80008000u;
    // D2's signs for the lane's input columns (bit 15: even, bit 31: odd)
    uint32_t m2[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 8 * g + 2 * j;
            m2[b][j] = (((t.d2[b] >> e) & 1) << 15) | (((t.d2[b] >> (e + 1)) & 1) << 31);
        }
    // A operand tiles (-1)^s H_32; D2 is applied to the input by sign-bit
    // XORs (16 registers of tiles instead of 64 with D2 folded in: five
    // waves per SIMD for the non-prefetching kernel)
    bf16x8 hA[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        hA[tt][0] = as_bf16x8(hw[tt]);
        hA[tt][1] = as_bf16x8(hwn[tt]);
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

    // each wave takes 16 vectors per iteration; with PREFETCH the next
    // iteration's inputs are loaded while the current ones are processed
    // (unconditionally: lanes past the end load the last vector again, so
    // the loaded registers need no loop-carried copies)
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
    if (PREFETCH && base < nvec) load_inputs(base);
    for (; base < nvec; base += stride) {
        if (!PREFETCH) load_inputs(base);
        const bool valid = valid_next;
        const int64_t pv = pv_next;
        // D2 x: sign flips of the loaded bf16 pairs
        uint32_t w[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[b][j] = wn[b][j] ^ m2[b][j];
        if (PREFETCH) load_inputs(base + stride);

        // Norm, as float64 rounds it to fp16.  First in fp32 from exact bf16
        // products (v_dot2): its error stays below 19 fp32 ulps of n (32
        // roundings of positive partial sums, the lane sum, and v_sqrt_f32's
        // 1-ulp result), so unless n lies within 32 ulps of an fp16 rounding midpoint
        // it rounds to the same fp16 as float64.  Those vectors, and norms
        // outside fp16's normal range [2^-14, 60000] (where the midpoint test
        // does not apply; products may also be subnormal), take the float64
        // sum.  The 4 lanes of a vector hold bitwise-identical
        // sums, so they decide alike.
        float s32 = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) s32 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[b][j]), as_bf16x2(w[b][j]), s32, false);
        s32 += __shfl_xor(s32, 16);
        s32 += __shfl_xor(s32, 32);
        const float n32 = __builtin_amdgcn_sqrtf(s32);
        const int mid = int(__float_as_uint(n32) & 0x1FFFu) - 0x1000;
        const bool exact64 = (mid > -32 && mid < 32) || !(n32 >= 0x1p-14f && n32 <= 60000.f);
        double nrm = n32;
        uint16_t nbits = static_cast<uint16_t>(__builtin_bit_cast(unsigned short, static_cast<_Float16>(n32)));
        if (__any(exact64)) {
            double nsq = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wj = opaque(w[b][j]);
                    const double lo = bf16_lo(wj), hi = bf16_hi(wj);
                    nsq = fma(lo, lo, nsq);
                    nsq = fma(hi, hi, nsq);
                }
            nsq += __shfl_xor(nsq, 16);
            nsq += __shfl_xor(nsq, 32);
            if (exact64) {
                nrm = sqrt(nsq);
                nbits = half_bits_rne(nrm);
            }
        }
        if (valid && g == 0) a.out.norms[pv] = nbits;

        // keep fp32 sums in range: rescale by a power of two (exact for bf16)
        float nf = static_cast<float>(nrm);
        const bool far = nrm > 0.0 && !(nrm >= 0x1p-60 && nrm <= 0x1p60);
        if (__any(far)) {
            const int e = far ? ilogb(nrm) : 0;
            const float sc = ldexpf(1.f, -e);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wj = opaque(w[b][j]);
                    const uint32_t lo = __float_as_uint(bf16_lo(wj) * sc) >> 16;
                    const uint32_t hi = __float_as_uint(bf16_hi(wj) * sc) & 0xFFFF0000u;
                    w[b][j] = lo | hi;
                }
            if (far) nf = static_cast<float>(ldexp(nrm, -e));
        }

        // y_b' = sum_b (-1)^popcount(b' & b) H_32 D2 x_b, all on matrix cores:
        // lane gets coordinates 32 b' + 8 g + 4 tt + r of vector n
        bf16x8 xb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) xb[b] = as_bf16x8(w[b]);
        // Codes of coordinates 32 b + 8 g + j, j = 4 tt + r, as 8-code chunks
        // (code(z) = count of positive thresholds below |z|, with every bit
        // flipped when z < 0, and 2^(b-1) set for z >= 0; a coordinate of
        // exactly 0 is a tie between the two middle codes).  One output block
        // at a time keeps 8 accumulators live.
        float T[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) T[j] = p[j] * nf;
        uint8_t * const row = a.out.codes + pv * (D * BITS / 8);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4 u[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hA[tt][__builtin_popcount(b & bi) & 1], xb[bi], acc, 0, 0, 0);
                u[tt] = acc;
            }
            // each 8-code chunk is built bit-serially from the top: the sign
            // bit straight from y, then each magnitude decision as a wave
            // mask shifted in by one add-with-carry
            uint32_t c = 0;
#pragma unroll
            for (int j = 7; j >= 0; --j) {
                const float y = u[j >> 2][j & 3];
                const float ya = fabsf(y);
                c = __builtin_amdgcn_alignbit(c, __float_as_uint(y), 31);  // the sign bit
                if constexpr (BITS == 4) {
                    const bool t1 = ya > T[3];
                    const float q2 = t1 ? T[5] : T[1];
                    const float hi3 = t1 ? T[6] : T[2];
                    const float lo3 = t1 ? T[4] : T[0];
                    const bool t2 = ya > q2;
                    const bool t3 = ya > (t2 ? hi3 : lo3);
                    c = shift_in(c, __ballot(t1));
                    c = shift_in(c, __ballot(t2));
                    c = shift_in(c, __ballot(t3));
                } else if constexpr (BITS == 3) {
                    const bool t1 = ya > T[1];
                    const bool t2 = ya > (t1 ? T[2] : T[0]);
                    c = shift_in(c, __ballot(t1));
                    c = shift_in(c, __ballot(t2));
                } else {
                    const bool t1 = ya > T[0];
                    c = shift_in(c, __ballot(t1));
                }
            }
            {
                // fields are [sign, magnitude bits]: flip the magnitude bits of
                // negative coordinates and every sign bit
                constexpr uint32_t low = BITS == 2 ? 0x5555u : BITS == 3 ? 0x249249u : 0x11111111u;
                const uint32_t m = (c >> (BITS - 1)) & low;
                const uint32_t spread = m * ((1u << (BITS - 1)) - 1);
                c = nrm > 0.0 ? c ^ spread ^ (xm[b] ^ (low << (BITS - 1))) : zero_chunk;
            }
            if constexpr (BITS == 4) {
                if (valid) reinterpret_cast<uint32_t *>(row + 16 * b)[g] = c;
            } else if constexpr (BITS == 3) {
                // block dword g = bits 32g..32g+31 = chunk g (24 bits at 24 g) and chunk g+1
                const uint32_t nx = __shfl_down(c, 16);
                const uint32_t dw = (c >> (8 * g)) | (nx << (24 - 8 * g));
                if (valid && g < 3) reinterpret_cast<uint32_t *>(row + 12 * b)[g] = dw;
            } else {
                const uint32_t nx = __shfl_down(c, 16);
                if (valid && (g & 1) == 0) reinterpret_cast<uint32_t *>(row + 8 * b)[g >> 1] = c | (nx << 16);
            }
        }
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
        if (bf16 && (D == 64 || D == 128)) {
            constexpr int DM = D == 64 ? 64 : 128;
            // Up to 4 iterations per resident block: one round of blocks,
            // each taking the same number of 64-vector iterations, with the
            // next iteration's inputs prefetched.  Larger inputs: a fixed grid
            // striding over the vectors, loading at each iteration's start.
            static std::atomic<int> per_cu_cache{0};  // same on every gfx950 device
            int per_cu = per_cu_cache.load(std::memory_order_relaxed);
            if (per_cu == 0) {
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, encode_mfma_kernel<DM, BITS, true, false>, 256, 0) !=
                        hipSuccess ||
                    per_cu <= 0)
                    per_cu = 4;
                per_cu_cache.store(per_cu, std::memory_order_relaxed);
            }
            const int cap = current_cu_count() * per_cu;
            const int64_t need = (int64_t(nvec) + 63) / 64;
            const int64_t iters = (need + cap - 1) / cap;
            encode_args f;
            const bool flat = fold_flat(a, f);
            if (iters <= 4) {
                const int64_t mb = (need + iters - 1) / iters;
                if (flat)
                    hipLaunchKernelGGL((encode_mfma_kernel<DM, BITS, true, true>), dim3(mb), dim3(256), 0, s, t, f, gi, nvec);
                else
                    hipLaunchKernelGGL((encode_mfma_kernel<DM, BITS, true, false>), dim3(mb), dim3(256), 0, s, t, a, gi, nvec);
            } else {
                const int64_t mb = need < 256 * 16 ? need : 256 * 16;
                if (flat)
                    hipLaunchKernelGGL((encode_mfma_kernel<DM, BITS, false, true>), dim3(mb), dim3(256), 0, s, t, f, gi, nvec);
                else
                    hipLaunchKernelGGL((encode_mfma_kernel<DM, BITS, false, false>), dim3(mb), dim3(256), 0, s, t, a, gi, nvec);
            }
        } else if (bf16)
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
    if (t.haar || t.norm_group || t.norm_corr) return launch_encode_variant(t, a, s);
    const uint32_t nvec = static_cast<uint32_t>(a.n0 * a.n1 * a.n2);
    if (encode_qjl_mfma_supported(t, a)) return launch_encode_qjl_mfma(t, a, nvec, s);
    switch (t.d) {
        case 32: return launch_encode_d<32>(t, a, nvec, s);
        case 64: return launch_encode_d<64>(t, a, nvec, s);
        case 128: return launch_encode_d<128>(t, a, nvec, s);
        case 256: return launch_encode_d<256>(t, a, nvec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
