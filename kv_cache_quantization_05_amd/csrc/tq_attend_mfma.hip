// Fused decode attention on matrix cores, d = 128, 4 query heads per KV head.
//
// The 4 grouped queries sharing one KV head form a real dense contraction
// against the dequantised codes, so both products run on matrix cores:
//   logits  S[h, t] = sum_i q'[h, i] c[code_ti] on the 16x16x32 fp16 MFMA:
//           columns are 16 tokens, rows the fp16 hi parts (rows 0..3) and lo
//           parts (rows 4..7) of the 4 rotated queries (~22 bits of q'),
//           rows 8..15 zero; lane l feeds 8 decoded values of code block
//           l / 16 of token l % 16.  Two row swaps (permlane16/32) add the
//           parts and leave lane l with the 4 head logits of token l.
//   values  O[h, i] += sum_t w[h, t] c[code_ti] on the 16-block 4x4x4 fp16
//           MFMA, whose 4-row blocks match the 4 heads exactly: k runs over
//           4 tokens.  A lane holds dims of one token, so each 4-dim group
//           is first transposed within its quad of lanes by a 4x4x4 MFMA
//           against the identity (exact), then multiplied by the quad's
//           weights, which come back from LDS transposed with
//           ds_read_b64_tr_b16.
// 3- and 4-bit codes are decoded two at a time through one 64 KB LDS table
// indexed by a byte of the code row (a byte permute forms the whole
// address); 2-bit codes with byte permutes in registers.
// Query rotation once per head ([TQ+ guide] §5.3), online softmax
// ([TQ explainer] §4.3), the output stays in the rotated domain until the
// merge kernel rotates it back ([TQ+ guide] §6.1).
//
// Memory: each wave streams a contiguous token range with buffer loads whose
// per-lane offsets are fixed; each step's resources start at the step's first
// token and end at the (batch, head)'s valid length, so positions past it
// read as zero.  The next step's codes are loaded while the current one is
// processed (ping-pong register sets; a load is issued for every step, and
// one past the wave's range gets empty resources, so it costs no memory
// traffic).
//
// Softmax bookkeeping per wave, in base-2 units: a wave-uniform reference m
// per head, raised only when a weight w = 2^(s - m) * N_v/sqrt(d) would exceed
// e^kSlack (so most steps need no cross-lane max); w stays safe in fp16
// whatever the norms, and the row sum accumulates 2^(s - m) in fp32.
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_unpack.h"

namespace tq {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;
constexpr int kStep = 64;                  // tokens per wave iteration (one per lane)
constexpr int kPass = 16;                  // tokens per V tile pass
constexpr int kPasses = kStep / kPass;
constexpr int kStage = kG * kD * 4;       // wave results (epilogue)
constexpr int kPTile = kStep * 8;          // 64 tokens x 4 heads x fp16
constexpr int kWaveLds = kStage + kPTile;
static_assert(kG * (kD + 2) * 4 <= kWaveLds, "wave results fit the wave's LDS");
constexpr float kSlack = 10.0f;  // w <= e^10 ~ 2.2e4 stays well inside fp16
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the packed-cache loads: non-temporal (each byte is read
// once per call).  A loads-only copy of the kernel's access pattern streams
// the 128K layer's 419 MB in 63 us with it against 71 us without.
constexpr int kNT = 2;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Largest of four fp16 norms packed in two dwords.
__device__ __forceinline__ float max_norm4(u32x2 w) {
    return fmaxf(fmaxf(half_bits_to_float(static_cast<uint16_t>(w.x & 0xFFFFu)), half_bits_to_float(static_cast<uint16_t>(w.x >> 16))),
                 fmaxf(half_bits_to_float(static_cast<uint16_t>(w.y & 0xFFFFu)), half_bits_to_float(static_cast<uint16_t>(w.y >> 16))));
}

__device__ __forceinline__ half4 tr_read4(const uint8_t * lds_base, int off) {
    const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(lds_base + off));
    half4 h;
    __builtin_memcpy(&h, &a, 8);
    return h;
}

// Four fp32 values that are exact in fp16 -> half4 (round toward zero is exact).
__device__ __forceinline__ half4 to_half4(floatx4 c) {
    const auto lo = __builtin_amdgcn_cvt_pkrtz(c[0], c[1]);
    const auto hi = __builtin_amdgcn_cvt_pkrtz(c[2], c[3]);
    half4 h;
    __builtin_memcpy(&h, &lo, 4);
    __builtin_memcpy(reinterpret_cast<char *>(&h) + 4, &hi, 4);
    return h;
}

__device__ __forceinline__ half8 as_half8(const uint32_t * w) {
    half8 h;
    __builtin_memcpy(&h, w, 16);
    return h;
}

__device__ __forceinline__ half4 as_half4(uint32_t lo, uint32_t hi) {
    const u32x2 v = {lo, hi};
    half4 h;
    __builtin_memcpy(&h, &v, 8);
    return h;
}

// 4x4x4 MFMA whose A operand comes from block `abid` for all 16 blocks
// (CBSZ = 4).  abid must fold to a constant once the caller's loops unroll.
template <int ABID>
__device__ __forceinline__ floatx4 mfma4_bcast_t(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}

__device__ __forceinline__ floatx4 mfma4_bcast(int abid, half4 a, half4 b, floatx4 c) {
    switch (abid) {
        case 0: return mfma4_bcast_t<0>(a, b, c);
        case 1: return mfma4_bcast_t<1>(a, b, c);
        case 2: return mfma4_bcast_t<2>(a, b, c);
        case 3: return mfma4_bcast_t<3>(a, b, c);
        case 4: return mfma4_bcast_t<4>(a, b, c);
        case 5: return mfma4_bcast_t<5>(a, b, c);
        case 6: return mfma4_bcast_t<6>(a, b, c);
        case 7: return mfma4_bcast_t<7>(a, b, c);
        case 8: return mfma4_bcast_t<8>(a, b, c);
        case 9: return mfma4_bcast_t<9>(a, b, c);
        case 10: return mfma4_bcast_t<10>(a, b, c);
        case 11: return mfma4_bcast_t<11>(a, b, c);
        case 12: return mfma4_bcast_t<12>(a, b, c);
        case 13: return mfma4_bcast_t<13>(a, b, c);
        case 14: return mfma4_bcast_t<14>(a, b, c);
        default: return mfma4_bcast_t<15>(a, b, c);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void * base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// N consecutive dwords at byte offset voff + soff.
template <int N>
__device__ __forceinline__ void buf_dwords(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t * w) {
    int k = 0;
#pragma unroll
    for (; k + 4 <= N; k += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * k, soff, kNT);
        w[k] = v.x;
        w[k + 1] = v.y;
        w[k + 2] = v.z;
        w[k + 3] = v.w;
    }
    if constexpr (N % 4 == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff + 4 * (N - 3), soff, kNT);
        w[N - 3] = v.x;
        w[N - 2] = v.y;
        w[N - 1] = v.z;
    } else if constexpr (N % 4 == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 4 * (N - 2), soff, kNT);
        w[N - 2] = v.x;
        w[N - 1] = v.y;
    } else if constexpr (N % 4 == 1) {
        w[N - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * (N - 1), soff, kNT);
    }
}

template <int KB, int VB, bool QJL, bool BN>
struct step_regs {
    uint32_t kw[4 * KB];     // K code block lane/16 of tokens lane%16 + 16 tg, tg = 0..3
    uint32_t vw[kPasses][VB];  // V block (lane>>4) of token 16 pass + (lane&15)
    uint32_t ks[QJL ? 4 : 1];
    uint16_t kr;             // QJL residual norm
    uint16_t nk, nv;         // K and V norms of token lane
    // block norms: K norm of block lane/16 of token lane%16 + 16 tg; the four
    // V norms of each pass's token and (last) of token lane
    uint16_t nkb[BN ? 4 : 1];
    u32x2 nvb[BN ? kPasses + 1 : 1];
};

// Waves per SIMD the register budget is sized for: 2 (at most 256 VGPRs; two
// blocks' 78 KB of LDS fill a compute unit) for the common 3-bit MSE-only
// case, else the compiler's choice.  Throughput barely depends on occupancy
// here (one wave per SIMD already reaches most of it), so registers go to the
// pipelined step data and accumulators.
// Register sets of step data (NS - 1 steps in flight).  Two suffice: with
// 3 or 4 sets (2 waves per SIMD) the 128K layer measured the same, and a
// loads-only copy of the kernel reaches ~5.9 TB/s either way.
template <int KB, int VB, bool QJL>
constexpr int step_sets() {
    return 2;
}

template <int KB, int VB, bool QJL>
constexpr int waves_per_simd() {
    return (!QJL && VB == 3 && KB <= 3) ? 2 : 1;
}

template <int KB, int VB, bool QJL, bool BN>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 256), amdgpu_waves_per_eu(waves_per_simd<KB, VB, QJL>())))
void attend_mfma_kernel(const dev_tables kt, const dev_tables vt,
                                                          const attend_args a) {
    // BN: one norm per 32-code block for keys and values.  The logits then
    // use rows 4 blk + h of the 16x16x32 product (head h restricted to block
    // blk, hi and lo parts in two products), so each lane gets the four
    // heads' partial logits of its block, weights them by that block's norm,
    // and the row swaps that place token group tg in lane group tg also sum
    // the four blocks.  A value block is scaled by its norm over the token's
    // largest block norm (<= 1, exact enough in fp16), and the token's
    // softmax weight carries that largest norm.
    constexpr int NN = BN ? 4 : 1;  // norms per vector
    constexpr uint32_t kKcb = kD * KB / 8, kVcb = kD * VB / 8;
    // one LDS array: the 3/4-bit byte tables (keys in the low half of each
    // 256-byte entry, values in the high half) at offset 0, where a byte
    // permute yields the whole address; then the block's queries and the
    // four waves' tiles
    constexpr int kByte = (pair_table<KB>() || pair_table<VB>()) ? kByteTabBytes : 0;
    constexpr int kQStage = kG * 2 * kD * 4;  // the block's rotated queries and S q'
    __shared__ __align__(16) uint8_t lds_all[kByte + kQStage + 4 * kWaveLds];
    float * const qst = reinterpret_cast<float *>(lds_all + kByte);  // [kG][2 kD]
    uint8_t * const lds = lds_all + kByte + kQStage;
    const uint8_t * const tab_bytes = lds_all;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    uint8_t * ptile = lds + wave * kWaveLds + kStage;  // the wave's softmax weights

    int64_t L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    L = L < 0 ? 0 : (L > a.t_max ? a.t_max : L);
    const int64_t wspan = a.chunk / 4;
    const int64_t w_begin = int64_t(chunk) * a.chunk + wave * wspan;
    const int64_t w_end = w_begin + wspan < L ? w_begin + wspan : L;

    // ---- query operands.  K-step gs (0..31) covers dims of block gs/8 at
    // positions 4(gs%8)..+3; its query comes from block gs%16, i.e. lanes
    // 4(gs%16)..+3 (row = head).  This lane sources k-steps lane/4 and lane/4+16.
    // ---- per-step buffer resources.  A step's resources start at its first
    // token and end at the (batch, head)'s valid length L, so a lane whose
    // token is at or past L reads zeros: the range check of a raw buffer load
    // covers the per-lane offset, not the scalar one, so the step position
    // lives in the base address.  A step at or past the wave's end gets empty
    // resources: its loads return zeros without touching memory, and the wait
    // counts stay static.
    const uint32_t ks2 = static_cast<uint32_t>(a.k.stride[2]);
    const uint32_t vs2 = static_cast<uint32_t>(a.v.stride[2]);
    const int64_t kvec = int64_t(b) * a.k.stride[0] + int64_t(g) * a.k.stride[1];
    const int64_t vvec = int64_t(b) * a.v.stride[0] + int64_t(g) * a.v.stride[1];
    const uint8_t * const kc0 = a.k.codes + kvec * kKcb;
    const uint16_t * const kn0 = a.k.norms + kvec * NN;
    const uint8_t * const vc0 = a.v.codes + vvec * kVcb;
    const uint16_t * const vn0 = a.v.norms + vvec * NN;
    const uint8_t * const ks0 = QJL ? a.k.signs + kvec * (kD / 8) : nullptr;
    const uint16_t * const kr0 = QJL ? a.k.rnorms + kvec : nullptr;
    // per-lane byte offsets relative to the step's first token
    uint32_t vo_k[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) vo_k[tg] = uint32_t((lane & 15) + 16 * tg) * ks2 * kKcb + (lane >> 4) * 4 * KB;
    const uint32_t vo_kn = uint32_t(lane) * ks2 * 2;
    const uint32_t vo_ks = uint32_t(lane) * ks2 * (kD / 8);
    const uint32_t vo_vn = uint32_t(lane) * vs2 * 2;
    uint32_t vo_v[kPasses];
#pragma unroll
    for (int hp = 0; hp < kPasses; ++hp)
        vo_v[hp] = uint32_t(kPass * hp + 4 * (lane >> 4) + (lane & 3)) * vs2 * kVcb + ((lane >> 2) & 3) * 4 * VB;
    // block norms: K block lane/16 of token lane%16 + 16 tg; V norms of the
    // pass tokens (as above) and of token lane
    uint32_t vo_knb[BN ? 4 : 1], vo_vnb[BN ? kPasses : 1];
    if constexpr (BN) {
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) vo_knb[tg] = (uint32_t((lane & 15) + 16 * tg) * ks2 * 4 + (lane >> 4)) * 2;
#pragma unroll
        for (int hp = 0; hp < kPasses; ++hp) vo_vnb[hp] = uint32_t(kPass * hp + 4 * (lane >> 4) + (lane & 3)) * vs2 * 8;
    }

    using regs = step_regs<KB, VB, QJL, BN>;
    auto load_step = [&](int64_t j0, regs & r) {
        const int64_t j = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(j0 < w_end ? j0 : L));  // wave-uniform
        const uint32_t left = static_cast<uint32_t>(L - j);  // tokens from j to L (0 past the end)
        const int64_t kj = j * ks2, vj = j * vs2;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc0 + kj * kKcb, left * ks2 * kKcb);
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) buf_dwords<KB>(rk, vo_k[tg], 0, r.kw + KB * tg);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc0 + vj * kVcb, left * vs2 * kVcb);
#pragma unroll
        for (int hp = 0; hp < kPasses; ++hp) buf_dwords<VB>(rv, vo_v[hp], 0, r.vw[hp]);
        if constexpr (BN) {
            const __amdgpu_buffer_rsrc_t rkn = make_rsrc(kn0 + kj * 4, left * ks2 * 8);
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) r.nkb[tg] = __builtin_amdgcn_raw_buffer_load_b16(rkn, vo_knb[tg], 0, kNT);
            const __amdgpu_buffer_rsrc_t rvn = make_rsrc(vn0 + vj * 4, left * vs2 * 8);
#pragma unroll
            for (int hp = 0; hp < kPasses; ++hp) r.nvb[hp] = __builtin_amdgcn_raw_buffer_load_b64(rvn, vo_vnb[hp], 0, kNT);
            r.nvb[kPasses] = __builtin_amdgcn_raw_buffer_load_b64(rvn, vo_vn * 4, 0, kNT);
        } else {
            r.nk = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(kn0 + kj, left * ks2 * 2), vo_kn, 0, kNT);
            r.nv = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(vn0 + vj, left * vs2 * 2), vo_vn, 0, kNT);
        }
        if constexpr (QJL) {
            buf_dwords<4>(make_rsrc(ks0 + kj * (kD / 8), left * ks2 * (kD / 8)), vo_ks, 0, r.ks);
            r.kr = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(kr0 + kj, left * ks2 * 2), vo_kn, 0, kNT);
        }
    };

    // The queries are loaded first: vector-memory waits are in order, so a
    // load issued after the first step's codes would wait for them.  Then the
    // codes are in flight while the queries and tables are set up (NS
    // register sets: the steps NS - 1 ahead are in flight while one is
    // processed).
    // (a dense-rotation context has its queries rotated by the query kernel
    // beforehand: they are read from the prepared rows instead)
    float4 qv0 = {0.f, 0.f, 0.f, 0.f}, qv1 = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) {
        const int64_t qrow = int64_t(b) * a.Hq + g * kG + (lane >> 4);
        const float4 * src = reinterpret_cast<const float4 *>(
            (kt.haar ? a.qp + qrow * a.qp_stride : a.q + qrow * kD) + 8 * (lane & 15));
        qv0 = src[0];
        qv1 = src[1];
    }
    // QJL keys: this lane's half row of S (row 32 w + lane / 2), for S q'
    float4 srow[QJL ? 16 : 1];
    if constexpr (QJL) {
        const float4 * sp = reinterpret_cast<const float4 *>(kt.S + int64_t(32 * wave + (lane >> 1)) * kD + 64 * (lane & 1));
#pragma unroll
        for (int c = 0; c < 16; ++c) srow[c] = sp[c];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the codes
    constexpr int NS = step_sets<KB, VB, QJL>();
    regs rs[NS];
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) load_step(w_begin + i * kStep, rs[i]);
    const lut16 klut = make_lut(kt.cb);
    const lut16 vlut = make_lut(vt.cb);

    // byte tables: thread t writes copies 4 (t % 8) .. + 3 of entries
    // t / 8 + 32 k with one 16-byte store; entry e holds the centroids of
    // the codes in its low and high BITS bits (3-bit entries ignore bits 6, 7)
    // (centroid bits from the byte planes, not a per-lane kernel-argument
    // index, which would be a vector load)
    auto fill_byte_table = [&](const lut16 & tl, int offset, auto bits_c) {
        constexpr int B = decltype(bits_c)::value, M = (1 << B) - 1;
#pragma unroll
        for (int e = tid >> 3; e < 256; e += 32) {
            const uint32_t v = lut_bits<B>(tl, uint32_t(e & M)) | (lut_bits<B>(tl, uint32_t((e >> B) & M)) << 16);
            *reinterpret_cast<u32x4 *>(lds_all + offset + e * 256 + 16 * (tid & 7)) = u32x4{v, v, v, v};
        }
    };
    if constexpr (pair_table<KB>()) fill_byte_table(klut, 0, std::integral_constant<int, KB>{});
    if constexpr (pair_table<VB>()) fill_byte_table(vlut, 128, std::integral_constant<int, VB>{});

    // ---- rotated queries, once per block: wave 0 rotates the block's 4 heads
    // (q' = D1 H D2 q / sqrt(d), [TQ+ guide] §5.3): lane l holds coordinates
    // 8(l%16)..+7 of head l/16; three butterfly stages run in registers, four
    // across the 16 lanes of the head.  For QJL keys the four waves then form
    // S q' (rows 32 w .. 32 w + 31, two lanes per row).
    if (wave == 0 && kt.haar) {
        const int h = lane >> 4, e0 = 8 * (lane & 15);
        float4 * dst = reinterpret_cast<float4 *>(qst + h * 2 * kD + e0);
        dst[0] = qv0;
        dst[1] = qv1;
    } else if (wave == 0) {
        const int h = lane >> 4, e0 = 8 * (lane & 15);
        float v[8] = {qv0.x, qv0.y, qv0.z, qv0.w, qv1.x, qv1.y, qv1.z, qv1.w};
        // sign words picked from the (uniform) four words by selects: a
        // per-lane index into the kernel arguments would be a vector load,
        // waiting behind the codes already in flight
        const int wi = e0 >> 5;
        const uint32_t d2w = wi == 0 ? kt.d2[0] : wi == 1 ? kt.d2[1] : wi == 2 ? kt.d2[2] : kt.d2[3];
        const uint32_t d1w = wi == 0 ? kt.d1[0] : wi == 1 ? kt.d1[1] : wi == 2 ? kt.d1[2] : kt.d1[3];
        const uint32_t s2 = d2w >> (e0 & 31), s1 = d1w >> (e0 & 31);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((s2 >> i) & 1) v[i] = -v[i];
#pragma unroll
        for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & hh) == 0) {
                    const float x0 = v[i], x1 = v[i + hh];
                    v[i] = x0 + x1;
                    v[i + hh] = x0 - x1;
                }
        {
            const float sg = (lane & 1) ? -1.f : 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sg, v[i], lane_xor<1>(v[i]));
        }
        {
            const float sg = (lane & 2) ? -1.f : 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sg, v[i], lane_xor<2>(v[i]));
        }
        {
            const float sg = (lane & 4) ? -1.f : 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sg, v[i], lane_xor<4>(v[i]));
        }
        {
            const float sg = (lane & 8) ? -1.f : 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sg, v[i], lane_xor<8>(v[i]));
        }
        const float rs = 1.0f / sqrtf(float(kD));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ((s1 >> i) & 1) ? -v[i] * rs : v[i] * rs;
        float4 * dst = reinterpret_cast<float4 *>(qst + h * 2 * kD + e0);
        dst[0] = float4{v[0], v[1], v[2], v[3]};
        dst[1] = float4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();  // q' staged (and the pair tables filled)
    if constexpr (QJL) {
        const int row = 32 * wave + (lane >> 1), half = lane & 1;
        float u[kG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float4 sv = srow[c];
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const float4 qv = *reinterpret_cast<const float4 *>(qst + h * 2 * kD + 64 * half + 4 * c);
                u[h] = fmaf(sv.x, qv.x, fmaf(sv.y, qv.y, fmaf(sv.z, qv.z, fmaf(sv.w, qv.w, u[h]))));
            }
        }
#pragma unroll
        for (int h = 0; h < kG; ++h) u[h] += lane_xor<1>(u[h]);
        if (half == 0) {
#pragma unroll
            for (int h = 0; h < kG; ++h) qst[h * 2 * kD + kD + row] = u[h];
        }
        __syncthreads();
    }
    const float * const qsrc = qst;
    constexpr int64_t qstride = 2 * kD;

    // Key operand of the logits (16x16x32 MFMA, rows = query parts, columns =
    // tokens): lane l holds row l % 16 at k-slots 8 (l / 16) .. + 7 of each of
    // the 4 k-steps ks, i.e. dims 32 (l / 16) + pos(8 ks + e) of code block
    // l / 16; rows 0..3 are the fp16 hi parts of heads 0..3, rows 4..7 the lo
    // parts, rows 8..15 zero.
    half8 aqk[4], aql[BN ? 4 : 1];
    if constexpr (BN) {
        // rows 4 blk + h: head h on block blk's k-slots (lane group blk), zero
        // elsewhere; hi parts in aqk, lo parts in aql
        const int row = lane & 15, bl = lane >> 4;
        const float * qrow = qsrc + (row & 3) * qstride;
        const bool mine = (row >> 2) == bl;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = qrow[32 * bl + decoded_code_of_pos<KB>(8 * ks + e)];
                const _Float16 hi = static_cast<_Float16>(x);
                const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
                aqk[ks][e] = mine ? hi : static_cast<_Float16>(0.f);
                aql[ks][e] = mine ? lo : static_cast<_Float16>(0.f);
            }
    } else {
        const int row = lane & 15, bl = lane >> 4;
        const float * qrow = qsrc + (row & 3) * qstride;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = qrow[32 * bl + decoded_code_of_pos<KB>(8 * ks + e)];
                const _Float16 hi = static_cast<_Float16>(x);
                const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
                aqk[ks][e] = row < 4 ? hi : row < 8 ? lo : static_cast<_Float16>(0.f);
            }
    }
    // QJL keys: S q' as the broadcast A operand of the 4x4x4 sign products
    // (block gs % 16 of k-step gs holds head lane & 3 at dims of k-step gs).
    // fp16 suffices: the sketch term is a small correction weighted by the
    // residual norm, so 2^-11 relative error in S q' stays far below the
    // logit tolerance.  The signs enter as b in {0, 1} (expand_signs): the A
    // value of bit position k' carries 2^(24 - k' - E), E from the block's
    // largest |S q'| (every A value a normal fp16 below 2^15), and each head's
    // accumulator starts at -sum(S q') 2^-(E+1); scaled by 2^(E+1) it is
    // sum (S q')_i sigma_i.
    half4 au[2];
    floatx4 sq0 = {0.f, 0.f, 0.f, 0.f};
    int qe = 0;
    if constexpr (QJL) {
        // the same figures in every wave: lane l reads S q' entries l + 64 j
        // of the four heads (max), and 8 entries of head l / 16 (sum)
        float mu = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = lane + 64 * j;
            mu = fmaxf(mu, fabsf(qsrc[(f >> 7) * qstride + kD + (f & 127)]));
        }
        int ex;
        frexpf(wave_max_uniform(mu), &ex);  // the largest |S q'| < 2^ex
        qe = ex + 9;
        float su = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) su += qsrc[(lane >> 4) * qstride + kD + 8 * (lane & 15) + j];
        su += lane_xor<1>(su);
        su += lane_xor<2>(su);
        su += lane_xor<4>(su);
        su += lane_xor<8>(su);
#pragma unroll
        for (int h = 0; h < kG; ++h)
            sq0[h] = ldexpf(-__int_as_float(__builtin_amdgcn_readlane(__float_as_int(su), 16 * h)), -(qe + 1));
        const float * qrow = qsrc + (lane & 3) * qstride;
#pragma unroll
        for (int set = 0; set < 2; ++set) {
            const int gs = (lane >> 2) + 16 * set;
            const int bl = gs >> 3, kk = gs & 7;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                au[set][i] = static_cast<_Float16>(
                    ldexpf(qrow[kD + 32 * bl + sign_bit_of_pos(4 * kk + i)], 24 - sign_shift_of_pos(4 * kk + i) - qe));
        }
    }
    const uint32_t lane_off = uint32_t(lane & 31) * 4;  // pair-table copy of this lane
    const float inv_sqrt_d = 1.0f / sqrtf(float(kD));
    // logits are kept in base-2 units (scaled by log2 e), so weights are plain
    // exp2; the reference is converted back to natural units at the end
    const float kscale = a.scale * (BN ? 1.0f / sqrtf(32.f) : inv_sqrt_d) * float(M_LOG2E);
    const float qjl_gain = ldexpf(sqrtf(0.5f * float(M_PI)) / float(kD) * sqrtf(float(kD)), qe + 1);
    const float w_cap = __expf(kSlack);

    // acc[gd]: heads x dim (32 blk + 4 gd + (lane & 3)), blk = (lane >> 2) & 3,
    // summed over the tokens of quad lane >> 4 of every pass
    floatx4 acc[8];
#pragma unroll
    for (int gd = 0; gd < 8; ++gd) acc[gd] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mref[kG], lsum[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        mref[h] = -INFINITY;
        lsum[h] = 0.f;
    }

    // transposed read of the weights: lane j of 16-lane group q points at
    // token 4 q + j / 4 of the pass and receives head j % 4 of the quad's 4
    // tokens (the A operand of blocks 4 q .. 4 q + 3)
    const int p_off = (4 * (lane >> 4) + ((lane & 15) >> 2)) * 8;
    // 4x4 identity as the B operand: lane 4 b + n holds column n
    const half4 ident = as_half4((lane & 3) == 0 ? 0x3C00u : (lane & 3) == 1 ? 0x3C000000u : 0u,
                                 (lane & 3) == 2 ? 0x3C00u : (lane & 3) == 3 ? 0x3C000000u : 0u);

    auto process = [&](int64_t j0, const regs & r) {
        // ---------------- logits, 16 tokens per 16x16x32 MFMA chain: the B
        // operand of lane l is 8 decoded values of code block l / 16 of token
        // 16 tg + l % 16 (columns = tokens), so D[tg] holds the hi parts of the
        // 4 heads in lanes 0..15 and the lo parts in lanes 16..31.  Two row
        // swaps add the parts and place token group tg in row tg: lane l <- 4
        // heads of token j0 + l.
        floatx4 D[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const uint32_t * wb = r.kw + KB * tg;
            D[tg] = floatx4{0.f, 0.f, 0.f, 0.f};
            uint32_t bq[16];
            if constexpr (KB == 4) {
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    bq[p] = *reinterpret_cast<const uint32_t *>(tab_bytes + byte_pair_offset(wb, p, lane_off));
            } else if constexpr (KB == 3) {
                const block3_shifts sh = shift_block3(wb);
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    bq[p] = *reinterpret_cast<const uint32_t *>(tab_bytes + byte3_pair_offset(sh, p, lane_off));
            } else {
                unpack_block<KB>(klut, wb, bq);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                D[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqk[ks], as_half8(bq + 4 * ks), D[tg], 0, 0, 0);
                if constexpr (BN)
                    D[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aql[ks], as_half8(bq + 4 * ks), D[tg], 0, 0, 0);
            }
            if constexpr (BN) {
                const float nb = half_bits_to_float(r.nkb[tg]);   // norm of block lane/16
#pragma unroll
                for (int h = 0; h < kG; ++h) D[tg][h] *= nb;
            }
        }
        floatx4 S;
        if constexpr (BN) {
            // rows of D[tg]: lane group = block; sum the four blocks while
            // moving token group tg to lane group tg
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(D[0][h]), __float_as_uint(D[1][h]), false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(D[2][h]), __float_as_uint(D[3][h]), false, false);
                const float a01 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
                const float a23 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
                const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(a01), __float_as_uint(a23), false, false);
                S[h] = __uint_as_float(z[0]) + __uint_as_float(z[1]);
            }
        } else {
            floatx4 P0, P1;
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                // rows: D0 = [hi0, lo0, 0, 0] and D1 = [hi1, lo1, 0, 0] -> [hi0, hi1] + [lo0, lo1]
                const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(D[0][h]), __float_as_uint(D[1][h]), false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(D[2][h]), __float_as_uint(D[3][h]), false, false);
                P0[h] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
                P1[h] = __uint_as_float(y[0]) + __uint_as_float(y[1]);
                // [s0, s1, 0, 0] and [s2, s3, 0, 0] -> [s0, s1, s2, s3]
                const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(P0[h]), __float_as_uint(P1[h]), false, false);
                S[h] = __uint_as_float(z[0]);
            }
        }
        if constexpr (QJL) {
            floatx4 Sq[2] = {sq0, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int bl = 0; bl < 4; ++bl) {
                uint32_t bs[16];
                expand_signs(r.ks[bl], bs);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int gs = 8 * bl + kk;
                    const half4 bk = as_half4(bs[2 * kk], bs[2 * kk + 1]);
                    Sq[gs & 1] = mfma4_bcast(gs & 15, au[gs >> 4], bk, Sq[gs & 1]);
                }
            }
            const float gam = half_bits_to_float(r.kr) * qjl_gain;
#pragma unroll
            for (int h = 0; h < kG; ++h) S[h] = fmaf(gam, Sq[0][h] + Sq[1][h], S[h]);
        }
        // ---------------- online softmax over the wave's tokens
        const bool own = j0 + lane < w_end;
        float ks_tok, nv;
        if constexpr (BN) {
            ks_tok = own ? kscale : 0.f;
            nv = max_norm4(r.nvb[kPasses]) * (1.0f / sqrtf(32.f));
        } else {
            ks_tok = own ? half_bits_to_float(r.nk) * kscale : 0.f;
            nv = half_bits_to_float(r.nv) * inv_sqrt_d;
        }
        float s[kG], p[kG];
        bool over = false;
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            s[h] = own ? S[h] * ks_tok : -INFINITY;
            p[h] = __builtin_amdgcn_exp2f(s[h] - mref[h]);
            over |= !(p[h] * nv <= w_cap);  // also catches inf * 0 before the first max
        }
        if (__any(over)) {
            const float lam = __builtin_amdgcn_logf(fmaxf(nv, 1e-26f));  // log2
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const float mn = fmaxf(mref[h], wave_max_uniform(s[h] + lam));
                const float alpha = mref[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[h] - mn);
                mref[h] = mn;
                lsum[h] *= alpha;
#pragma unroll
                for (int gd = 0; gd < 8; ++gd) acc[gd][h] *= alpha;
                p[h] = __builtin_amdgcn_exp2f(s[h] - mn);
            }
        }
#pragma unroll
        for (int h = 0; h < kG; ++h) lsum[h] += p[h];
        *reinterpret_cast<u32x2 *>(ptile + lane * 8) =
            u32x2{uint32_t(f16_bits(p[0] * nv)) | (uint32_t(f16_bits(p[1] * nv)) << 16),
                  uint32_t(f16_bits(p[2] * nv)) | (uint32_t(f16_bits(p[3] * nv)) << 16)};

        // ---------------- values, 16 tokens per pass.  Lane 16 q + 4 blk + m
        // holds dims of block blk of token 4 q + m; a 4x4x4 MFMA against the
        // identity transposes each 4-dim group within the quad of lanes
        // (lane 4 b + n <- dim n of the quad's 4 tokens, exact), and a second
        // one multiplies by the quad's weights.
#pragma unroll
        for (int hp = 0; hp < kPasses; ++hp) {
            uint32_t o[16];
            if constexpr (VB == 4) {
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    o[p] = *reinterpret_cast<const uint32_t *>(tab_bytes + byte_pair_offset(r.vw[hp], p, lane_off | 128u));
            } else if constexpr (VB == 3) {
                const block3_shifts sh = shift_block3(r.vw[hp]);
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    o[p] = *reinterpret_cast<const uint32_t *>(tab_bytes + byte3_pair_offset(sh, p, lane_off | 128u));
            } else {
                unpack_block<VB>(vlut, r.vw[hp], o);
            }
            if constexpr (BN) {
                // this lane's block over its token's largest block norm
                const u32x2 nb = r.nvb[hp];
                const int blk = (lane >> 2) & 3;
                const float nref = max_norm4(nb);
                const uint32_t w = blk < 2 ? nb.x : nb.y;
                const float nbk = half_bits_to_float(static_cast<uint16_t>((blk & 1) ? (w >> 16) : (w & 0xFFFFu)));
                const _Float16 rt = static_cast<_Float16>(nref > 0.f ? nbk / nref : 0.f);
                half2v r2 = {rt, rt};
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    half2v v2;
                    __builtin_memcpy(&v2, &o[p], 4);
                    v2 = v2 * r2;
                    __builtin_memcpy(&o[p], &v2, 4);
                }
            }
            const half4 aw = tr_read4(ptile, kPass * hp * 8 + p_off);
            // all 8 transposes first, then the products: each product reads a
            // transpose result a few instructions later, not at once
            floatx4 t[8];
#pragma unroll
            for (int gd = 0; gd < 8; ++gd)
                t[gd] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(o[2 * gd], o[2 * gd + 1]), ident,
                                                           floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int gd = 0; gd < 8; ++gd) acc[gd] = __builtin_amdgcn_mfma_f32_4x4x4f16(aw, to_half4(t[gd]), acc[gd], 0, 0, 0);
        }
    };

    // Ping-pong register sets: step i+1 loads into the set step i is not using.
    // Loads are issued for every step so that the wait counts stay static.
    // Waves sharing a SIMD are otherwise served oldest first, which leaves the
    // youngest finishing alone; a wave drops its issue priority by one level
    // per quarter of its range done, so lagging waves catch up.
    const int64_t span = w_end > w_begin ? w_end - w_begin : 0;
    const int64_t q1 = w_begin + span / 4, q2 = w_begin + span / 2, q3 = w_end - span / 4;
    for (int64_t j0 = w_begin; j0 < w_end; j0 += NS * kStep) {
        switch (int(j0 >= q1) + int(j0 >= q2) + int(j0 >= q3)) {
            case 0: __builtin_amdgcn_s_setprio(3); break;
            case 1: __builtin_amdgcn_s_setprio(2); break;
            case 2: __builtin_amdgcn_s_setprio(1); break;
            default: __builtin_amdgcn_s_setprio(0); break;
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int64_t jj = j0 + i * kStep;
            if (i > 0 && jj >= w_end) break;
            load_step(jj + (NS - 1) * kStep, rs[(i + NS - 1) % NS]);
            process(jj, rs[i]);
        }
    }

    // ---- wave results: m, l (summed over the token lanes), acc
#pragma unroll
    for (int h = 0; h < kG; ++h) lsum[h] = wave_sum_dpp(lsum[h]);
    __syncthreads();
    // sum the four token quads (lanes 16 q + j), then lanes j < 16 hold
    // block (j >> 2) & 3, dims 4 gd + (j & 3) of it
#pragma unroll
    for (int gd = 0; gd < 8; ++gd)
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            acc[gd][h] = add_xor16(add_xor32(acc[gd][h]));
        }
    float * res = reinterpret_cast<float *>(lds + wave * kWaveLds);  // [kG][kD + 2]
    if (lane < 16) {
#pragma unroll
        for (int gd = 0; gd < 8; ++gd) {
            const int dim = 32 * ((lane >> 2) & 3) + decoded_code_of_pos<VB>(4 * gd + (lane & 3));
#pragma unroll
            for (int h = 0; h < kG; ++h) res[h * (kD + 2) + 2 + dim] = acc[gd][h];
        }
    }
    if (lane < kG) {
        res[lane * (kD + 2)] = mref[lane] * float(M_LN2);
        res[lane * (kD + 2) + 1] = lsum[lane];
    }
    __syncthreads();
    // ---- combine the four waves and write the block's partial state
    for (int i = tid; i < kG * (kD + 2); i += 256) {
        const int h = i / (kD + 2), e = i % (kD + 2);
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
            mw[wv] = reinterpret_cast<float *>(lds + wv * kWaveLds)[h * (kD + 2)];
            M = fmaxf(M, mw[wv]);
        }
        float v;
        if (e == 0) {
            v = M;
        } else {
            v = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int wv = 0; wv < 4; ++wv)
                    if (mw[wv] != -INFINITY)
                        v += __expf(mw[wv] - M) * reinterpret_cast<float *>(lds + wv * kWaveLds)[h * (kD + 2) + e];
            }
        }
        a.partial[((int64_t(b) * a.Hq + g * kG + h) * a.n_chunks + chunk) * (kD + 2) + e] = v;
    }
}

template <int KB, int VB, bool QJL>
hipError_t launch_t(const dev_tables & kt, const dev_tables & vt, const attend_args & a, hipStream_t s) {
    const dim3 grid(a.n_chunks, a.Hkv, a.B);
    if constexpr (!QJL) {
        if (kt.norm_group) {
            hipLaunchKernelGGL((attend_mfma_kernel<KB, VB, false, true>), grid, dim3(256), 0, s, kt, vt, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attend_mfma_kernel<KB, VB, QJL, false>), grid, dim3(256), 0, s, kt, vt, a);
    return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t launch_kb(const dev_tables & kt, const dev_tables & vt, const attend_args & a, hipStream_t s) {
    switch (vt.bits) {
        case 2: return launch_t<KB, 2, QJL>(kt, vt, a, s);
        case 3: return launch_t<KB, 3, QJL>(kt, vt, a, s);
        case 4: return launch_t<KB, 4, QJL>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

template <int KB, int VB, bool QJL, bool BN>
int slots_t() {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_mfma_kernel<KB, VB, QJL, BN>, 256, 0) != hipSuccess)
        per_cu = 1;
    return per_cu;
}

template <int KB, bool QJL, bool BN>
int slots_kb(int vb) {
    return vb == 2 ? slots_t<KB, 2, QJL, BN>() : vb == 3 ? slots_t<KB, 3, QJL, BN>() : slots_t<KB, 4, QJL, BN>();
}

}  // namespace

int attend_mfma_blocks_per_cu(const dev_tables & kt, const dev_tables & vt) {
    const bool bn = kt.norm_group != 0;
    switch (kt.bits) {
        case 2: return kt.qjl ? slots_kb<2, true, false>(vt.bits) : bn ? slots_kb<2, false, true>(vt.bits) : slots_kb<2, false, false>(vt.bits);
        case 3: return kt.qjl ? slots_kb<3, true, false>(vt.bits) : bn ? slots_kb<3, false, true>(vt.bits) : slots_kb<3, false, false>(vt.bits);
        case 4: return kt.qjl ? slots_kb<4, true, false>(vt.bits) : bn ? slots_kb<4, false, true>(vt.bits) : slots_kb<4, false, false>(vt.bits);
    }
    return 1;
}

int attend_mfma_chunk_quantum() { return 4 * kStep; }

bool attend_mfma_shape_ok(const dev_tables & kt, const dev_tables & vt, int32_t Hq, int32_t Hkv) {
    // keys and values both with one norm per vector, or both per 32-code
    // block; a dense rotation only with MSE-only keys (its queries come
    // prepared)
    return kt.d == kD && vt.d == kD && Hq == kG * Hkv && (!kt.qjl || kt.m == kD) && kt.norm_group == vt.norm_group &&
           (!kt.haar || !kt.qjl);
}

bool attend_mfma_supported(const dev_tables & kt, const dev_tables & vt, const attend_args & a) {
    if (!attend_mfma_shape_ok(kt, vt, a.Hq, a.Hkv)) return false;
    if (a.chunk % (4 * kStep) != 0) return false;
    // buffer sizes and per-lane offsets are 32-bit: the furthest byte of any
    // plane of one (batch, head), or of a step's 64 rows, stays below 2^31
    const int64_t row = kD * 4 / 8;  // widest code row (4 bits)
    const int64_t span = a.t_max + kStep;
    return span * a.k.stride[2] * row < (int64_t(1) << 31) && span * a.v.stride[2] * row < (int64_t(1) << 31);
}

hipError_t launch_attend_mfma_partial(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                                      hipStream_t s) {
    switch (kt.bits) {
        case 2: return kt.qjl ? launch_kb<2, true>(kt, vt, a, s) : launch_kb<2, false>(kt, vt, a, s);
        case 3: return kt.qjl ? launch_kb<3, true>(kt, vt, a, s) : launch_kb<3, false>(kt, vt, a, s);
        case 4: return kt.qjl ? launch_kb<4, true>(kt, vt, a, s) : launch_kb<4, false>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
