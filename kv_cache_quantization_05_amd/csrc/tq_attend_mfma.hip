// Fused decode attention on matrix cores, d = 128, 4 query heads per KV head.
//
// The grouped queries sharing one KV head form a real dense contraction
// against the dequantised codes, so both products run on MFMA
// (v_mfma_f32_16x16x32_f16):
//   logits   S[h, j] = sum_i q'[h, i] c[code_ji]   (rows: 4 heads as fp16 hi
//            parts + 4 heads as fp16 lo parts, so q' keeps ~22 bits; columns:
//            16 tokens; k: the 32 codes of one block per lane group);
//   values   O[h, i] += sum_j w[h, j] c[code_ji]   (k = 32 tokens; the
//            dequantised V tile goes through LDS and comes back transposed
//            with ds_read_b64_tr_b16).
// Query rotation once per head ([TQ+ guide] §5.3), online softmax
// ([TQ explainer] §4.3), the output stays in the rotated domain until the
// merge kernel rotates it back ([TQ+ guide] §6.1).
//
// Memory: each wave streams a contiguous token range with buffer loads whose
// per-lane offsets are fixed and whose per-step offset is one scalar; the
// resource's size is the (batch, head)'s valid length, so positions past it
// read as zero.  The next step's codes are loaded while the current one is
// unpacked (ping-pong registers).
//
// Softmax bookkeeping per wave: a wave-uniform reference m per head, raised
// only when s + ln(N_v/sqrt d) exceeds it by more than kSlack (so most steps
// need no cross-lane max).  p = exp(s - m) feeds the row sum; the PV weight
// w = p * N_v/sqrt(d) <= e^kSlack stays safe in fp16 whatever the norms.
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_unpack.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;
constexpr int kStep = 32;                  // tokens per wave iteration
constexpr int kVRow = 2 * kD + 32;         // bytes per token row of the V tile (padded)
constexpr int kVTile = kStep * kVRow;      // 9216 B
constexpr int kPRow = 32;                  // 16 heads x fp16
constexpr int kPTile = kStep * kPRow;      // 1024 B
constexpr int kWaveLds = kVTile + kPTile;
constexpr float kSlack = 4.0f;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ half8 as_half8(const uint32_t * d) {
    half8 h;
    __builtin_memcpy(&h, d, 16);
    return h;
}

// Byte offset of token row r in a wave's V tile: rows are 288 B apart, with
// 16 B more for rows with bit 2 set.  The 8 rows written together by
// 16-byte stores start in 8 distinct 16-byte bank slots, and the 4 rows read
// together by ds_read_b64_tr_b16 cover the 128 bytes of banks exactly once;
// offsets stay affine in the column, so they fold into instruction offsets.
__device__ __forceinline__ int vrow_off(int r) { return r * kVRow + ((r >> 2) & 1) * 16; }

__device__ __forceinline__ half8 tr_read(const uint8_t * lds_base, int off0, int off1) {
    const shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(lds_base + off0));
    const shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(lds_base + off1));
    half8 h;
    __builtin_memcpy(&h, &a, 8);
    __builtin_memcpy(reinterpret_cast<char *>(&h) + 8, &b, 8);
    return h;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void * base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// BITS dwords of one 32-code block at byte offset voff + soff.
template <int BITS>
__device__ __forceinline__ void buf_block(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t * w) {
    if constexpr (BITS == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        w[0] = v.x;
        w[1] = v.y;
    } else if constexpr (BITS == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
    } else {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    }
}

template <int KB, int VB, bool QJL>
struct step_regs {
    uint32_t kw[2][KB];   // K block (lane group) of token tile 0 / 1
    uint32_t vw[2][VB];   // V blocks (lane >> 5) and (lane >> 5) + 2 of token lane & 31
    uint32_t ks[2];       // QJL sign words
    uint16_t kr[2];       // QJL residual norms
    uint16_t nk, nv;      // K and V norms of token lane & 31
};

template <int KB, int VB, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QJL ? 2 : 3, QJL ? 2 : 3))) void attend_mfma_kernel(const dev_tables kt, const dev_tables vt,
                                                             const attend_args a) {
    constexpr uint32_t kKcb = kD * KB / 8, kVcb = kD * VB / 8;
    __shared__ __align__(16) uint8_t lds[4 * kWaveLds];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    uint8_t * vtile = lds + wave * kWaveLds;
    uint8_t * ptile = vtile + kVTile;

    int64_t L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    L = L < 0 ? 0 : (L > a.t_max ? a.t_max : L);
    const int64_t wspan = a.chunk / 4;
    const int64_t w_begin = int64_t(chunk) * a.chunk + wave * wspan;
    const int64_t w_end = w_begin + wspan < L ? w_begin + wspan : L;

    // ---- query operands: rows 0..3 = fp16 hi part of heads 0..3, rows 4..7 = lo part
    half8 aq[4];
    half8 au[4];
    {
        const int h = lrow & 3;
        const bool lo = (lrow >> 2) == 1;
        const float live = lrow < 8 ? 1.f : 0.f;
        const float * qrow = a.qp + (int64_t(b) * a.Hq + g * kG + h) * a.qp_stride;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int dim = 32 * lgrp + block_code_of_pos<KB>(8 * mi + i);
                const float x = live * qrow[dim];
                const _Float16 hi = static_cast<_Float16>(x);
                aq[mi][i] = lo ? static_cast<_Float16>(x - static_cast<float>(hi)) : hi;
                if constexpr (QJL) {
                    const int sdim = 32 * lgrp + sign_bit_of_pos(8 * mi + i);
                    const float u = live * qrow[kD + sdim];
                    const _Float16 uh = static_cast<_Float16>(u);
                    au[mi][i] = lo ? static_cast<_Float16>(u - static_cast<float>(uh)) : uh;
                }
            }
        }
    }
    const lut16 klut = make_lut(kt.cb);
    const lut16 vlut = make_lut(vt.cb);
    const float inv_sqrt_d = 1.0f / sqrtf(float(kD));
    const float kscale = a.scale * inv_sqrt_d;
    const float qjl_gain = sqrtf(0.5f * float(M_PI)) / float(kD) * sqrtf(float(kD));

    // heads 4..15 of the weight tile stay zero
    if (lane < 32) {
        uint32_t * pr = reinterpret_cast<uint32_t *>(ptile + lane * kPRow);
#pragma unroll
        for (int k = 2; k < 8; ++k) pr[k] = 0;
    }

    floatx4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mref[kG], lsum[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        mref[h] = -INFINITY;
        lsum[h] = 0.f;
    }

    // ---- buffer resources over this (batch, KV head)'s valid positions
    const uint32_t ks2 = static_cast<uint32_t>(a.k.stride[2]);
    const uint32_t vs2 = static_cast<uint32_t>(a.v.stride[2]);
    const uint32_t Lu = static_cast<uint32_t>(L);
    const int64_t kvec = int64_t(b) * a.k.stride[0] + int64_t(g) * a.k.stride[1];
    const int64_t vvec = int64_t(b) * a.v.stride[0] + int64_t(g) * a.v.stride[1];
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k.codes + kvec * kKcb, Lu * ks2 * kKcb);
    const __amdgpu_buffer_rsrc_t rkn = make_rsrc(a.k.norms + kvec, Lu * ks2 * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v.codes + vvec * kVcb, Lu * vs2 * kVcb);
    const __amdgpu_buffer_rsrc_t rvn = make_rsrc(a.v.norms + vvec, Lu * vs2 * 2);
    __amdgpu_buffer_rsrc_t rks = rk, rkr = rk;
    if constexpr (QJL) {
        rks = make_rsrc(a.k.signs + kvec * (kD / 8), Lu * ks2 * (kD / 8));
        rkr = make_rsrc(a.k.rnorms + kvec, Lu * ks2 * 2);
    }
    // per-lane byte offsets relative to the step's first token
    uint32_t vo_k[2], vo_ks[2], vo_kr[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t tok = 16 * t + lrow;
        vo_k[t] = tok * ks2 * kKcb + lgrp * 4 * KB;
        vo_ks[t] = tok * ks2 * (kD / 8) + lgrp * 4;
        vo_kr[t] = tok * ks2 * 2;
    }
    const uint32_t own_tok = lane & 31;
    const uint32_t vo_kn = own_tok * ks2 * 2;
    const uint32_t vo_vn = own_tok * vs2 * 2;
    const uint32_t vo_v0 = own_tok * vs2 * kVcb + (lane >> 5) * 4 * VB;
    const uint32_t vo_v1 = vo_v0 + 2 * 4 * VB;

    using regs = step_regs<KB, VB, QJL>;
    auto load_step = [&](int64_t j0, regs & r) {
        const uint32_t j = static_cast<uint32_t>(j0);
        const uint32_t sk = j * ks2 * kKcb, sv = j * vs2 * kVcb;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            buf_block<KB>(rk, vo_k[t], sk, r.kw[t]);
            if constexpr (QJL) {
                r.ks[t] = __builtin_amdgcn_raw_buffer_load_b32(rks, vo_ks[t], j * ks2 * (kD / 8), 0);
                r.kr[t] = __builtin_amdgcn_raw_buffer_load_b16(rkr, vo_kr[t], j * ks2 * 2, 0);
            }
        }
        buf_block<VB>(rv, vo_v0, sv, r.vw[0]);
        buf_block<VB>(rv, vo_v1, sv, r.vw[1]);
        r.nk = __builtin_amdgcn_raw_buffer_load_b16(rkn, vo_kn, j * ks2 * 2, 0);
        r.nv = __builtin_amdgcn_raw_buffer_load_b16(rvn, vo_vn, j * vs2 * 2, 0);
    };

    // transposed-read addresses (fixed per lane)
    const int tr_row = 8 * lgrp + (lrow >> 2);
    const int tr_half = 4 * (lrow & 3);
    const int p_off0 = tr_row * kPRow + tr_half * 2;
    const int p_off1 = p_off0 + 4 * kPRow;
    const int v_off0 = vrow_off(tr_row) + tr_half * 2;
    const int v_off1 = vrow_off(tr_row + 4) + tr_half * 2;

    auto process = [&](int64_t j0, const regs & r) {
        // ---------------- logits for tokens j0 .. j0+31 (two 16-token tiles)
        floatx4 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint32_t bq[16];
            unpack_block<KB>(klut, r.kw[t], bq);
            floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[mi], as_half8(bq + 4 * mi), s, 0, 0, 0);
            if constexpr (QJL) {
                uint32_t bs[16];
                unpack_signs(r.ks[t], bs);
                floatx4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    sq = __builtin_amdgcn_mfma_f32_16x16x32_f16(au[mi], as_half8(bs + 4 * mi), sq, 0, 0, 0);
                const float gam = half_bits_to_float(r.kr[t]) * qjl_gain;
#pragma unroll
                for (int q = 0; q < 4; ++q) s[q] = fmaf(gam, sq[q], s[q]);
            }
            // hi rows (lanes 0-15) + lo rows (lanes 16-31)
#pragma unroll
            for (int q = 0; q < 4; ++q) s[q] += lane_xor<16>(s[q]);
            st[t] = s;
        }
        // lane l < 32 owns token j0 + l: tile l/16, column l%16
        const bool own = lane < 32 && j0 + lane < w_end;
        const float ks_tok = own ? half_bits_to_float(r.nk) * kscale : 0.f;
        const float nv = half_bits_to_float(r.nv) * inv_sqrt_d;
        const float lam = __logf(fmaxf(nv, 1e-26f));
        float s[kG];
        bool over = false;
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            const float v = (lane & 16) ? st[1][h] : st[0][h];
            s[h] = own ? v * ks_tok : -INFINITY;
            over |= s[h] + lam > mref[h] + kSlack;
        }
        if (__any(over)) {
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const float mn = fmaxf(mref[h], wave_max(s[h] + lam));
                const float alpha = mref[h] == -INFINITY ? 0.f : __expf(mref[h] - mn);
                mref[h] = mn;
                lsum[h] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[dt][h] *= alpha;
            }
        }
        uint32_t wp[2];
#pragma unroll
        for (int h = 0; h < kG; h += 2) {
            const float p0 = __expf(s[h] - mref[h]);
            const float p1 = __expf(s[h + 1] - mref[h + 1]);
            lsum[h] += p0;
            lsum[h + 1] += p1;
            wp[h / 2] = uint32_t(f16_bits(p0 * nv)) | (uint32_t(f16_bits(p1 * nv)) << 16);
        }
        if (lane < 32) *reinterpret_cast<u32x2 *>(ptile + lane * kPRow) = u32x2{wp[0], wp[1]};

        // ---------------- values: dequantise 32 tokens x 4 blocks into LDS
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int blk = (lane >> 5) + 2 * u;
            uint32_t o[16];
            unpack_block<VB>(vlut, r.vw[u], o);
            uint8_t * dst = vtile + vrow_off(lane & 31) + blk * 64;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *reinterpret_cast<u32x4 *>(dst + c * 16) = u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
        }
        // ---------------- O[h, :] += W[h, 32 tokens] . V[32 tokens, :]
        const half8 aw = tr_read(ptile, p_off0, p_off1);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const half8 bv = tr_read(vtile, v_off0 + 32 * dt, v_off1 + 32 * dt);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bv, acc[dt], 0, 0, 0);
        }
    };

    regs cur, nxt;
    if (w_begin < w_end) load_step(w_begin, cur);
    for (int64_t j0 = w_begin; j0 < w_end; j0 += kStep) {
        if (j0 + kStep < w_end) load_step(j0 + kStep, nxt);
        process(j0, cur);
        cur = nxt;
    }

    // ---- wave results: m, l (summed over the 32 token lanes), acc rows 0..3
#pragma unroll
    for (int h = 0; h < kG; ++h) lsum[h] = wave_sum(lsum[h]);
    __syncthreads();
    float * res = reinterpret_cast<float *>(lds + wave * kWaveLds);  // [kG][kD + 2]
    if (lane < 16) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int c = 16 * dt + lrow;  // V tile column -> rotated-domain dim
            const int dim = 32 * (c >> 5) + block_code_of_pos<VB>(c & 31);
#pragma unroll
            for (int h = 0; h < kG; ++h) res[h * (kD + 2) + 2 + dim] = acc[dt][h];
        }
    }
    if (lane < kG) {
        res[lane * (kD + 2)] = mref[lane];
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
    hipLaunchKernelGGL((attend_mfma_kernel<KB, VB, QJL>), grid, dim3(256), 0, s, kt, vt, a);
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

template <int KB, int VB, bool QJL>
int slots_t() {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_mfma_kernel<KB, VB, QJL>, 256, 0) != hipSuccess)
        per_cu = 1;
    return per_cu;
}

template <int KB, bool QJL>
int slots_kb(int vb) {
    return vb == 2 ? slots_t<KB, 2, QJL>() : vb == 3 ? slots_t<KB, 3, QJL>() : slots_t<KB, 4, QJL>();
}

}  // namespace

int attend_mfma_blocks_per_cu(const dev_tables & kt, const dev_tables & vt) {
    switch (kt.bits) {
        case 2: return kt.qjl ? slots_kb<2, true>(vt.bits) : slots_kb<2, false>(vt.bits);
        case 3: return kt.qjl ? slots_kb<3, true>(vt.bits) : slots_kb<3, false>(vt.bits);
        case 4: return kt.qjl ? slots_kb<4, true>(vt.bits) : slots_kb<4, false>(vt.bits);
    }
    return 1;
}

bool attend_mfma_shape_ok(const dev_tables & kt, const dev_tables & vt, int32_t Hq, int32_t Hkv) {
    return kt.d == kD && vt.d == kD && Hq == kG * Hkv && (!kt.qjl || kt.m == kD);
}

bool attend_mfma_supported(const dev_tables & kt, const dev_tables & vt, const attend_args & a) {
    if (!attend_mfma_shape_ok(kt, vt, a.Hq, a.Hkv)) return false;
    if (a.chunk % (4 * kStep) != 0) return false;
    // buffer offsets are 32-bit: the furthest byte of any plane of one (batch, head)
    const int64_t row = kD * 4 / 8;  // widest code row (4 bits)
    return a.t_max * a.k.stride[2] * row < (int64_t(1) << 31) &&
           a.t_max * a.v.stride[2] * row < (int64_t(1) << 31);
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
