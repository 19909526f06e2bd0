// Prefill attention over the packed cache: a block of Tq new positions per
// sequence, each attending causally to the cached positions at or before it
// ([TQ explainer] §4.3 attention; the prefill context scaling of [TQ+ guide]
// §1.2 and the flash-attention path of §5.3, with pre-rotated queries).
//
// Many queries share each key, so both products are real dense contractions
// on the 16x16x32 fp16 matrix cores, in transposed form:
//   S^T[t, q] = sum_i c[code_ti] q'[q, i]       A = dequantised keys (16
//             tokens x 32 dims, fp16-exact centroids), B = rotated queries
//             split into fp16 hi + lo (two products, ~22 bits of q');
//   O^T[i, q] += sum_t c[vcode_ti] w[t, q]      A = dequantised values
//             (16 dims x 32 tokens), B = softmax weights in fp16.
// The result layout of the first product is the operand layout of the
// second: lane l holds rows 4 (l / 16) + j of query column l % 16, and the
// key rows of a 16-token tile are permuted so that those rows are tokens
// 8 (l / 16) + j (even tile) and 8 (l / 16) + 4 + j (odd tile), i.e. the
// 8 consecutive tokens the lane supplies at k-slots 8 (l / 16) .. + 7 of
// the value product.  No data moves between the two products.
//
// A workgroup owns one (batch, KV head) and 16 NCT NW query rows (P
// positions x G heads); per 64-token tile its threads dequantise the keys
// (row major) and values (transposed) into LDS once for all NW waves.  Online
// softmax in base-2 units per query column; value norms enter the weights,
// scaled per tile by the tile's largest norm so they stay in [0, 1] in fp16.
// The output stays in the rotated domain; a second kernel rotates it back.
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_unpack.h"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPT = 64;   // tokens per KV tile

__device__ __forceinline__ f16x8 lds_f16x8(const uint16_t * p) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    f16x8 r;
    __builtin_memcpy(&r, &w, 16);
    return r;
}

// Token (within a 64-token tile) of row r of 16-row key tile rt.
__device__ __forceinline__ int tile_token(int rt, int r) {
    return 32 * (rt >> 1) + 8 * (r >> 2) + 4 * (rt & 1) + (r & 3);
}

// Two waves per SIMD for MSE-only keys (the query operands and accumulators
// of two column tiles, plus the prefetched codes, fit 256 registers); QJL
// keys add S q' operands and run one.
template <bool QJL>
constexpr int prefill_waves() { return QJL ? 1 : 2; }

template <int D, int KB, int VB, bool QJL, int NCT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(prefill_waves<QJL>()))) void prefill_kernel(const dev_tables kt, const dev_tables vt, const prefill_args a) {
    constexpr int KS = D / 32;          // k-steps of the logits
    constexpr int DT = D / 16;          // 16-dim tiles of the output
    constexpr int KRS = D + 8;          // key rows in LDS (halves): rows 16 B apart in the banks
    constexpr int VRS = kPT + 8;        // value rows (one per dim) in LDS
    __shared__ __align__(16) uint16_t klds[kPT * KRS];
    __shared__ __align__(16) uint16_t vlds[D * VRS];
    __shared__ __align__(16) float knl[kPT], vnl[kPT], krl[QJL ? kPT : 1];
    __shared__ uint32_t ksl[QJL ? kPT : 1][QJL ? D / 32 : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int rows = 16 * NW * NCT;                // query rows of the workgroup
    const int P = rows / G;                        // positions of the workgroup
    const int qt = gridDim.x - 1 - blockIdx.x;     // latest positions (most keys) first
    const int g = blockIdx.y, b = blockIdx.z;
    int64_t L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.t_max ? a.t_max : L);
    const int64_t base_pos = L - a.Tq;             // position of query 0

    // this lane's query column in each column tile
    int64_t qrow[NCT], qpos[NCT];
    bool qvalid[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int r = 16 * (NCT * wave + ct) + c16;
        const int h = g * G + r / P;
        const int64_t i = int64_t(qt) * P + r % P;
        qvalid[ct] = i < a.Tq;
        qrow[ct] = (int64_t(b) * a.Hq + h) * a.Tq + (qvalid[ct] ? i : 0);
        qpos[ct] = base_pos + i;
    }
    const int64_t last = base_pos + int64_t(qt) * P + P - 1;   // latest position of the workgroup
    const int64_t kend = last + 1 < L ? last + 1 : L;           // keys the workgroup needs

    // B operands: q' as fp16 hi + lo at dims 32 ks + 8 g4 .. + 7 (and S q')
    f16x8 qh[NCT][KS], ql[NCT][KS], qu[NCT][QJL ? KS : 1];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const float * src = a.qp + qrow[ct] * a.qp_stride;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 x0 = *reinterpret_cast<const float4 *>(src + 32 * ks + 8 * g4);
            const float4 x1 = *reinterpret_cast<const float4 *>(src + 32 * ks + 8 * g4 + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const _Float16 hi = static_cast<_Float16>(xs[j]);
                qh[ct][ks][j] = hi;
                ql[ct][ks][j] = static_cast<_Float16>(xs[j] - static_cast<float>(hi));
            }
            if constexpr (QJL) {
                const float4 u0 = *reinterpret_cast<const float4 *>(src + D + 32 * ks + 8 * g4);
                const float4 u1 = *reinterpret_cast<const float4 *>(src + D + 32 * ks + 8 * g4 + 4);
                const float us[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) qu[ct][ks][j] = static_cast<_Float16>(us[j]);
            }
        }
    }
    const lut16 klut = make_lut(kt.cb), vlut = make_lut(vt.cb);
    const float inv_sqrt_d = 1.0f / sqrtf(float(D));
    const float qjl_coef = sqrtf(0.5f * float(M_PI)) / float(D);
    const float s2scale = a.scale * float(M_LOG2E);   // logits in base-2 units

    f32x4 acc[NCT][DT];
    float m_run[NCT], l_run[NCT];
    float vrun = 0.f;   // running largest value weight scale: acc is in units of it
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        m_run[ct] = -INFINITY;
        l_run[ct] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int64_t kvb = int64_t(b) * a.k.stride[0] + int64_t(g) * a.k.stride[1];
    const int64_t vvb = int64_t(b) * a.v.stride[0] + int64_t(g) * a.v.stride[1];

    // The next tile's codes, signs and norms are loaded into registers while
    // the current tile is processed (each thread decodes the same units of
    // every tile: unit u = (token u % kPT, block u / kPT), u = tid + 256 i).
    constexpr int kUnits = kPT * KS;
    constexpr int UPT = (kUnits + 255) / 256;
    uint32_t kwn[UPT][KB], vwn[UPT][VB], ksn[UPT];
    uint16_t knn[UPT], krn[UPT], vnn[UPT];
    auto load_tile = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + 256 * i;
            if (u >= kUnits) break;
            const int tt = u % kPT, bl = u / kPT;
            const int64_t t = t0 + tt;
            const bool ok = t < kend;
            const int64_t kv = kvb + (ok ? t : 0) * a.k.stride[2];
            const int64_t vv = vvb + (ok ? t : 0) * a.v.stride[2];
            const uint32_t * kc = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8)) + bl * KB;
            const uint32_t * vc = reinterpret_cast<const uint32_t *>(a.v.codes + vv * (D * VB / 8)) + bl * VB;
#pragma unroll
            for (int k = 0; k < KB; ++k) kwn[i][k] = ok ? kc[k] : 0u;
#pragma unroll
            for (int k = 0; k < VB; ++k) vwn[i][k] = ok ? vc[k] : 0u;
            if constexpr (QJL) ksn[i] = ok ? reinterpret_cast<const uint32_t *>(a.k.signs + kv * (D / 8))[bl] : 0u;
            if (bl == 0) {
                knn[i] = ok ? a.k.norms[kv] : uint16_t(0);
                vnn[i] = ok ? a.v.norms[vv] : uint16_t(0);
                if constexpr (QJL) krn[i] = ok ? a.k.rnorms[kv] : uint16_t(0);
            }
        }
    };
    if (kend > 0) load_tile(0);

    for (int64_t t0 = 0; t0 < kend; t0 += kPT) {
        __syncthreads();   // the previous tile's LDS reads are done
        // ---- dequantise the tile: unit (token, 32-code block), a wave's 64
        // lanes taking one block of the tile's 64 tokens, so the transposed
        // value stores of one instruction fill consecutive halves of one row
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + 256 * i;
            if (u >= kUnits) break;
            const int tt = u % kPT, bl = u / kPT;
            const bool ok = t0 + tt < kend;
            {
                uint32_t kp[16];
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    uint32_t sel = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) sel |= block_code<KB>(kwn[i], 4 * q4 + j) << (8 * j);
                    lut4<KB>(klut, sel, kp[2 * q4], kp[2 * q4 + 1]);
                }
                uint4 * kd = reinterpret_cast<uint4 *>(&klds[tt * KRS + 32 * bl]);
#pragma unroll
                for (int c = 0; c < 4; ++c) kd[c] = uint4{kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]};
                if constexpr (QJL) ksl[tt][bl] = ksn[i];
                if (bl == 0) {
                    // per-token factors: the key norm with the logit scale (base
                    // 2) and 1/sqrt(d); the QJL term's gamma sqrt(pi/2)/m on top
                    const float nk = ok ? half_bits_to_float(knn[i]) * s2scale : 0.f;
                    knl[tt] = nk * inv_sqrt_d;
                    if constexpr (QJL) krl[tt] = ok ? half_bits_to_float(krn[i]) * qjl_coef * nk : 0.f;
                }
            }
            {
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    uint32_t vsel = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) vsel |= block_code<VB>(vwn[i], 4 * q4 + j) << (8 * j);
                    uint32_t v0, v1;
                    lut4<VB>(vlut, vsel, v0, v1);
                    const int dim0 = 32 * bl + 4 * q4;
                    vlds[(dim0 + 0) * VRS + tt] = static_cast<uint16_t>(v0);
                    vlds[(dim0 + 1) * VRS + tt] = static_cast<uint16_t>(v0 >> 16);
                    vlds[(dim0 + 2) * VRS + tt] = static_cast<uint16_t>(v1);
                    vlds[(dim0 + 3) * VRS + tt] = static_cast<uint16_t>(v1 >> 16);
                }
                if (bl == 0) vnl[tt] = ok ? half_bits_to_float(vnn[i]) * inv_sqrt_d : 0.f;
            }
        }
        if (t0 + kPT < kend) load_tile(t0 + kPT);
        __syncthreads();
        // the running largest value weight scale (weights stay in [0, 1] in
        // fp16); the same in every wave of the workgroup
        float vmax = vnl[lane];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
        const float vnew = fmaxf(vrun, vmax);
        const float vrescale = vnew > vrun && vrun > 0.f ? vrun / vnew : 1.f;   // acc to the new units
        vrun = vnew;
        const float inv_v = vrun > 0.f ? 1.0f / vrun : 0.f;
        // per-token factors of this lane's 16 tokens (4 consecutive per key tile)
        float4 kf[4], vf[4], kq[QJL ? 4 : 1];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int t4 = 32 * (rt >> 1) + 8 * g4 + 4 * (rt & 1);
            kf[rt] = *reinterpret_cast<const float4 *>(&knl[t4]);
            vf[rt] = *reinterpret_cast<const float4 *>(&vnl[t4]);
            if constexpr (QJL) kq[rt] = *reinterpret_cast<const float4 *>(&krl[t4]);
        }
        const bool tile_full = t0 + kPT <= kend;

#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            // ---- logits S^T for 4 key tiles of 16 tokens
            f32x4 s[4], su[QJL ? 4 : 1];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                s[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (QJL) su[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int tr = tile_token(rt, c16);   // the key row this lane supplies
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8 ak = lds_f16x8(&klds[tr * KRS + 32 * ks + 8 * g4]);
                    s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qh[ct][ks], s[rt], 0, 0, 0);
                    s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, ql[ct][ks], s[rt], 0, 0, 0);
                    if constexpr (QJL) {
                        const uint32_t byte = (ksl[tr][ks] >> (8 * g4)) & 0xFFu;
                        f16x8 sg;
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            sg[j] = ((byte >> j) & 1u) ? static_cast<_Float16>(1.f) : static_cast<_Float16>(-1.f);
                        su[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sg, qu[ct][ks], su[rt], 0, 0, 0);
                    }
                }
            }
            // ---- scale, mask, running maximum (base 2); tiles wholly below
            // every column's position need no mask
            float x[4][4];
            float mt = -INFINITY;
            const bool nomask = __all(qvalid[ct] && tile_full && t0 + kPT - 1 <= qpos[ct]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v = s[rt][j] * kf[rt][j];
                    if constexpr (QJL) v = fmaf(kq[rt][j], su[rt][j], v);
                    if (!nomask) {
                        const int64_t t = t0 + 32 * (rt >> 1) + 8 * g4 + 4 * (rt & 1) + j;
                        v = (qvalid[ct] && t <= qpos[ct] && t < kend) ? v : -INFINITY;
                    }
                    x[rt][j] = v;
                    mt = fmaxf(mt, v);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // (no branch per column: a column with nothing visible yet gets
            // zero weights, and the matrix products stay wave-uniform)
            const float m_new = fmaxf(m_run[ct], mt);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float corr = m_run[ct] == -INFINITY ? 0.f : exp2f(m_run[ct] - m_new);
            m_run[ct] = m_new;
            float ps = 0.f;
            f16x8 w[2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(x[rt][j] - m_use);
                    ps += p;
                    w[rt >> 1][4 * (rt & 1) + j] = static_cast<_Float16>(p * (vf[rt][j] * inv_v));
                }
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            l_run[ct] = l_run[ct] * corr + ps;
            // ---- O^T += V^T W (value norms folded into the weights, in units
            // of the running scale); the rescale is skipped when no column of
            // the wave needs one (the common case once the maxima settle)
            const float pre = corr * vrescale;
            if (!__all(pre == 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[ct][dt] *= pre;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const f16x8 av = lds_f16x8(&vlds[(16 * dt + c16) * VRS + 32 * k2 + 8 * g4]);
                    acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, w[k2], acc[ct][dt], 0, 0, 0);
                }
            }
        }
    }
    // ---- normalise and store the rotated-domain rows (dims 16 dt + 4 g4 + j)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        if (!qvalid[ct]) continue;
        const float inv = l_run[ct] > 0.f ? vrun / l_run[ct] : 0.f;
        float * dst = a.out_rot + qrow[ct] * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * g4) =
                float4{acc[ct][dt][0] * inv, acc[ct][dt][1] * inv, acc[ct][dt][2] * inv, acc[ct][dt][3] * inv};
    }
}

// The same prefill on 32x32x16 fp16 matrix cores (MSE-only keys, d = 64 or
// 128), which deliver twice the products per clock of the 16x16x32 form.
// A wave owns 32 query rows; per 32-token half of a 64-token tile:
//   S^T[t, q] = sum_i c[code_ti] q'[q, i]    A = keys (32 tokens x 16 dims,
//             row r = token r of the half), B = q' as fp16 hi + lo;
//   the result gives lane l the 16 tokens 8 i + 4 (l / 32) + j (register
//   4 i + j) of query column l % 32;
//   O^T[i, q] += sum_t c[vcode_ti] w[t, q]   A = values (32 dims x 16
//             tokens), B = weights: k-step s takes registers 8 s .. 8 s + 7
//             of the lane, i.e. tokens 16 s + 8 (m / 4) + 4 (l / 32) + m % 4
//             at k-slot 8 (l / 32) + m; the transposed value rows store token
//             t at column t with bits 2 and 3 swapped, so each lane's 8
//             k-slots are 8 consecutive halves of its dim row.
// No data moves between the two products, as in the 16x16 kernel.
__device__ __forceinline__ int value_column(int tt) {
    return (tt & ~12) | ((tt & 4) << 1) | ((tt & 8) >> 1);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill32_kernel(const dev_tables kt, const dev_tables vt, const prefill_args a) {
    constexpr int NW = 4;               // waves, 32 query rows each
    constexpr int KS = D / 16;          // k-steps of the logits
    constexpr int DT = D / 32;          // 32-dim tiles of the output
    constexpr int KRS = D + 8;          // key rows in LDS (halves)
    constexpr int VRS = kPT + 8;        // value rows (one per dim) in LDS
    __shared__ __align__(16) uint16_t klds[kPT * KRS];
    __shared__ __align__(16) uint16_t vlds[D * VRS];
    __shared__ __align__(16) float knl[kPT], vnl[kPT];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, h2 = lane >> 5;
    const int G = a.Hq / a.Hkv;
    constexpr int rows = 32 * NW;                  // query rows of the workgroup
    const int P = rows / G;                        // positions of the workgroup
    const int qt = gridDim.x - 1 - blockIdx.x;     // latest positions (most keys) first
    const int g = blockIdx.y, b = blockIdx.z;
    int64_t L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.t_max ? a.t_max : L);
    const int64_t base_pos = L - a.Tq;             // position of query 0

    // this lane's query column
    const int r = 32 * wave + c32;
    const int64_t qi = int64_t(qt) * P + r % P;
    const bool qvalid = qi < a.Tq;
    const int64_t qrow = (int64_t(b) * a.Hq + g * G + r / P) * a.Tq + (qvalid ? qi : 0);
    const int64_t qpos = base_pos + qi;
    const int64_t last = base_pos + int64_t(qt) * P + P - 1;   // latest position of the workgroup
    const int64_t kend = last + 1 < L ? last + 1 : L;           // keys the workgroup needs

    // B operands: q' as fp16 hi + lo at dims 16 ks + 8 h2 .. + 7
    f16x8 qh[KS], ql[KS];
    {
        const float * src = a.qp + qrow * a.qp_stride;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 x0 = *reinterpret_cast<const float4 *>(src + 16 * ks + 8 * h2);
            const float4 x1 = *reinterpret_cast<const float4 *>(src + 16 * ks + 8 * h2 + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const _Float16 hi = static_cast<_Float16>(xs[j]);
                qh[ks][j] = hi;
                ql[ks][j] = static_cast<_Float16>(xs[j] - static_cast<float>(hi));
            }
        }
    }
    const lut16 klut = make_lut(kt.cb), vlut = make_lut(vt.cb);
    const float inv_sqrt_d = 1.0f / sqrtf(float(D));
    const float s2scale = a.scale * float(M_LOG2E);   // logits in base-2 units

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    float vrun = 0.f;   // running largest value weight scale: acc is in units of it
    const int64_t kvb = int64_t(b) * a.k.stride[0] + int64_t(g) * a.k.stride[1];
    const int64_t vvb = int64_t(b) * a.v.stride[0] + int64_t(g) * a.v.stride[1];

    // the next tile's codes and norms are loaded into registers while the
    // current tile is processed (unit u = (token u % kPT, block u / kPT))
    constexpr int kUnits = kPT * (D / 32);
    constexpr int UPT = (kUnits + 255) / 256;
    uint32_t kwn[UPT][KB], vwn[UPT][VB];
    uint16_t knn[UPT], vnn[UPT];
    auto load_tile = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + 256 * i;
            if (u >= kUnits) break;
            const int tt = u % kPT, bl = u / kPT;
            const int64_t t = t0 + tt;
            const bool ok = t < kend;
            const int64_t kv = kvb + (ok ? t : 0) * a.k.stride[2];
            const int64_t vv = vvb + (ok ? t : 0) * a.v.stride[2];
            const uint32_t * kc = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8)) + bl * KB;
            const uint32_t * vc = reinterpret_cast<const uint32_t *>(a.v.codes + vv * (D * VB / 8)) + bl * VB;
#pragma unroll
            for (int k = 0; k < KB; ++k) kwn[i][k] = ok ? kc[k] : 0u;
#pragma unroll
            for (int k = 0; k < VB; ++k) vwn[i][k] = ok ? vc[k] : 0u;
            if (bl == 0) {
                knn[i] = ok ? a.k.norms[kv] : uint16_t(0);
                vnn[i] = ok ? a.v.norms[vv] : uint16_t(0);
            }
        }
    };
    if (kend > 0) load_tile(0);

    for (int64_t t0 = 0; t0 < kend; t0 += kPT) {
        __syncthreads();   // the previous tile's LDS reads are done
        // ---- dequantise the tile (as in the 16x16 kernel; value columns
        // permuted by value_column)
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + 256 * i;
            if (u >= kUnits) break;
            const int tt = u % kPT, bl = u / kPT;
            const bool ok = t0 + tt < kend;
            {
                uint32_t kp[16];
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    uint32_t sel = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) sel |= block_code<KB>(kwn[i], 4 * q4 + j) << (8 * j);
                    lut4<KB>(klut, sel, kp[2 * q4], kp[2 * q4 + 1]);
                }
                uint4 * kd = reinterpret_cast<uint4 *>(&klds[tt * KRS + 32 * bl]);
#pragma unroll
                for (int c = 0; c < 4; ++c) kd[c] = uint4{kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]};
                if (bl == 0) knl[tt] = ok ? half_bits_to_float(knn[i]) * s2scale * inv_sqrt_d : 0.f;
            }
            {
                const int col = value_column(tt);
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    uint32_t vsel = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) vsel |= block_code<VB>(vwn[i], 4 * q4 + j) << (8 * j);
                    uint32_t v0, v1;
                    lut4<VB>(vlut, vsel, v0, v1);
                    const int dim0 = 32 * bl + 4 * q4;
                    vlds[(dim0 + 0) * VRS + col] = static_cast<uint16_t>(v0);
                    vlds[(dim0 + 1) * VRS + col] = static_cast<uint16_t>(v0 >> 16);
                    vlds[(dim0 + 2) * VRS + col] = static_cast<uint16_t>(v1);
                    vlds[(dim0 + 3) * VRS + col] = static_cast<uint16_t>(v1 >> 16);
                }
                if (bl == 0) vnl[tt] = ok ? half_bits_to_float(vnn[i]) * inv_sqrt_d : 0.f;
            }
        }
        if (t0 + kPT < kend) load_tile(t0 + kPT);
        __syncthreads();
        // the running largest value weight scale (weights stay in [0, 1] in
        // fp16); the same in every wave of the workgroup
        float vmax = vnl[lane];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
        const float vnew = fmaxf(vrun, vmax);
        const float vrescale = vnew > vrun && vrun > 0.f ? vrun / vnew : 1.f;   // acc to the new units
        vrun = vnew;
        const float inv_v = vrun > 0.f ? 1.0f / vrun : 0.f;

#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int tb = 32 * th;   // the half's first token in the tile
            // ---- logits S^T for the half's 32 tokens
            f32x16 s = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 ak = lds_f16x8(&klds[(tb + c32) * KRS + 16 * ks + 8 * h2]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qh[ks], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, ql[ks], s, 0, 0, 0);
            }
            // ---- scale, mask, running maximum (base 2); halves wholly below
            // every column's position need no mask
            const bool nomask = __all(qvalid && t0 + tb + 31 < kend && t0 + tb + 31 <= qpos);
            float x[16];
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 kf = *reinterpret_cast<const float4 *>(&knl[tb + 8 * i + 4 * h2]);
                const float kfs[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v = s[4 * i + j] * kfs[j];
                    if (!nomask) {
                        const int64_t t = t0 + tb + 8 * i + 4 * h2 + j;
                        v = (qvalid && t <= qpos && t < kend) ? v : -INFINITY;
                    }
                    x[4 * i + j] = v;
                    mt = fmaxf(mt, v);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float corr = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
            m_run = m_new;
            float ps = 0.f;
            f16x8 w[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 vf = *reinterpret_cast<const float4 *>(&vnl[tb + 8 * i + 4 * h2]);
                const float vfs[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(x[4 * i + j] - m_use);
                    ps += p;
                    w[i >> 1][4 * (i & 1) + j] = static_cast<_Float16>(p * (vfs[j] * inv_v));
                }
            }
            ps += __shfl_xor(ps, 32);
            // the value-scale change applies once per tile (first half)
            const float pre = corr * (th == 0 ? vrescale : 1.f);
            l_run = l_run * corr + ps;
            if (!__all(pre == 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= pre;
            }
            // ---- O^T += V^T W
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int ss = 0; ss < 2; ++ss) {
                    const f16x8 av = lds_f16x8(&vlds[(32 * dt + c32) * VRS + tb + 16 * ss + 8 * h2]);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, w[ss], acc[dt], 0, 0, 0);
                }
            }
        }
    }
    // ---- normalise and store the rotated-domain row (dims 32 dt + 8 i + 4 h2 + j)
    if (qvalid) {
        const float inv = l_run > 0.f ? vrun / l_run : 0.f;
        float * dst = a.out_rot + qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<float4 *>(dst + 32 * dt + 8 * i + 4 * h2) =
                    float4{acc[dt][4 * i] * inv, acc[dt][4 * i + 1] * inv, acc[dt][4 * i + 2] * inv,
                           acc[dt][4 * i + 3] * inv};
    }
}

// o = R^T o' per row: D2 H D1 o' / sqrt(d) for the structured rotation, or
// Q^T o' for the dense one ([TQ+ guide] §6.1, the inverse-rotation fix).
template <int D>
__global__ __launch_bounds__(256) void rotate_back_kernel(const dev_tables t, const float * src, float * dst) {
    __shared__ float s[D];
    const int64_t row = blockIdx.x;
    const int k = threadIdx.x;
    float x = src[row * D + k];
    if (t.haar) {
        s[k] = x;
        __syncthreads();
        float o = 0.f;
        for (int j = 0; j < D; ++j) o = fmaf(t.Q[int64_t(j) * D + k], s[j], o);
        dst[row * D + k] = o;
        return;
    }
    if ((t.d1[k >> 5] >> (k & 31)) & 1) x = -x;
    s[k] = x;
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
        __syncthreads();
        if ((k & h) == 0) {
            const float u = s[k], v = s[k + h];
            s[k] = u + v;
            s[k + h] = u - v;
        }
    }
    __syncthreads();
    float y = s[k] * (1.0f / sqrtf(float(D)));
    if ((t.d2[k >> 5] >> (k & 31)) & 1) y = -y;
    dst[row * D + k] = y;
}

template <int D, int KB, int VB, bool QJL>
hipError_t launch_t(const dev_tables & kt, const dev_tables & vt, const prefill_args & a, hipStream_t s) {
    // four waves per workgroup (eight sharing each dequantised tile measured
    // 16% slower at 8K); one column tile per wave at d = 256, where the query
    // operands and accumulators of two would fill the registers
    constexpr int NCT = D >= 256 ? 1 : 2;
    constexpr int NW = 4;
    const int G = a.Hq / a.Hkv;
    const int P = 16 * NW * NCT / G;
    const int64_t tiles = (a.Tq + P - 1) / P;
    const dim3 grid(static_cast<uint32_t>(tiles), a.Hkv, a.B);
    // MSE-only keys at d <= 128: the 32x32x16 kernel (128 query rows per
    // workgroup, the same grid)
    if constexpr (!QJL && D <= 128) {
        static_assert(16 * NW * NCT == 128, "both kernels take 128 query rows per workgroup");
        hipLaunchKernelGGL((prefill32_kernel<D, KB, VB>), grid, dim3(256), 0, s, kt, vt, a);
    } else {
        hipLaunchKernelGGL((prefill_kernel<D, KB, VB, QJL, NCT, NW>), grid, dim3(64 * NW), 0, s, kt, vt, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((rotate_back_kernel<D>), dim3(static_cast<uint32_t>(int64_t(a.B) * a.Hq * a.Tq)), dim3(D), 0, s,
                       vt, a.out_rot, a.out);
    return hipGetLastError();
}

template <int D, int KB>
hipError_t launch_kb(const dev_tables & kt, const dev_tables & vt, const prefill_args & a, hipStream_t s) {
    switch (vt.bits * 2 + (kt.qjl ? 1 : 0)) {
        case 4: return launch_t<D, KB, 2, false>(kt, vt, a, s);
        case 5: return launch_t<D, KB, 2, true>(kt, vt, a, s);
        case 6: return launch_t<D, KB, 3, false>(kt, vt, a, s);
        case 7: return launch_t<D, KB, 3, true>(kt, vt, a, s);
        case 8: return launch_t<D, KB, 4, false>(kt, vt, a, s);
        case 9: return launch_t<D, KB, 4, true>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const dev_tables & kt, const dev_tables & vt, const prefill_args & a, hipStream_t s) {
    switch (kt.bits) {
        case 2: return launch_kb<D, 2>(kt, vt, a, s);
        case 3: return launch_kb<D, 3>(kt, vt, a, s);
        case 4: return launch_kb<D, 4>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(const dev_tables & kt, const dev_tables & vt) {
    return (kt.d == 64 || kt.d == 128 || kt.d == 256) && !kt.norm_group && !vt.norm_group && (!kt.qjl || kt.m == kt.d);
}

hipError_t launch_prefill(const dev_tables & kt, const dev_tables & vt, const prefill_args & a, hipStream_t s) {
    hipError_t e = launch_query_prep(kt, a.q, int64_t(a.B) * a.Hq * a.Tq, a.qp, a.qp_stride, s);
    if (e != hipSuccess) return e;
    switch (kt.d) {
        case 64: return launch_d<64>(kt, vt, a, s);
        case 128: return launch_d<128>(kt, vt, a, s);
        case 256: return launch_d<256>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
