// Decode attention straight from packed K/V codes (general kernels).
//
//  * query prep: q' = R q once per query head, and u = S q' for QJL keys --
//    the pre-rotate-queries identity <q, R^T c> = <R q, c> ([TQ+ guide] §5.3)
//    replaces a d-point inverse rotation per cached position by one rotation
//    of the query;
//  * partial kernel (split-K over the context, "flash decoding"): logits from
//    codes, online softmax, value accumulation in the rotated domain
//    ([TQ explainer] §4.3 attention; full-precision query §2.2.2);
//  * merge kernel: log-sum-exp merge of the chunks, then the output is rotated
//    back, o = R^T o' ([TQ+ guide] §6.1, the inverse-rotation fix).
#pragma once

#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace v1 {

constexpr int kSub = 256;  // tokens per sub-tile (= threads per block)

// In-LDS Walsh-Hadamard transform of D floats by D threads (unnormalised).
template <int D>
__device__ __forceinline__ void lds_fwht(float * s, int k) {
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
        __syncthreads();
        if ((k & h) == 0) {
            float a = s[k], b = s[k + h];
            s[k] = a + b;
            s[k + h] = a - b;
        }
    }
    __syncthreads();
}

template <int D, bool QJL>
__global__ __launch_bounds__(256) void query_prep_kernel(const dev_tables t, const float * q,
                                                         float * qp, int64_t stride) {
    __shared__ float s[D];
    const int64_t i = blockIdx.x;
    const int k = threadIdx.x;
    float y;
    if (t.haar) {
        // dense rotation: q'_k = sum_j Q_kj q_j ([TQ+ guide] §4, the O(d^2) form);
        // the row's loads all issued at once and four partial sums (the
        // launch is a few dozen blocks: latency, not bandwidth, sets its time)
        s[k] = q[i * D + k];
        __syncthreads();
        const float4 * row = reinterpret_cast<const float4 *>(t.Q + int64_t(k) * D);
        float4 r[D / 4];
#pragma unroll
        for (int j = 0; j < D / 4; ++j) r[j] = row[j];
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 4; ++j)
            acc[j & 3] = fmaf(r[j].x, s[4 * j], fmaf(r[j].y, s[4 * j + 1], fmaf(r[j].z, s[4 * j + 2], fmaf(r[j].w, s[4 * j + 3], acc[j & 3]))));
        y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    } else {
        float x = q[i * D + k];
        if ((t.d2[k >> 5] >> (k & 31)) & 1) x = -x;
        s[k] = x;
        lds_fwht<D>(s, k);
        y = s[k] * (1.0f / sqrtf(static_cast<float>(D)));
        if ((t.d1[k >> 5] >> (k & 31)) & 1) y = -y;
    }
    qp[i * stride + k] = y;
    if constexpr (QJL) {
        __syncthreads();
        s[k] = y;
        __syncthreads();
        // m == d rows of S; row k
        const float * srow = t.S + int64_t(k) * D;
        float u = 0.f;
        for (int e = 0; e < D; ++e) u = fmaf(srow[e], s[e], u);
        qp[i * stride + D + k] = u;
    }
}

template <int D, int KB, int VB, bool QJL, int G>
__global__ __launch_bounds__(256) void attend_partial_kernel(const dev_tables kt, const dev_tables vt,
                                                             const attend_args a) {
    constexpr int VW = VB * D / 32;       // dwords per V code row
    constexpr int PARTS = 256 / D;        // token partitions in the PV phase
    __shared__ __align__(16) float qs[D][G];
    __shared__ __align__(16) float us[QJL ? D : 1][QJL ? G : 1];
    __shared__ __align__(16) float sc[kSub][G];
    __shared__ uint32_t vcode[kSub][VW + 1];
    __shared__ float vnb[kSub][D / 32 + 1];   // value block norms (norm_group 32)
    __shared__ float cbk[16], cbv[16];
    __shared__ float red[4][G];
    __shared__ float accred[PARTS][G][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    int64_t L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.t_max ? a.t_max : L);
    const int64_t j_begin = int64_t(chunk) * a.chunk;
    const int64_t j_end = j_begin + a.chunk < L ? j_begin + a.chunk : L;

    for (int i = tid; i < G * D; i += 256) {
        const int h = i / D, e = i % D;
        const float * row = a.qp + (int64_t(b) * a.Hq + g * G + h) * a.qp_stride;
        qs[e][h] = row[e];
        if constexpr (QJL) us[e][h] = row[D + e];
    }
    if (tid < 16) {
        cbk[tid] = kt.cb[tid];
        cbv[tid] = vt.cb[tid];
    }
    const int e_dim = tid % D, part = tid / D;
    float acc[G];
    float run_m[G], run_l[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        acc[h] = 0.f;
        run_m[h] = -INFINITY;
        run_l[h] = 0.f;
    }
    const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
    const float qjl_coef = QJL ? sqrtf(0.5f * static_cast<float>(M_PI)) / static_cast<float>(D) : 0.f;
    // one norm per 32-code block (norm_group 32): block b of a key scores
    // (N_b / sqrt(32)) <q'_b, c[code_b]>, and a value block is scaled alike
    const bool kbn = kt.norm_group != 0, vbn = vt.norm_group != 0;
    const float k_inv_len = kbn ? 1.0f / sqrtf(32.f) : inv_sqrt_d;
    const float v_inv_len = vbn ? 1.0f / sqrtf(32.f) : inv_sqrt_d;
    const int64_t kb = int64_t(b) * a.k.stride[0] + int64_t(g) * a.k.stride[1];
    const int64_t vb = int64_t(b) * a.v.stride[0] + int64_t(g) * a.v.stride[1];
    __syncthreads();

    for (int64_t j0 = j_begin; j0 < j_end; j0 += kSub) {
        const int64_t j = j0 + tid;
        const bool valid = j < j_end;
        float s[G];
        float wv_norm = 0.f;
        if (valid) {
            const int64_t kv = kb + j * a.k.stride[2];
            const uint32_t * crow = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8));
            float dot[G];
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
            for (int bl = 0; bl < D / 32; ++bl) {
                uint32_t w[KB];
#pragma unroll
                for (int k = 0; k < KB; ++k) w[k] = crow[bl * KB + k];
                float bd[G];
#pragma unroll
                for (int h = 0; h < G; ++h) bd[h] = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const float cv = cbk[block_code<KB>(w, i)];
#pragma unroll
                    for (int h = 0; h < G; ++h) bd[h] = fmaf(qs[bl * 32 + i][h], cv, bd[h]);
                }
                const float wb = kbn ? half_bits_to_float(a.k.norms[kv * (D / 32) + bl]) : 1.f;
#pragma unroll
                for (int h = 0; h < G; ++h) dot[h] = fmaf(wb, bd[h], dot[h]);
            }
            const float nk = kbn ? 1.f : half_bits_to_float(a.k.norms[kv]);
            if constexpr (QJL) {
                const uint32_t * srow = reinterpret_cast<const uint32_t *>(a.k.signs + kv * (D / 8));
                float dq[G];
#pragma unroll
                for (int h = 0; h < G; ++h) dq[h] = 0.f;
#pragma unroll
                for (int bl = 0; bl < D / 32; ++bl) {
                    const uint32_t sw = srow[bl];
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        const float sg = ((sw >> i) & 1) ? 1.f : -1.f;
#pragma unroll
                        for (int h = 0; h < G; ++h) dq[h] = fmaf(us[bl * 32 + i][h], sg, dq[h]);
                    }
                }
                const float gam = half_bits_to_float(a.k.rnorms[kv]);
#pragma unroll
                for (int h = 0; h < G; ++h)
                    s[h] = a.scale * nk * (dot[h] * inv_sqrt_d + gam * qjl_coef * dq[h]);
            } else {
#pragma unroll
                for (int h = 0; h < G; ++h) s[h] = a.scale * nk * k_inv_len * dot[h];
            }
            const int64_t vv = vb + j * a.v.stride[2];
            if (vbn) {
                wv_norm = v_inv_len;
#pragma unroll
                for (int bl = 0; bl < D / 32; ++bl) vnb[tid][bl] = half_bits_to_float(a.v.norms[vv * (D / 32) + bl]);
            } else {
                wv_norm = half_bits_to_float(a.v.norms[vv]) * inv_sqrt_d;
            }
            const uint32_t * vrow = reinterpret_cast<const uint32_t *>(a.v.codes + vv * (D * VB / 8));
#pragma unroll
            for (int k = 0; k < VW; ++k) vcode[tid][k] = vrow[k];
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = -INFINITY;
#pragma unroll
            for (int k = 0; k < VW; ++k) vcode[tid][k] = 0;
            // a slot past the length has weight 0; its block norms must be
            // finite too (0 * NaN from stale LDS would poison the sums)
            if (vbn) {
#pragma unroll
                for (int bl = 0; bl < D / 32; ++bl) vnb[tid][bl] = 0.f;
            }
        }
        // sub-tile max per head
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float m = wave_max(s[h]);
            if (lane == 0) red[wv][h] = m;
        }
        __syncthreads();
        float scale_old[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float m = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
            float new_m = fmaxf(run_m[h], m);
            scale_old[h] = run_m[h] == -INFINITY ? 0.f : __expf(run_m[h] - new_m);
            run_m[h] = new_m;
            float p = valid ? __expf(s[h] - new_m) : 0.f;
            sc[tid][h] = p * wv_norm;
            s[h] = p;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float sum = wave_sum(s[h]);
            if (lane == 0) red[wv][h] = sum;
        }
        // PV: dim e_dim over tokens part, part + PARTS, ...
        float pv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = 0.f;
        const int bit = VB * e_dim;
        const int wi = bit >> 5, off = bit & 31;
        for (int jj = part; jj < kSub; jj += PARTS) {
            uint32_t c = vcode[jj][wi] >> off;
            if (off + VB > 32) c |= vcode[jj][wi + 1] << (32 - off);
            const float cv = vbn ? cbv[c & ((1u << VB) - 1)] * vnb[jj][e_dim >> 5] : cbv[c & ((1u << VB) - 1)];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = fmaf(sc[jj][h], cv, pv[h]);
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float sum = red[0][h] + red[1][h] + red[2][h] + red[3][h];
            run_l[h] = run_l[h] * scale_old[h] + sum;
            acc[h] = acc[h] * scale_old[h] + pv[h];
        }
        __syncthreads();
    }

    // combine token partitions and write the chunk's partial state
#pragma unroll
    for (int h = 0; h < G; ++h) accred[part][h][e_dim] = acc[h];
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
        const int h = i / D, e = i % D;
        float v = 0.f;
#pragma unroll
        for (int p = 0; p < PARTS; ++p) v += accred[p][h][e];
        float * dst = a.partial + ((int64_t(b) * a.Hq + g * G + h) * a.n_chunks + chunk) * (D + 2);
        dst[2 + e] = v;
        if (e == 0) {
            dst[0] = run_m[h];
            dst[1] = run_l[h];
        }
    }
}

// Sign word i of a rotation sign vector held in the kernel arguments, picked
// by selects among the (scalar) words: indexing the argument array with a
// per-lane index would be a memory load on the critical path.
template <int D>
__device__ __forceinline__ uint32_t sign_word(const uint32_t * w, int i) {
    uint32_t r = w[0];
#pragma unroll
    for (int k = 1; k < (D + 31) / 32; ++k) r = i == k ? w[k] : r;
    return r;
}

// Log-sum-exp merge of the per-chunk states of one (batch, query head), then
// the inverse rotation o = R^T o' back to the original domain.  One pass:
// the chunks are dealt to the four waves round-robin, CB per wave per batch;
// each batch's loads (m, l and the lane's dims lane + 64 i of every chunk)
// are all issued before any is used, and the wave keeps a running maximum.
// The four waves' states are combined through LDS, and wave 0 applies R^T
// with the Walsh-Hadamard butterflies run across lanes (no block barriers).
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(const dev_tables vt, const attend_args a) {
    constexpr int PER = D >= 64 ? D / 64 : 1;  // dims per lane
    constexpr int CB = 16;                     // chunks per wave per batch
    __shared__ float wm[4], wl[4];
    __shared__ float wacc[4][PER * 64];
    __shared__ float ost[D];  // normalised rotated-domain output (dense rotation)
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float * base = a.partial + (int64_t(b) * a.Hq + h) * a.n_chunks * (D + 2);
    const int n = a.n_chunks;
    float M = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    for (int c0 = 0; c0 < n; c0 += 4 * CB) {
        float mc[CB], lc[CB], vc[CB][PER];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int c = c0 + 4 * u + wave;
            const float * p = base + int64_t(c < n ? c : 0) * (D + 2);
            mc[u] = c < n ? p[0] : -INFINITY;
            lc[u] = p[1];
#pragma unroll
            for (int i = 0; i < PER; ++i) vc[u][i] = (lane + 64 * i < D) ? p[2 + lane + 64 * i] : 0.f;
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < CB; ++u) mb = fmaxf(mb, mc[u]);
        if (mb != -INFINITY) {
            const float sc = M == -INFINITY ? 0.f : __expf(M - mb);
            l *= sc;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] *= sc;
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const float w = mc[u] == -INFINITY ? 0.f : __expf(mc[u] - mb);
                l = fmaf(w, lc[u], l);
#pragma unroll
                for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, vc[u][i], acc[i]);
            }
            M = mb;
        }
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = l;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) wacc[wave][lane + 64 * i] = acc[i];
    __syncthreads();
    const float Mx = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    float sw[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        sw[w] = wm[w] == -INFINITY ? 0.f : __expf(wm[w] - Mx);
        L = fmaf(sw[w], wl[w], L);
    }
    const bool ok = Mx != -INFINITY && L > 0.f;
    const float inv = ok ? 1.0f / L : 0.f;
    if (vt.haar) {
        // dense rotation: o = Q^T o'  ([TQ+ guide] §6.1, rotated back with
        // the value context's rotation).  o' staged in LDS by wave 0; each wave
        // then sums a quarter of the rows j for every output dim, its loads all
        // issued at once (a serial pass over j was latency-bound), and wave 0
        // adds the four parts.
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int dim = lane + 64 * i;
                if (dim < D) {
                    float o = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) o = fmaf(sw[w], wacc[w][dim], o);
                    ost[dim] = o * inv;
                }
            }
        }
        __syncthreads();
        constexpr int JW = (D + 3) / 4;  // rows per wave
        float part[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int dim = lane + 64 * i;
            const int dd = dim < D ? dim : 0;
            float qv[JW];
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) {
                const int j = wave * JW + jj;
                qv[jj] = j < D ? vt.Q[int64_t(j) * D + dd] : 0.f;
            }
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) {
                const int j = wave * JW + jj;
                const float sj = j < D ? ost[j] : 0.f;
                if (jj & 1)
                    p1 = fmaf(qv[jj], sj, p1);
                else
                    p0 = fmaf(qv[jj], sj, p0);
            }
            part[i] = p0 + p1;
        }
        __syncthreads();  // every wave has read ost: wacc is reused for the parts
#pragma unroll
        for (int i = 0; i < PER; ++i) wacc[wave][lane + 64 * i] = part[i];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int dim = lane + 64 * i;
            if (dim < D)
                a.out[(int64_t(b) * a.Hq + h) * D + dim] = (wacc[0][dim] + wacc[1][dim]) + (wacc[2][dim] + wacc[3][dim]);
        }
        return;
    }
    if (wave != 0) return;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int dim = lane + 64 * i;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) o = fmaf(sw[w], wacc[w][dim], o);
        o *= inv;
        // o_orig = R^T o = D2 . H . D1 . o / sqrt(d)
        if (dim < D && ((sign_word<D>(vt.d1, dim >> 5) >> (dim & 31)) & 1)) o = -o;
        x[i] = dim < D ? o : 0.f;
    }
    // butterflies: strides of 64 and up inside the lane, below 64 across lanes
#pragma unroll
    for (int hh = 1; hh < PER; hh <<= 1)
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if ((i & hh) == 0) {
                const float u = x[i], v = x[i + hh];
                x[i] = u + v;
                x[i + hh] = u - v;
            }
    constexpr int LANES = D >= 64 ? 64 : D;
#pragma unroll
    for (int hh = 1; hh < LANES; hh <<= 1)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float pv = __shfl_xor(x[i], hh);
            x[i] = (lane & hh) ? pv - x[i] : x[i] + pv;
        }
    const float rs = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int dim = lane + 64 * i;
        if (dim < D) {
            float y = x[i] * rs;
            if ((sign_word<D>(vt.d2, dim >> 5) >> (dim & 31)) & 1) y = -y;
            a.out[(int64_t(b) * a.Hq + h) * D + dim] = y;
        }
    }
}

template <int D, int KB, int VB, bool QJL>
hipError_t launch_attend_g(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                           hipStream_t s) {
    const dim3 grid(a.n_chunks, a.Hkv, a.B);
    const bool mfma = attend_mfma_supported(kt, vt, a);
    // the matrix-core kernel rotates its queries itself (D1.H.D2 contexts)
    if (!mfma || kt.haar) {
        hipError_t e = launch_query_prep(kt, a.q, int64_t(a.B) * a.Hq, a.qp, a.qp_stride, s);
        if (e != hipSuccess) return e;
    }
    if (mfma) {
        hipError_t e = launch_attend_mfma_partial(kt, vt, a, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((attend_merge_kernel<D>), dim3(a.Hq, a.B), dim3(256), 0, s, vt, a);
        return hipGetLastError();
    }
    switch (a.Hq / a.Hkv) {
        case 1: hipLaunchKernelGGL((attend_partial_kernel<D, KB, VB, QJL, 1>), grid, dim3(256), 0, s, kt, vt, a); break;
        case 2: hipLaunchKernelGGL((attend_partial_kernel<D, KB, VB, QJL, 2>), grid, dim3(256), 0, s, kt, vt, a); break;
        case 4: hipLaunchKernelGGL((attend_partial_kernel<D, KB, VB, QJL, 4>), grid, dim3(256), 0, s, kt, vt, a); break;
        case 8: hipLaunchKernelGGL((attend_partial_kernel<D, KB, VB, QJL, 8>), grid, dim3(256), 0, s, kt, vt, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attend_merge_kernel<D>), dim3(a.Hq, a.B), dim3(256), 0, s, vt, a);
    return hipGetLastError();
}

template <int D, int KB>
hipError_t launch_attend_kb(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                            hipStream_t s) {
    switch (vt.bits) {
        case 2: return kt.qjl ? launch_attend_g<D, KB, 2, true>(kt, vt, a, s) : launch_attend_g<D, KB, 2, false>(kt, vt, a, s);
        case 3: return kt.qjl ? launch_attend_g<D, KB, 3, true>(kt, vt, a, s) : launch_attend_g<D, KB, 3, false>(kt, vt, a, s);
        case 4: return kt.qjl ? launch_attend_g<D, KB, 4, true>(kt, vt, a, s) : launch_attend_g<D, KB, 4, false>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_attend_d(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                           hipStream_t s) {
    switch (kt.bits) {
        case 2: return launch_attend_kb<D, 2>(kt, vt, a, s);
        case 3: return launch_attend_kb<D, 3>(kt, vt, a, s);
        case 4: return launch_attend_kb<D, 4>(kt, vt, a, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_prep_d(const dev_tables & t, const float * q, int64_t n, float * qp, int64_t stride,
                         hipStream_t s) {
    if (t.qjl)
        hipLaunchKernelGGL((query_prep_kernel<D, true>), dim3(n), dim3(D), 0, s, t, q, qp, stride);
    else
        hipLaunchKernelGGL((query_prep_kernel<D, false>), dim3(n), dim3(D), 0, s, t, q, qp, stride);
    return hipGetLastError();
}

}  // namespace v1
}  // namespace tq
