// Scores of rotated queries against packed keys, and fused top-k search.
//
// s = scale * N * ( <R q, c[code]> / sqrt(d) + gamma sqrt(pi/2)/m <S R q, sigma> )
// read straight from the codes: the query is rotated once ([TQ+ guide] §5.3,
// pre-rotate-queries), stays at full precision ([TQ explainer] §2.2.2), and
// the QJL sign bits enter as +-1 ([TQ explainer] §2.2; [Orión plan] Fase 3).
// Inner-product search over a database of packed vectors follows the pages'
// vector-search use ([TQ explainer] §3.4); the score matrix is never stored:
// each block keeps a running top-k per query in LDS, a final pass merges the
// per-range lists (ties -> lower index).
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_unpack.h"

namespace tq {
namespace {

constexpr int kKeys = 256;   // keys per block sub-tile (one per thread)
constexpr int kQT = 16;      // queries per block

template <int D, int KB, bool QJL>
__device__ __forceinline__ void score_key(const dev_tables & t, const scores_args & a, const float (*qs)[kQT],
                                          const float (*us)[kQT], const float * cb, int64_t j,
                                          float (&out)[kQT]) {
    const int64_t kv = j * a.k.stride[2];
    const uint32_t * crow = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8));
    float dot[kQT];
#pragma unroll
    for (int i = 0; i < kQT; ++i) dot[i] = 0.f;
    // one norm per 32-code block (norm_group 32): block b weighs in with
    // N_b / sqrt(32) instead of one N / sqrt(d)
    const bool bn = t.norm_group != 0;
#pragma unroll 1
    for (int bl = 0; bl < D / 32; ++bl) {
        uint32_t w[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) w[k] = crow[bl * KB + k];
        float bd[kQT];
#pragma unroll
        for (int i = 0; i < kQT; ++i) bd[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float cv = cb[block_code<KB>(w, e)];
#pragma unroll
            for (int i = 0; i < kQT; ++i) bd[i] = fmaf(qs[bl * 32 + e][i], cv, bd[i]);
        }
        const float wb = bn ? half_bits_to_float(a.k.norms[kv * (D / 32) + bl]) : 1.f;
#pragma unroll
        for (int i = 0; i < kQT; ++i) dot[i] = fmaf(wb, bd[i], dot[i]);
    }
    const float n = bn ? 1.f : half_bits_to_float(a.k.norms[kv]);
    const float inv_sqrt_d = bn ? 1.0f / sqrtf(32.f) : 1.0f / sqrtf(static_cast<float>(D));
    if constexpr (QJL) {
        const uint32_t * srow = reinterpret_cast<const uint32_t *>(a.k.signs + kv * (D / 8));
        float dq[kQT];
#pragma unroll
        for (int i = 0; i < kQT; ++i) dq[i] = 0.f;
#pragma unroll 1
        for (int bl = 0; bl < D / 32; ++bl) {
            const uint32_t sw = srow[bl];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float sg = ((sw >> e) & 1) ? 1.f : -1.f;
#pragma unroll
                for (int i = 0; i < kQT; ++i) dq[i] = fmaf(us[bl * 32 + e][i], sg, dq[i]);
            }
        }
        const float gam = half_bits_to_float(a.k.rnorms[kv]) * sqrtf(0.5f * static_cast<float>(M_PI)) /
                          static_cast<float>(D);
#pragma unroll
        for (int i = 0; i < kQT; ++i) out[i] = a.scale * n * (dot[i] * inv_sqrt_d + gam * dq[i]);
    } else {
#pragma unroll
        for (int i = 0; i < kQT; ++i) out[i] = a.scale * n * inv_sqrt_d * dot[i];
    }
}

template <int D, bool QJL>
__device__ __forceinline__ void load_query_tile(const scores_args & a, int64_t q0, float (*qs)[kQT],
                                                float (*us)[kQT], int tid) {
    for (int i = tid; i < kQT * D; i += 256) {
        const int qi = i / D, e = i % D;
        const int64_t qq = q0 + qi;
        const float * row = a.qp + (qq < a.n_q ? qq : a.n_q - 1) * a.qp_stride;
        qs[e][qi] = row[e];
        if constexpr (QJL) us[e][qi] = row[D + e];
    }
}

template <int D, int KB, bool QJL>
__global__ __launch_bounds__(256) void scores_full_kernel(const dev_tables t, const scores_args a) {
    __shared__ __align__(16) float qs[D][kQT];
    __shared__ __align__(16) float us[QJL ? D : 1][kQT];
    __shared__ float cb[16];
    const int tid = threadIdx.x;
    const int64_t q0 = int64_t(blockIdx.y) * kQT;
    load_query_tile<D, QJL>(a, q0, qs, us, tid);
    if (tid < 16) cb[tid] = t.cb[tid];
    __syncthreads();
    const int64_t j = int64_t(blockIdx.x) * kKeys + tid;
    if (j >= a.n_k) return;
    float s[kQT];
    score_key<D, KB, QJL>(t, a, qs, us, cb, j, s);
#pragma unroll
    for (int i = 0; i < kQT; ++i)
        if (q0 + i < a.n_q) a.out_scores[(q0 + i) * a.n_k + j] = s[i];
}

// (score desc, index asc) ordering
__device__ __forceinline__ bool better(float s1, int64_t i1, float s2, int64_t i2) {
    return s1 > s2 || (s1 == s2 && i1 < i2);
}

// One wave merges the candidate scores cs[0..255] (indices ci) of a query into
// its sorted list (ls, li) of length K, keeping the K best.
__device__ void wave_merge_topk(float * ls, int64_t * li, int K, const float * cs, const int64_t * ci,
                                int lane, float * tmp_s, int64_t * tmp_i) {
    // lane-local candidates: 4 new + list entries k with k % 64 == lane
    float c_s[5];
    int64_t c_i[5];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        c_s[r] = cs[lane + 64 * r];
        c_i[r] = ci[lane + 64 * r];
    }
    // the list is at most 64 long -> one entry per lane
    c_s[4] = lane < K ? ls[lane] : -INFINITY;
    c_i[4] = lane < K ? li[lane] : INT64_MAX;
    for (int k = 0; k < K; ++k) {
        float bs = -INFINITY;
        int64_t bi = INT64_MAX;
        int br = -1;
#pragma unroll
        for (int r = 0; r < 5; ++r)
            if (better(c_s[r], c_i[r], bs, bi)) {
                bs = c_s[r];
                bi = c_i[r];
                br = r;
            }
        float ws = bs;
        int64_t wi = bi;
        for (int o = 32; o > 0; o >>= 1) {
            float os = __shfl_xor(ws, o);
            int64_t oi = __shfl_xor(wi, o);
            if (better(os, oi, ws, wi)) {
                ws = os;
                wi = oi;
            }
        }
        // the owner removes the winner (indices are unique among candidates)
        if (br >= 0 && bi == wi && bs == ws) {
#pragma unroll
            for (int r = 0; r < 5; ++r)
                if (r == br) {
                    c_s[r] = -INFINITY;
                    c_i[r] = INT64_MAX;
                }
        }
        if (lane == 0) {
            tmp_s[k] = ws;
            tmp_i[k] = wi;
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < K) {
        ls[lane] = tmp_s[lane];
        li[lane] = tmp_i[lane];
    }
    __builtin_amdgcn_wave_barrier();
}

template <int D, int KB, bool QJL>
__global__ __launch_bounds__(256) void scores_topk_kernel(const dev_tables t, const scores_args a) {
    __shared__ __align__(16) float qs[D][kQT];
    __shared__ __align__(16) float us[QJL ? D : 1][kQT];
    __shared__ float cb[16];
    __shared__ float cand_s[kQT][kKeys];
    __shared__ float list_s[kQT][64];
    __shared__ int64_t list_i[kQT][64];
    __shared__ float tmp_s[4][64];
    __shared__ int64_t tmp_i[4][64];
    __shared__ int64_t key_idx[kKeys];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int K = a.top_k;
    const int64_t q0 = int64_t(blockIdx.y) * kQT;
    load_query_tile<D, QJL>(a, q0, qs, us, tid);
    if (tid < 16) cb[tid] = t.cb[tid];
    for (int i = tid; i < kQT * 64; i += 256) {
        list_s[i / 64][i % 64] = -INFINITY;
        list_i[i / 64][i % 64] = INT64_MAX;
    }
    const int64_t per = (a.n_k + a.n_ranges - 1) / a.n_ranges;
    const int64_t k_begin = int64_t(blockIdx.x) * per;
    const int64_t k_end = k_begin + per < a.n_k ? k_begin + per : a.n_k;
    __syncthreads();
    for (int64_t j0 = k_begin; j0 < k_end; j0 += kKeys) {
        const int64_t j = j0 + tid;
        float s[kQT];
        if (j < k_end) {
            score_key<D, KB, QJL>(t, a, qs, us, cb, j, s);
        } else {
#pragma unroll
            for (int i = 0; i < kQT; ++i) s[i] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < kQT; ++i) cand_s[i][tid] = s[i];
        key_idx[tid] = j < k_end ? j : INT64_MAX;
        __syncthreads();
        // wave wv handles queries wv, wv+4, ...
        for (int qi = wv; qi < kQT; qi += 4) {
            const float thr = list_s[qi][K - 1];
            bool any = false;
#pragma unroll
            for (int r = 0; r < 4; ++r) any |= cand_s[qi][lane + 64 * r] > thr;
            if (__any(any)) wave_merge_topk(list_s[qi], list_i[qi], K, cand_s[qi], key_idx, lane, tmp_s[wv], tmp_i[wv]);
        }
        __syncthreads();
    }
    for (int i = tid; i < kQT * K; i += 256) {
        const int qi = i / K, k = i % K;
        const int64_t qq = q0 + qi;
        if (qq >= a.n_q) continue;
        const int64_t o = (int64_t(blockIdx.x) * a.n_q + qq) * K + k;
        a.cand_s[o] = list_s[qi][k];
        a.cand_i[o] = list_i[qi][k];
    }
}

// Final merge: one wave per query over n_ranges sorted lists of length K.
__global__ __launch_bounds__(64) void topk_merge_kernel(const scores_args a) {
    const int64_t qq = blockIdx.x;
    const int lane = threadIdx.x;
    const int K = a.top_k;
    // cursor per list: lane owns lists lane, lane+64, ...
    const int per_lane = (a.n_ranges + 63) / 64;
    int cur[4];
    for (int r = 0; r < 4; ++r) cur[r] = 0;
    for (int k = 0; k < K; ++k) {
        float bs = -INFINITY;
        int64_t bi = INT64_MAX;
        int br = -1;
        for (int r = 0; r < per_lane && r < 4; ++r) {
            const int list = lane + 64 * r;
            if (list >= a.n_ranges || cur[r] >= K) continue;
            const int64_t o = (int64_t(list) * a.n_q + qq) * K + cur[r];
            const float s = a.cand_s[o];
            const int64_t i = a.cand_i[o];
            if (better(s, i, bs, bi)) {
                bs = s;
                bi = i;
                br = r;
            }
        }
        float ws = bs;
        int64_t wi = bi;
        for (int o = 32; o > 0; o >>= 1) {
            float os = __shfl_xor(ws, o);
            int64_t oi = __shfl_xor(wi, o);
            if (better(os, oi, ws, wi)) {
                ws = os;
                wi = oi;
            }
        }
        if (br >= 0 && bs == ws && bi == wi) {
            for (int r = 0; r < 4; ++r)
                if (r == br) ++cur[r];
        }
        if (lane == 0) {
            a.out_scores[qq * K + k] = ws;
            a.out_idx[qq * K + k] = wi;
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core scorer on 16 x 16 tiles, d = 128 or 256, for top-k lists
// longer than the 32 x 32-tile scorer keeps (16 < k <= 64).  The score
// matrix of 16 queries x 16 keys is a real dense contraction:
// v_mfma_f32_16x16x32_f16 with the queries as the A operand (held in
// registers for the whole key range: R q as fp16 hi + lo, ~22 bits, and
// S R q as fp16, whose contribution is scaled by gamma sqrt(pi/2)/m and needs
// no more) and the keys as the B operand (fp16 centroids and +-1 signs,
// exact, unpacked with byte permutes).  Lane group g
// (lanes 16g..16g+15) unpacks blocks d/128 g .. of its key, so a lane's key
// is also the key of its output column: norms and gamma stay in the lane.
// Top-k keeps a sorted list per query in LDS, touched only by scores that
// reach the current k-th best.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8 as_half8(const uint32_t * w) {
    half8 h;
    __builtin_memcpy(&h, w, 16);
    return h;
}

// Insert (s, idx) into the sorted list (ls, li) of length K (one wave).
__device__ __forceinline__ void wave_insert(float * ls, int32_t * li, int K, float s, int32_t idx, int lane) {
    const float es = lane < K ? ls[lane] : -INFINITY;
    const int32_t ei = lane < K ? li[lane] : INT32_MAX;
    const bool ahead = lane < K && (es > s || (es == s && ei < idx));
    const int pos = __popcll(__ballot(ahead));
    const float ps = __shfl_up(es, 1);
    const int32_t pi = __shfl_up(ei, 1);
    if (pos < K && lane < K && lane >= pos) {
        ls[lane] = lane == pos ? s : ps;
        li[lane] = lane == pos ? idx : pi;
    }
    __builtin_amdgcn_wave_barrier();
}

// Four waves per block, one 16-query tile each, over the same key range: the
// key codes are fetched once into L1 for the four, and the 3/4-bit codes go
// through one shared LDS pair table.
template <int D, int KB, bool QJL, bool TOPK>
__global__ __launch_bounds__(256) void scores_mfma_kernel(const dev_tables t, const scores_args a) {
    constexpr int NBL = D / 128;  // code blocks per lane group
    constexpr int KS = 4 * NBL;   // k-steps (8 values per lane each)
    constexpr int kTab = pair_tab_bytes<KB>();
    __shared__ __align__(16) uint32_t tab[kTab > 0 ? kTab / 4 : 1];
    __shared__ float lst_s[4][TOPK ? 16 : 1][64];
    __shared__ int32_t lst_i[4][TOPK ? 16 : 1][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    // XCD-aware order: blocks are dealt to the 8 XCDs round-robin, so block b
    // takes work item (b % 8) * (grid / 8) + b / 8, and the query tiles of one
    // key range run on one XCD and share its L2 (the grid is padded to a
    // multiple of 8; padding blocks exit)
    const int64_t n_qt4 = ((a.n_q + 15) / 16 + 3) / 4;
    const int64_t item = int64_t(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    if (item >= n_qt4 * a.n_ranges) return;
    const int64_t range = item / n_qt4;
    const int64_t q0 = ((item % n_qt4) * 4 + wave) * 16;
    const int64_t k_begin = range * a.keys_per_range;
    if constexpr (pair_table<KB>()) {
        constexpr int E = 1 << (2 * KB), M = (1 << KB) - 1;
        for (int e = tid >> 3; e < E; e += 32) {
            const uint32_t v = uint32_t(f16_bits(t.cb[e & M])) | (uint32_t(f16_bits(t.cb[e >> KB])) << 16);
            *reinterpret_cast<uint4 *>(tab + e * kPairCopies + 4 * (tid & 7)) = uint4{v, v, v, v};
        }
        __syncthreads();
    }
    const uint32_t lane_off = uint32_t(lane & 31) * 4;
    const int64_t k_end = k_begin + a.keys_per_range < a.n_k ? k_begin + a.keys_per_range : a.n_k;

    // A operands: query n16, values of the k-step order of the B operand
    half8 aqh[KS], aql[KS], au[QJL ? KS : 1];
    {
        const int64_t qq = q0 + n16 < a.n_q ? q0 + n16 : a.n_q - 1;
        const float * qrow = a.qp + qq * a.qp_stride;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int bl = NBL * g + ks / 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = qrow[32 * bl + decoded_code_of_pos<KB>(8 * (ks % 4) + e)];
                const _Float16 hi = static_cast<_Float16>(x);
                aqh[ks][e] = hi;
                aql[ks][e] = static_cast<_Float16>(x - static_cast<float>(hi));
                if constexpr (QJL) au[ks][e] = static_cast<_Float16>(qrow[D + 32 * bl + sign_bit_of_pos(8 * (ks % 4) + e)]);
            }
        }
    }
    const lut16 lut = make_lut(t.cb);
    const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
    const float qjl_gain = sqrtf(0.5f * static_cast<float>(M_PI)) / static_cast<float>(D);
    const int K = a.top_k;
    float thr[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if constexpr (TOPK) {
        for (int qi = 0; qi < 16; ++qi) {
            lst_s[wave][qi][lane] = -INFINITY;
            lst_i[wave][qi][lane] = INT32_MAX;
        }
        __builtin_amdgcn_wave_barrier();
    }

    // the next 16 keys' codes, signs and norms are loaded while the current
    // ones are scored
    uint32_t wn[NBL * KB], swn[NBL];
    uint16_t nkn = 0, rkn = 0;
    auto load_keys = [&](int64_t j0) {
        const int64_t key = j0 + n16;
        const int64_t kv = (key < k_end ? key : k_end - 1) * a.k.stride[2];
        const uint32_t * crow = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8)) + NBL * KB * g;
#pragma unroll
        for (int i = 0; i < NBL * KB; ++i) wn[i] = crow[i];
        if constexpr (QJL) {
            const uint32_t * srow = reinterpret_cast<const uint32_t *>(a.k.signs + kv * (D / 8)) + NBL * g;
#pragma unroll
            for (int i = 0; i < NBL; ++i) swn[i] = srow[i];
            rkn = a.k.rnorms[kv];
        }
        nkn = a.k.norms[kv];
    };
    if (k_begin < k_end) load_keys(k_begin);
    for (int64_t j0 = k_begin; j0 < k_end; j0 += 16) {
        const int64_t key = j0 + n16;
        const bool valid = key < k_end;
        uint32_t w[NBL * KB], sw[NBL];
#pragma unroll
        for (int i = 0; i < NBL * KB; ++i) w[i] = wn[i];
#pragma unroll
        for (int i = 0; i < NBL; ++i) sw[i] = QJL ? swn[i] : 0u;
        const float nk = half_bits_to_float(nkn);
        const float gam = QJL ? half_bits_to_float(rkn) * qjl_gain : 0.f;
        if (j0 + 16 < k_end) load_keys(j0 + 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NBL; ++b) {
            uint32_t o[16];
            if constexpr (pair_table<KB>()) {
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    o[p] = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(tab) +
                                                               pair_offset<KB>(w + KB * b, p, lane_off));
            } else {
                unpack_block<KB>(lut, w + KB * b, o);
            }
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const half8 bk = as_half8(o + 4 * kq);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh[4 * b + kq], bk, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aql[4 * b + kq], bk, acc, 0, 0, 0);
            }
            if constexpr (QJL) {
                uint32_t so[16];
                unpack_signs(sw[b], so);
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
                    accq = __builtin_amdgcn_mfma_f32_16x16x32_f16(au[4 * b + kq], as_half8(so + 4 * kq), accq, 0, 0, 0);
            }
        }
        // this lane: queries q0 + 4g + i (rows), key `key` (column n16)
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = a.scale * nk * (acc[i] * inv_sqrt_d + gam * accq[i]);
        if constexpr (!TOPK) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t q = q0 + 4 * g + i;
                if (valid && q < a.n_q) a.out_scores[q * a.n_k + key] = sc[i];
            }
        } else {
            bool cand = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) cand |= valid && sc[i] >= thr[i];
            if (__any(cand)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint64_t mask = __ballot(valid && sc[i] >= thr[i]);
                    while (mask) {
                        const int src = __builtin_ctzll(mask);
                        mask &= mask - 1;
                        const int qi = 4 * (src >> 4) + i;
                        const float sv = __shfl(sc[i], src);
                        const int32_t iv = static_cast<int32_t>(__shfl(static_cast<int32_t>(key), src));
                        wave_insert(lst_s[wave][qi], lst_i[wave][qi], K, sv, iv, lane);
                        if ((lane >> 4) == (src >> 4)) thr[i] = lst_s[wave][qi][K - 1];
                    }
                }
            }
        }
    }
    if constexpr (TOPK) {
        for (int qi = 0; qi < 16; ++qi) {
            const int64_t q = q0 + qi;
            if (q < a.n_q && lane < K) {
                const int64_t o = (range * a.n_q + q) * K + lane;
                a.cand_s[o] = lst_s[wave][qi][lane];
                a.cand_i[o] = lst_i[wave][qi][lane] == INT32_MAX ? INT64_MAX : int64_t(lst_i[wave][qi][lane]);
            }
        }
    }
}

template <int D, int KB, bool QJL>
hipError_t launch_scores_t(const dev_tables & t, const scores_args & a, hipStream_t s) {
    if (scores_tile32_supported(D, t.norm_group != 0, a.top_k)) {
        hipError_t e = launch_scores_tile32(t, a, s);
        if (e != hipSuccess || a.top_k == 0) return e;
        hipLaunchKernelGGL(topk_merge_kernel, dim3(a.n_q), dim3(64), 0, s, a);
        return hipGetLastError();
    }
    if constexpr (D >= 128) {
        if (!t.norm_group) {
            const int64_t items = ((a.n_q + 15) / 16 + 3) / 4 * a.n_ranges;
            const dim3 grid(static_cast<uint32_t>((items + 7) / 8 * 8));
            if (a.top_k == 0) {
                hipLaunchKernelGGL((scores_mfma_kernel<D, KB, QJL, false>), grid, dim3(256), 0, s, t, a);
                return hipGetLastError();
            }
            hipLaunchKernelGGL((scores_mfma_kernel<D, KB, QJL, true>), grid, dim3(256), 0, s, t, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(topk_merge_kernel, dim3(a.n_q), dim3(64), 0, s, a);
            return hipGetLastError();
        }
    }
    const int64_t qtiles = (a.n_q + kQT - 1) / kQT;
    if (a.top_k == 0) {
        dim3 grid((a.n_k + kKeys - 1) / kKeys, qtiles);
        hipLaunchKernelGGL((scores_full_kernel<D, KB, QJL>), grid, dim3(256), 0, s, t, a);
        return hipGetLastError();
    }
    dim3 grid(a.n_ranges, qtiles);
    hipLaunchKernelGGL((scores_topk_kernel<D, KB, QJL>), grid, dim3(256), 0, s, t, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(a.n_q), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_scores_d(const dev_tables & t, const scores_args & a, hipStream_t s) {
    switch (t.bits * 2 + (t.qjl ? 1 : 0)) {
        case 4: return launch_scores_t<D, 2, false>(t, a, s);
        case 5: return launch_scores_t<D, 2, true>(t, a, s);
        case 6: return launch_scores_t<D, 3, false>(t, a, s);
        case 7: return launch_scores_t<D, 3, true>(t, a, s);
        case 8: return launch_scores_t<D, 4, false>(t, a, s);
        case 9: return launch_scores_t<D, 4, true>(t, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// 32 x 32-tile path (d = 128 or 256, one norm per vector, top_k <= 16): one
// wave per (32 queries, range), about 2048 waves in all (two per SIMD), the
// ranges a multiple of the waves per block and of 32 keys.  16 x 16-tile path
// (d >= 128, one norm per vector, larger top_k): about 4096 waves in all (one
// per 16 queries and range), ranges a multiple of 16 keys.  Both at most 256
// ranges (the final merge reads up to 4 lists per lane).  VALU path: ranges
// of ~4096 keys.
void scores_plan(int d, bool block_norms, int64_t n_q, int64_t n_k, int32_t top_k, int32_t & ranges,
                 int64_t & keys_per_range) {
    int64_t r;
    if (scores_tile32_supported(d, block_norms, top_k)) {
        const int64_t qtiles = (n_q + 31) / 32;
        const int64_t w = scores_tile32_waves();
        r = (2048 + qtiles - 1) / qtiles;
        r = (r + w - 1) / w * w;
        const int64_t max_r = (n_k + 31) / 32;
        if (r > max_r) r = max_r;
        if (r > 256) r = 256;
        if (r < 1) r = 1;
        int64_t per = (n_k + r - 1) / r;
        per = (per + 31) / 32 * 32;
        keys_per_range = per;
        r = (n_k + per - 1) / per;
    } else if (d >= 128 && !block_norms) {
        const int64_t qtiles = (n_q + 15) / 16;
        r = (4096 + qtiles - 1) / qtiles;
        const int64_t max_r = (n_k + 15) / 16;
        if (r > max_r) r = max_r;
        if (r > 256) r = 256;
        if (r < 1) r = 1;
        int64_t per = (n_k + r - 1) / r;
        per = (per + 15) / 16 * 16;
        keys_per_range = per;
        r = (n_k + per - 1) / per;
    } else {
        r = (n_k + 4095) / 4096;
        if (r > 256) r = 256;
        if (r < 1) r = 1;
        keys_per_range = (n_k + r - 1) / r;
    }
    ranges = static_cast<int32_t>(r < 1 ? 1 : r);
}

hipError_t launch_scores(const dev_tables & t, const scores_args & a, hipStream_t s) {
    switch (t.d) {
        case 32: return launch_scores_d<32>(t, a, s);
        case 64: return launch_scores_d<64>(t, a, s);
        case 128: return launch_scores_d<128>(t, a, s);
        case 256: return launch_scores_d<256>(t, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
