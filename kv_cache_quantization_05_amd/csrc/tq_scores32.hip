// Matrix-core scorer on 32 x 32 tiles: d = 128 or 256, one norm per vector,
// the full score matrix or a top-k of at most 16.
//
// The scores of 32 queries against 32 keys are one dense contraction per
// 16-deep slice of the dimensions, v_mfma_f32_32x32x16_f16 with the queries
// as the A operand (rows) and the dequantised keys as the B operand
// (columns).  Per key and wave the codes and signs are unpacked once for 32
// queries, twice as many as a 16 x 16 tile serves, and a 32 x 32 tile needs
// half the operand bytes per product of a 16 x 16 one.
//   A: the rotated query R q as fp16 hi + lo (~22 bits; [TQ explainer]
//      §2.2.2, full-precision queries), and S R q as fp16 for the sketch term
//      ([TQ explainer] §2.2; [Orión plan] Fase 3).  The hi parts stay in
//      registers; the lo parts and S R q are staged once per workgroup in LDS
//      as ready-made fragments (16 bytes per lane and slice, read without
//      bank conflicts).
//   B: lane l serves key l % 32 and the half (l / 32) of its dimensions, so
//      its codes and signs are contiguous loads; the 8 k-slots of a slice are
//      8 consecutive decoded values of one 32-code block.  3- and 4-bit codes
//      are decoded two at a time through a 64 KB byte-indexed pair table in
//      LDS (one byte permute forms the address), 2-bit codes with byte
//      permutes in registers.  Sign bits enter as b in {0, 1} through
//      sigma = 2 b - 1: one AND keeps bits k and k + 16 of a sign word in
//      place, i.e. the fp16 values b 2^(k' - 24) (k' = k for k < 10, else
//      k - 6 after one shared shift: denormal, exact), and the query side
//      carries the matching factor 2^(24 - k' - E) (E from the tile's largest
//      |S R q|, so every A value is a normal fp16 below 2^15).  The
//      accumulator starts at -sum(S R q) 2^-(E+1) and the result is scaled by
//      2^(E+1), which gives sum (S R q)_i sigma_i.
//   D: lane l holds key l % 32 against queries 8 i + 4 (l / 32) + j in
//      register 4 i + j, so the key's norm and gamma stay in the lane:
//      s = scale * N * (<R q, c> / sqrt(d) + gamma sqrt(pi/2) / m <S R q, sigma>)
//      ([TQ+ guide] §5.3, pre-rotated queries).
// Top-k ([TQ explainer] §3.4, inner-product search): every wave scans its own
// key range and keeps, per query, a sorted list in registers (query
// 8 i + 4 h + j: register 4 i + j of lanes 32 h .. 32 h + k - 1, one row of
// 16 lanes, so an insertion is a ballot and a row shift); a final kernel
// merges the per-range lists (equal scores: lower index first).  The first 32 keys
// fill the lists by one sort per half-wave.  Afterwards a score enters only
// if it reaches the workgroup's threshold for its query, a value that at
// least k distinct keys already reach: the largest k-th best of the eight
// waves' lists, raised to the j-th largest of the lists' c-th bests (c =
// ceil(k / waves), j = ceil(k / c): j lists hold c keys each at or above it,
// j c >= k distinct keys).  The k-th best of all keys is at least that value,
// so no key of the final top-k is ever filtered out, and none is evicted from
// its list (fewer than k keys beat it).
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_unpack.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;   // waves per workgroup, each with its own key range
constexpr int kCap = 16;    // top-k list capacity per query

__device__ __forceinline__ half8 as_half8(const uint32_t * w) {
    half8 h;
    __builtin_memcpy(&h, w, 16);
    return h;
}

// (score desc, index asc) ordering
__device__ __forceinline__ bool ahead_of(float s1, int32_t i1, float s2, int32_t i2) {
    return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Lane l - 1's value within each row of 16 lanes (lane 0 of a row: x).
__device__ __forceinline__ int32_t row_shr1(int32_t x) { return __builtin_amdgcn_update_dpp(x, x, 0x111, 0xF, 0xF, false); }

// Eight values in registers sorted largest first (a 19-comparator network).
__device__ __forceinline__ void sort8_desc(float * e) {
    constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 1}, {2, 3},
                                {4, 5}, {6, 7}, {2, 4}, {3, 5}, {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
    for (int c = 0; c < 19; ++c) {
        const float a = e[net[c][0]], b = e[net[c][1]];
        e[net[c][0]] = fmaxf(a, b);
        e[net[c][1]] = fminf(a, b);
    }
}

// Bitonic sort of (s, i) within each 32-lane half of the wave, best first.
__device__ __forceinline__ void half_sort32(float & s, int32_t & i, int lane) {
#pragma unroll
    for (int size = 2; size <= 32; size <<= 1) {
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) {
            const float os = __shfl_xor(s, j);
            const int32_t oi = __shfl_xor(i, j);
            // blocks of `size` lanes alternate best-first / best-last, the
            // whole half best-first; the lower lane of a pair keeps the better
            const bool first = ((lane & size & 31) == 0) == ((lane & j) == 0);
            const bool other_ahead = ahead_of(os, oi, s, i);
            if (first == other_ahead) {
                s = os;
                i = oi;
            }
        }
    }
}

template <int D, int KB, bool QJL, bool TOPK>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(2, 2)))
void scores_tile32_kernel(const dev_tables t, const scores_args a) {
    constexpr int NBH = D / 64;    // 32-code blocks per lane half
    constexpr int KS = 4 * NBH;    // 16-deep slices
    constexpr int kTab = pair_table<KB>() ? kByteTabBytes : 0;
    constexpr int kFrag = KS * 64 * 16;  // one operand's fragments
    // fragments first, so that their offsets (< 64 KB) fit the LDS
    // instructions' offset field; the pair table after them
    constexpr int kFrags = kFrag * (QJL ? 2 : 1);
    __shared__ __align__(16) uint8_t lds_all[kFrags + kTab];
    // the workgroup's thresholds in the lane order of the D operand:
    // thr[h][4 i + j] belongs to query 8 i + 4 h + j
    __shared__ __align__(16) float thr[2][16];
    // each wave's c-th best per query
    __shared__ __align__(16) float pub[32][kWaves];
    __shared__ float sum_u[32];
    __shared__ float max_u;
    uint8_t * const frag_lo = lds_all;
    uint8_t * const frag_u = lds_all + kFrag;
    const uint8_t * const tab = lds_all + kFrags;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    // XCD-aware order: blocks are dealt to the 8 XCDs round-robin, so block b
    // takes work item (b % 8) * (grid / 8) + b / 8 and the query tiles of one
    // group of ranges run on one XCD, sharing its L2 (the grid is a multiple
    // of 8; padding blocks exit before any barrier)
    const int64_t n_qt = (a.n_q + 31) / 32;
    const int64_t n_rg = (a.n_ranges + kWaves - 1) / kWaves;
    const int64_t item = int64_t(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    if (item >= n_qt * n_rg) return;
    const int64_t q0 = (item % n_qt) * 32;
    const int64_t range = (item / n_qt) * kWaves + wave;
    const bool has_range = range < a.n_ranges;
    const int64_t k_begin = has_range ? range * a.keys_per_range : 0;
    const int64_t k_last = k_begin + a.keys_per_range < a.n_k ? k_begin + a.keys_per_range : a.n_k;
    const int64_t k_end = has_range ? k_last : 0;

    if constexpr (pair_table<KB>()) {
        // entry e (256 bytes apart) holds the centroids of the codes in its
        // low and high KB bits in 32 copies (copy c at +4 c), so the 32 lanes
        // served together never share a bank
        const lut16 tl = make_lut(t.cb);
        constexpr int M = (1 << KB) - 1;
        for (int e = tid >> 3; e < 256; e += 8 * kWaves) {
            const uint32_t v = lut_bits<KB>(tl, uint32_t(e & M)) | (lut_bits<KB>(tl, uint32_t((e >> KB) & M)) << 16);
            *reinterpret_cast<uint4 *>(lds_all + kFrags + e * 256 + 16 * (tid & 7)) = uint4{v, v, v, v};
        }
    }
    // fragments of slice s for lane l (query l % 32, half l / 32): k-slot e is
    // dimension 32 bl + pos(8 (s % 4) + e) of block bl = NBH (l / 32) + s / 4
    auto dim_of = [](int l, int s, int e) {
        return 32 * (NBH * (l >> 5) + s / 4) + decoded_code_of_pos<KB>(8 * (s % 4) + e);
    };
    auto sign_dim_of = [](int l, int s, int e) {
        return 32 * (NBH * (l >> 5) + s / 4) + sign_bit_of_pos(8 * (s % 4) + e);
    };
    auto qrow_of = [&](int l) {
        const int64_t qq = q0 + (l & 31) < a.n_q ? q0 + (l & 31) : a.n_q - 1;
        return a.qp + qq * a.qp_stride;
    };
    // S R q: per query the sum (16 lanes per query, fixed order) and the
    // tile's largest magnitude, which sets the exponent E of the A values
    int E = 0;
    if constexpr (QJL) {
        if (tid == 0) max_u = 0.f;
        __syncthreads();
        const int m = tid >> 4, j = tid & 15;
        const float * urow = qrow_of(m) + D;
        float su = 0.f, mu = 0.f;
        for (int e = j; e < D; e += 16) {
            su += urow[e];
            mu = fmaxf(mu, fabsf(urow[e]));
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            su += __shfl_xor(su, o);
            mu = fmaxf(mu, __shfl_xor(mu, o));
        }
        if (j == 0) {
            sum_u[m] = su;
            __hip_atomic_fetch_max(&max_u, mu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        __syncthreads();
        int ex;
        frexpf(max_u, &ex);  // max_u < 2^ex
        E = ex + 9;          // |S R q| 2^(24 - E) < 2^15
    }
    for (int i = tid; i < KS * 64; i += 64 * kWaves) {
        const int s = i >> 6, l = i & 63;
        const float * qrow = qrow_of(l);
        half8 lo, u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = qrow[dim_of(l, s, e)];
            const _Float16 hi = static_cast<_Float16>(x);
            lo[e] = static_cast<_Float16>(x - static_cast<float>(hi));
            u[e] = QJL ? static_cast<_Float16>(ldexpf(qrow[D + sign_dim_of(l, s, e)], 24 - sign_shift_of_pos(8 * (s % 4) + e) - E))
                       : static_cast<_Float16>(0.f);
        }
        *reinterpret_cast<half8 *>(frag_lo + 16 * i) = lo;
        if constexpr (QJL) *reinterpret_cast<half8 *>(frag_u + 16 * i) = u;
    }
    half8 aqh[KS];
    {
        const float * qrow = qrow_of(lane);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) aqh[s][e] = static_cast<_Float16>(qrow[dim_of(lane, s, e)]);
    }
    const int K = a.top_k;
    // c: (waves with a range) * c >= K, and jc = ceil(K / c) <= waves with a
    // range; a wave without a range holds -inf entries, below every jc-th
    // largest
    const int active = static_cast<int>(a.n_ranges - (item / n_qt) * kWaves < kWaves ? a.n_ranges - (item / n_qt) * kWaves
                                                                                  : kWaves);
    const int kc = (K + active - 1) / active;
    const int jc = (K + kc - 1) / kc;
    if constexpr (TOPK) {
        if (tid < 32) thr[tid >> 4][tid & 15] = -INFINITY;
        if (lane < 32) pub[lane][wave] = -INFINITY;
    }
    __syncthreads();

    const lut16 lut = make_lut(t.cb);
    const uint32_t lane_off = uint32_t(lane & 31) * 4;
    const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
    // sketch term: gamma sqrt(pi/2)/m times 2^(E+1) times the accumulator,
    // which starts at -sum(S R q) 2^-(E+1) for each of the lane's queries
    const float qjl_gain = ldexpf(sqrtf(0.5f * static_cast<float>(M_PI)) / static_cast<float>(D), E + 1);
    float cinit[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) cinit[v] = QJL ? ldexpf(-sum_u[8 * (v >> 2) + 4 * h + (v & 3)], -(E + 1)) : 0.f;

    // top-k lists: entry n of query 8 i + 4 h + j in register 4 i + j of lane
    // 32 h + n (n < K)
    float ls[TOPK ? 16 : 1];
    int32_t li[TOPK ? 16 : 1];
#pragma unroll
    for (int v = 0; v < (TOPK ? 16 : 1); ++v) {
        ls[v] = -INFINITY;
        li[v] = INT32_MAX;
    }

    // the next 32 keys' codes, signs and norms are loaded while the current
    // ones are scored
    uint32_t wn[NBH * KB], swn[QJL ? NBH : 1];
    uint16_t nkn = 0, rkn = 0;
    auto load_keys = [&](int64_t j0) {
        const int64_t key = j0 + n32;
        const int64_t kv = (key < k_end ? key : k_end - 1) * a.k.stride[2];
        const uint32_t * crow = reinterpret_cast<const uint32_t *>(a.k.codes + kv * (D * KB / 8)) + NBH * KB * h;
#pragma unroll
        for (int i = 0; i < NBH * KB; ++i) wn[i] = crow[i];
        if constexpr (QJL) {
            const uint32_t * srow = reinterpret_cast<const uint32_t *>(a.k.signs + kv * (D / 8)) + NBH * h;
#pragma unroll
            for (int i = 0; i < NBH; ++i) swn[i] = srow[i];
            rkn = a.k.rnorms[kv];
        }
        nkn = a.k.norms[kv];
    };
    if (k_begin < k_end) load_keys(k_begin);
    for (int64_t j0 = k_begin; j0 < k_end; j0 += 32) {
        // the LDS fragments are re-read every step, not hoisted into 128
        // registers for the whole loop
        asm volatile("" ::: "memory");
        const int64_t key = j0 + n32;
        const bool valid = key < k_end;
        uint32_t w[NBH * KB], sw[QJL ? NBH : 1];
#pragma unroll
        for (int i = 0; i < NBH * KB; ++i) w[i] = wn[i];
#pragma unroll
        for (int i = 0; i < (QJL ? NBH : 1); ++i) sw[i] = QJL ? swn[i] : 0u;
        const float alpha = a.scale * half_bits_to_float(nkn);
        const float beta = QJL ? alpha * half_bits_to_float(rkn) * qjl_gain : 0.f;
        if (j0 + 32 < k_end) load_keys(j0 + 32);
        f32x16 acc = {}, accq;
#pragma unroll
        for (int v = 0; v < 16; ++v) accq[v] = cinit[v];
#pragma unroll
        for (int b = 0; b < NBH; ++b) {
            uint32_t o[16];
            if constexpr (KB == 4) {
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    o[p] = *reinterpret_cast<const uint32_t *>(tab + byte_pair_offset(w + 4 * b, p, lane_off));
            } else if constexpr (KB == 3) {
                const block3_shifts sh = shift_block3(w + 3 * b);
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    o[p] = *reinterpret_cast<const uint32_t *>(tab + byte3_pair_offset(sh, p, lane_off));
            } else {
                unpack_block<KB>(lut, w + KB * b, o);
            }
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const int s = 4 * b + kq;
                const half8 bk = as_half8(o + 4 * kq);
                const half8 alo = *reinterpret_cast<const half8 *>(frag_lo + 16 * (64 * s + lane));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aqh[s], bk, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bk, acc, 0, 0, 0);
            }
            if constexpr (QJL) {
                uint32_t so[16];
                expand_signs(sw[b], so);
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const int s = 4 * b + kq;
                    const half8 au = *reinterpret_cast<const half8 *>(frag_u + 16 * (64 * s + lane));
                    accq = __builtin_amdgcn_mfma_f32_32x32x16_f16(au, as_half8(so + 4 * kq), accq, 0, 0, 0);
                }
            }
        }
        // register 4 i + j: query q0 + 8 i + 4 h + j against key `key`
        float sc[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[v] = QJL ? fmaf(alpha * inv_sqrt_d, acc[v], beta * accq[v]) : alpha * inv_sqrt_d * acc[v];
        if constexpr (!TOPK) {
            // rows q0 + 4 h + r, r = 8 i + j: one row pointer, uniform offsets
            float * const orow = a.out_scores + (q0 + 4 * h) * a.n_k + key;
            const int64_t rows_left = a.n_q - q0 - 4 * h;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + (v & 3);
                if (valid && r < rows_left) orow[int64_t(r) * a.n_k] = sc[v];
            }
        } else if (j0 == k_begin) {
            // the first 32 keys: the lists are empty, so each row's list is
            // the best K of its 32 scores (one sort per half-wave and row)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float sv = valid ? sc[v] : -INFINITY;
                int32_t iv = valid ? static_cast<int32_t>(key) : INT32_MAX;
                half_sort32(sv, iv, lane);
                const int m = 8 * (v >> 2) + 4 * h + (v & 3);
                if (n32 < K) {
                    ls[v] = sv;
                    li[v] = iv;
                }
                if (n32 == K - 1) __hip_atomic_fetch_max(&thr[h][v], sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (n32 == kc - 1) pub[m][wave] = sv;
            }
            __builtin_amdgcn_wave_barrier();
        } else {
            float th[16];
            {
                const float4 * tp = reinterpret_cast<const float4 *>(&thr[h][0]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 x = tp[c];
                    th[4 * c] = x.x;
                    th[4 * c + 1] = x.y;
                    th[4 * c + 2] = x.z;
                    th[4 * c + 3] = x.w;
                }
            }
            bool cand = false;
#pragma unroll
            for (int v = 0; v < 16; ++v) cand |= valid && sc[v] >= th[v];
            if (__any(cand)) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    uint64_t mask = __ballot(valid && sc[v] >= th[v]);
                    if (!mask) continue;
                    // one candidate of each half per round (rows m(v, 0) and
                    // m(v, 1) are independent lists)
                    while (mask) {
                        const uint32_t mlo = static_cast<uint32_t>(mask), mhi = static_cast<uint32_t>(mask >> 32);
                        const int s0 = mlo ? __builtin_ctz(mlo) : 0, s1 = mhi ? 32 + __builtin_ctz(mhi) : 32;
                        if (mlo) mask &= ~(uint64_t(1) << s0);
                        if (mhi) mask &= ~(uint64_t(1) << s1);
                        const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[v]), s0));
                        const float c1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[v]), s1));
                        const int32_t k0 = __builtin_amdgcn_readlane(static_cast<int32_t>(key), s0);
                        const int32_t k1 = __builtin_amdgcn_readlane(static_cast<int32_t>(key), s1);
                        const bool has = h ? mhi != 0 : mlo != 0;
                        const float cs = h ? c1 : c0;
                        const int32_t ci = h ? k1 : k0;
                        const bool ahead = n32 < K && (ls[v] > cs || (ls[v] == cs && li[v] < ci));
                        const uint64_t am = __ballot(ahead);
                        const int pos = h ? __popc(static_cast<uint32_t>(am >> 32)) : __popc(static_cast<uint32_t>(am));
                        const float up_s = __int_as_float(row_shr1(__float_as_int(ls[v])));
                        const int32_t up_i = row_shr1(li[v]);
                        if (has && n32 < K && n32 >= pos) {
                            ls[v] = n32 == pos ? cs : up_s;
                            li[v] = n32 == pos ? ci : up_i;
                        }
                    }
                    // publish the k-th and c-th best of both rows
                    const float kth0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[v]), K - 1));
                    const float kth1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[v]), 32 + K - 1));
                    const float cth0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[v]), kc - 1));
                    const float cth1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[v]), 32 + kc - 1));
                    if (lane < 2) {
                        const int m = 8 * (v >> 2) + 4 * lane + (v & 3);
                        __hip_atomic_fetch_max(&thr[lane][v], lane ? kth1 : kth0, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                        pub[m][wave] = lane ? cth1 : cth0;
                    }
                }
            }
            // every fourth step, queries 4 w .. 4 w + 3 (lane r: query 4 w + r):
            // the jc-th largest of the eight waves' c-th bests
            static_assert(kWaves == 8, "a sorting network of the eight waves' entries");
            if ((((j0 - k_begin) >> 5) & 3) == 0 && lane < 4) {
                const int m = 4 * wave + lane;
                const float4 x0 = *reinterpret_cast<const float4 *>(&pub[m][0]);
                const float4 x1 = *reinterpret_cast<const float4 *>(&pub[m][4]);
                float e[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                sort8_desc(e);
                float c = e[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) c = jc - 1 == i ? e[i] : c;
                __hip_atomic_fetch_max(&thr[(m >> 2) & 1][4 * (m >> 3) + (m & 3)], c, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    if constexpr (TOPK) {
        if (has_range) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t q = q0 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (q < a.n_q && n32 < K) {
                    const int64_t o = (range * a.n_q + q) * K + n32;
                    a.cand_s[o] = ls[v];
                    a.cand_i[o] = li[v] == INT32_MAX ? INT64_MAX : int64_t(li[v]);
                }
            }
        }
    }
}

template <int D, int KB, bool QJL>
hipError_t launch_t(const scores_args & a, const dev_tables & t, hipStream_t s) {
    const int64_t items = (a.n_q + 31) / 32 * ((a.n_ranges + kWaves - 1) / kWaves);
    const dim3 grid(static_cast<uint32_t>((items + 7) / 8 * 8));
    if (a.top_k == 0)
        hipLaunchKernelGGL((scores_tile32_kernel<D, KB, QJL, false>), grid, dim3(64 * kWaves), 0, s, t, a);
    else
        hipLaunchKernelGGL((scores_tile32_kernel<D, KB, QJL, true>), grid, dim3(64 * kWaves), 0, s, t, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const scores_args & a, const dev_tables & t, hipStream_t s) {
    switch (t.bits * 2 + (t.qjl ? 1 : 0)) {
        case 4: return launch_t<D, 2, false>(a, t, s);
        case 5: return launch_t<D, 2, true>(a, t, s);
        case 6: return launch_t<D, 3, false>(a, t, s);
        case 7: return launch_t<D, 3, true>(a, t, s);
        case 8: return launch_t<D, 4, false>(a, t, s);
        case 9: return launch_t<D, 4, true>(a, t, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool scores_tile32_supported(int d, bool block_norms, int32_t top_k) {
    return (d == 128 || d == 256) && !block_norms && top_k <= kCap;
}

int scores_tile32_waves() { return kWaves; }

hipError_t launch_scores_tile32(const dev_tables & t, const scores_args & a, hipStream_t s) {
    return t.d == 256 ? launch_d<256>(a, t, s) : launch_d<128>(a, t, s);
}

}  // namespace tq
