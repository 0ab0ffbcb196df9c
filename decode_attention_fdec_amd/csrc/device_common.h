// Device helpers for the libfdec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdec {

typedef _Float16 half2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

// Four e4m3 values (bytes, lowest first) to four bf16 values in two dwords
// (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Float8 tiles of 128-byte rows on the 16x16x32 matrix cores: the 16-byte slot
// of piece p in row r is p ^ fp8_row_swz(r). A K read (16 rows 16kb .. 16kb + 15,
// one piece) and a V transpose read (rows 4kq + 0..3 and 16 + 4kq + 0..3 of a
// 32-row half, one piece) then take distinct (row parity, slot) pairs in each
// group of 16 lanes: distinct banks.
__device__ __forceinline__ int fp8_row_swz(int r) { return ((r >> 1) & 7) ^ ((r >> 2) & 4); }

// The e4m3fn code (OCP float8: sign, 4 exponent bits with bias 7, 3 fraction
// bits) of a binary32 value, rounded to nearest with ties to even. Magnitudes
// of 448 (the largest finite code) and above saturate to +-448, NaN gives the
// NaN code 0x7f. Below 2^-6 the codes are the multiples of 2^-9 (a rounded to
// an integer count of them; 8 of them is the smallest normal code 0x08).
// Above, the top three fraction bits are kept and rounded on the rest; a
// carry out of the fraction moves into the exponent field by the addition.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = __builtin_fabsf(x);
    if (!(a == a)) return 0x7fu;
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
    const uint32_t ua = u & 0x7fffffffu;
    const uint32_t e = (ua >> 23) - 120u;  // binary32 exponent field - 127 + 7
    const uint32_t frac = ua & 0x7fffffu;
    const uint32_t rest = frac & 0xfffffu;
    uint32_t r = frac >> 20;
    r += (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ? 1u : 0u;
    return sign | ((e << 3) + r);
}

// The (request b, KV head g) descale of a float8 cache (1 without one), by a
// scalar load; P is the kernels' parameter block (Hkv KV heads).
template <class P>
__device__ __forceinline__ float kv_descale(const float *d, const P &p, int b, int g) {
    if (!d) return 1.0f;
    typedef const __attribute__((address_space(4))) float *cf_t;
    return ((cf_t)d)[(int64_t)b * p.Hkv + g];
}

// Element type operations: 0 = fp16, 1 = bf16. A packed dword holds elements
// (lo, hi) = (d, d + 1).
template <int DT> struct Elem;

template <> struct Elem<0> {
    static __device__ __forceinline__ float lo(uint32_t u) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t u) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
    // c + a.lo * b.lo + a.hi * b.hi with fp32 accumulation (v_dot2_f32_f16).
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_v, a), __builtin_bit_cast(half2_v, b), c,
                                      false);
    }
    // Round to nearest even (the default rounding mode of v_cvt_f16_f32).
    static __device__ __forceinline__ uint16_t from_float(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
};

template <> struct Elem<1> {
    static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
    // c + a.lo * b.lo + a.hi * b.hi with fp32 accumulation (v_dot2_f32_bf16).
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                               __builtin_bit_cast(bf16x2_v, b), c, false);
    }
    // Round to nearest even onto bfloat16 (NaN stays a quiet NaN).
    static __device__ __forceinline__ uint16_t from_float(float x) {
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};

// DPP lane permutations (within rows of 16 lanes).
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each group of 8
constexpr int kDppRowRor8 = 0x128;    // rotate right by 8 within 16 (= xor 8)
constexpr int kDppRowRor4 = 0x124;    // rotate right by 4 within 16

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Reductions without the LDS crossbar: DPP within rows of 16 lanes, then the
// gfx950 row swaps (v_permlane16_swap, v_permlane32_swap) across rows. Each
// step adds two values that every lane of the pair sees in one or the other
// order, so every lane of a reduced set ends with the same bits.

// x combined over lanes L, L ^ 16, L ^ 32, L ^ 48.
template <class Op> __device__ __forceinline__ float across_rows(float x, Op op) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
// x combined over the lanes of L's row with the same L & 3 (rotations by 8,
// then by 4: the pairs {j, j + 8} first, so every lane of the set gets the
// same bits).
template <class Op> __device__ __forceinline__ float within_row_mod4(float x, Op op) {
    x = op(x, dpp<kDppRowRor8>(x));
    return op(x, dpp<kDppRowRor4>(x));
}
struct AddOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Over the 16 lanes with the same L & 3 (the four query heads of the
// matrix-core map kernels' state layout).
__device__ __forceinline__ float sum_mod4(float x) { return across_rows(within_row_mod4(x, AddOp{}), AddOp{}); }
__device__ __forceinline__ float max_mod4(float x) { return across_rows(within_row_mod4(x, MaxOp{}), MaxOp{}); }

// Over the whole wave: quad butterfly, then the row and cross-row steps.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    return max_mod4(x);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    return sum_mod4(x);
}

// max of two floats that are already canonical (results of arithmetic): one
// v_max_f32, without the quieting that fmaxf adds for signalling NaNs.
__device__ __forceinline__ float fmax_nc(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float readlane(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// LDS-DMA load: 64 lanes x 16 bytes from base + voff (per lane) into LDS at
// lds_addr + 16 * lane. Issued as inline assembly so that the compiler neither
// waits for it before unrelated LDS reads nor counts it: every wait on these
// loads is one of the explicit waits below.
// base and lds_addr are wave-uniform; readfirstlane states that to the compiler.
// NT: the load carries the non-temporal cache policy (nt), for data read once
// per call (K/V tiles): streaming reads of an MI355X decode pattern measured
// ~9% faster with it than with the default policy (6.7 against 6.1 TB/s).
template <bool NT = false>
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t lds_addr) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    const uint32_t ul = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff),
                     "s"(reinterpret_cast<const char *>(ua)), "s"(ul) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff),
                     "s"(reinterpret_cast<const char *>(ua)), "s"(ul) : "memory", "m0");
}
// A vector load with the non-temporal cache policy (K/V pieces: read once per call).
template <class T> __device__ __forceinline__ T load_nt(const char *p);
template <> __device__ __forceinline__ uint4 load_nt<uint4>(const char *p) {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
template <> __device__ __forceinline__ uint2 load_nt<uint2>(const char *p) {
    typedef unsigned int u2v __attribute__((ext_vector_type(2)));
    const u2v x = __builtin_nontemporal_load(reinterpret_cast<const u2v *>(p));
    return make_uint2(x[0], x[1]);
}
// A K/V tile row piece: read once per call.
__device__ __forceinline__ void dma16_kv(const char *base, uint32_t voff, uint32_t lds_addr) {
    dma16<true>(base, voff, lds_addr);
}
template <int N> __device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
// wait until at most N k DMA loads are outstanding (k uniform, clamped to [0, 7])
template <int N> __device__ __forceinline__ void wait_vm_n(int k) {
    switch (k) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<N>(); break;
    case 2: wait_vm<2 * N>(); break;
    case 3: wait_vm<3 * N>(); break;
    case 4: wait_vm<4 * N>(); break;
    case 5: wait_vm<5 * N>(); break;
    case 6: wait_vm<6 * N>(); break;
    default: wait_vm<7 * N>(); break;
    }
}

// Sum and inclusive prefix sum of an int over the wave.
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    return __builtin_amdgcn_readfirstlane(x);  // the same in every lane
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

// LDS address of a shared-memory pointer, for m0.
__device__ __forceinline__ uint32_t lds_addr(const void *ptr) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)ptr;
}


// Merging S <= 256 partial states of one (b, h) (the reduce stage):
// m = max_i m_i, alpha_i = exp(m_i - m) (0 for an empty state), d = sum alpha_i d_i,
// out = sum alpha_i O~_i / d, lse = m + ln d. States are in natural-log units.
//
// The weighted sum runs over fixed groups of kMergeGroup consecutive states:
// each group is summed in split order, then the group sums are added in group
// order. One wave can take every group in turn (merge_states_wave) or one wave
// per group can take them side by side (merge_kernel_groups); both give the
// same bits, and so do the merge kernel and the single-kernel path.
constexpr int kMergeGroup = 32;

// Where the states of one (b, h) live: state s has its O~ row at row(s) (D
// floats) and its m, d at m(s), d(s).
template <int D> struct ContigStates {  // S consecutive states
    const float *po, *pm, *pd;
    __device__ __forceinline__ const float *row(int s) const { return po + (int64_t)s * D; }
    __device__ __forceinline__ float m(int s) const { return pm[s]; }
    __device__ __forceinline__ float d(int s) const { return pd[s]; }
};
template <int D> struct TwoRuns {  // n0 consecutive states, then the states of a second run
    ContigStates<D> a, b;
    int n0;
    __device__ __forceinline__ const float *row(int s) const { return s < n0 ? a.row(s) : b.row(s - n0); }
    __device__ __forceinline__ float m(int s) const { return s < n0 ? a.m(s) : b.m(s - n0); }
    __device__ __forceinline__ float d(int s) const { return s < n0 ? a.d(s) : b.d(s - n0); }
};

// M, dsum and the weights a[k] of states lane + 64 k (every lane of the wave).
template <int D, class Src>
__device__ __forceinline__ void merge_weights(const Src &src, int S, int lane, float &M, float &dsum, float a[4]) {
    float mv[4], dv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane + 64 * k;
        mv[k] = i < S ? src.m(i) : kNegInf;
        dv[k] = i < S ? src.d(i) : 0.0f;
    }
    M = wave_max(fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
    dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = (mv[k] == kNegInf || M == kNegInf) ? 0.0f : fexp2((mv[k] - M) * kLog2e);
        dsum += a[k] * dv[k];
    }
    dsum = wave_sum(dsum);
}

// The rows of group k (zeros past S): this lane's D / 64 elements of each.
template <int D, class Src>
__device__ __forceinline__ void merge_load_group(const Src &src, int S, int k, int lane,
                                                 float x[kMergeGroup][D / 64]) {
    constexpr int NV = D / 64;
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) {
        const int s = k * kMergeGroup + u;
        if (s < S) {
            const float *row = src.row(s) + lane * NV;
            if constexpr (NV == 2) {
                const float2 t = *reinterpret_cast<const float2 *>(row);
                x[u][0] = t.x;
                x[u][1] = t.y;
            } else {
#pragma unroll
                for (int e = 0; e < NV; ++e) x[u][e] = row[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < NV; ++e) x[u][e] = 0.0f;
        }
    }
}

// g = sum over group k's rows, in split order, of alpha_s * row_s.
template <int D>
__device__ __forceinline__ void merge_group_sum(const float x[kMergeGroup][D / 64], const float a[4], int S,
                                                int k, float g[D / 64]) {
    constexpr int NV = D / 64;
    const int j = k >> 1;  // state 32 k + u has its weight in lane 32 (k & 1) + u of a[j]
    const float aj = j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
#pragma unroll
    for (int e = 0; e < NV; ++e) g[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) {
        const float alpha = (k * kMergeGroup + u < S) ? readlane(aj, 32 * (k & 1) + u) : 0.0f;
#pragma unroll
        for (int e = 0; e < NV; ++e) g[e] = __builtin_fmaf(alpha, x[u][e], g[e]);
    }
}

template <int D>
__device__ __forceinline__ void merge_finish(const float acc[D / 64], float M, float dsum, float *out, float *lse,
                                             int lane) {
    constexpr int NV = D / 64;
    if (M == kNegInf) {
#pragma unroll
        for (int e = 0; e < NV; ++e) out[lane * NV + e] = 0.0f;
        if (lse && lane == 0) *lse = kNegInf;
        return;
    }
    const float inv = 1.0f / dsum;
    if constexpr (NV == 2) {
        *reinterpret_cast<float2 *>(out + lane * 2) = make_float2(acc[0] * inv, acc[1] * inv);
    } else {
#pragma unroll
        for (int e = 0; e < NV; ++e) out[lane * NV + e] = acc[e] * inv;
    }
    if (lse && lane == 0) *lse = M + flog2(dsum) * kLn2;
}

// One wave merges every group in turn; the first group's rows are requested
// together with m and d, so up to 32 splits merge in one memory round trip.
template <int D, class Src>
__device__ __forceinline__ void merge_states_wave(const Src &src, int S, float *out, float *lse, int lane) {
    constexpr int NV = D / 64;
    float x[kMergeGroup][NV];
    merge_load_group<D>(src, S, 0, lane, x);
    float M, dsum, a[4];
    merge_weights<D>(src, S, lane, M, dsum, a);
    float acc[NV];
    merge_group_sum<D>(x, a, S, 0, acc);
    const int K = (S + kMergeGroup - 1) / kMergeGroup;
    for (int k = 1; k < K; ++k) {
        merge_load_group<D>(src, S, k, lane, x);
        float g[NV];
        merge_group_sum<D>(x, a, S, k, g);
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[e] += g[e];
    }
    merge_finish<D>(acc, M, dsum, out, lse, lane);
}
template <int D>
__device__ __forceinline__ void merge_states_wave(const float *po, const float *pm, const float *pd, int S,
                                                  float *out, float *lse, int lane) {
    merge_states_wave<D>(ContigStates<D>{po, pm, pd}, S, out, lse, lane);
}

// The waves of a block (nw of them) take the groups of S states side by side,
// wave w groups w, w + nw, ...; the group sums meet in gs and are added in
// group order, which gives the bits of merge_states_wave. Every wave of the
// block calls it (waves without a group only meet the barrier).
template <int D, class Src>
__device__ __forceinline__ void merge_states_block(const Src &src, int S, float *out, float *lse, int lane, int w,
                                                   int nw, float (*gs)[D]) {
    constexpr int NV = D / 64;
    const int K = (S + kMergeGroup - 1) / kMergeGroup;
    float M = kNegInf, dsum = 0.0f, a[4];
    if (w < K || w == 0) {
        float x[kMergeGroup][NV];
        merge_load_group<D>(src, S, w, lane, x);
        merge_weights<D>(src, S, lane, M, dsum, a);
        for (int k = w; k < K; k += nw) {
            if (k != w) merge_load_group<D>(src, S, k, lane, x);
            float g[NV];
            merge_group_sum<D>(x, a, S, k, g);
#pragma unroll
            for (int e = 0; e < NV; ++e) gs[k][lane * NV + e] = g[e];
        }
    }
    __syncthreads();
    if (w != 0) return;
    float acc[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[e] = K > 0 ? gs[0][lane * NV + e] : 0.0f;
    for (int j = 1; j < K; ++j) {
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[e] += gs[j][lane * NV + e];
    }
    merge_finish<D>(acc, M, dsum, out, lse, lane);
}

}  // namespace fdec
