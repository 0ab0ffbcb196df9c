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

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float wave_max(float x) {
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
    return x;
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

// Merge S <= 256 partial states of one (b, h) with one wave (the reduce stage):
// m = max_i m_i, alpha_i = exp(m_i - m) (0 for an empty state), d = sum alpha_i d_i,
// out = sum alpha_i O~_i / d, lse = m + ln d. States are in natural-log units.
// The same code serves the merge kernel and the single-kernel path, so both give
// bitwise identical results. All loads are lane-varying vector loads; the first
// 32 state rows are requested together with m and d, so up to 32 splits merge in
// one memory round trip. Rows are accumulated in split order.
template <int D>
__device__ __forceinline__ void merge_states_wave(const float *po, const float *pm, const float *pd,
                                                  int S, float *out, float *lse, int lane) {
    constexpr int NV = D / 64;  // output elements per lane
    constexpr int NB = 32;      // rows per batch
    auto load_row = [&](int s, float *x) {
        const float *row = po + (int64_t)s * D + lane * NV;
        if constexpr (NV == 2) {
            const float2 t = *reinterpret_cast<const float2 *>(row);
            x[0] = t.x;
            x[1] = t.y;
        } else {
#pragma unroll
            for (int e = 0; e < NV; ++e) x[e] = row[e];
        }
    };
    float x[NB][NV];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        if (u < S) {
            load_row(u, x[u]);
        } else {
#pragma unroll
            for (int e = 0; e < NV; ++e) x[u][e] = 0.0f;
        }
    }
    float mv[4], dv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int i = lane + 64 * k;
        mv[k] = i < S ? pm[i] : kNegInf;
        dv[k] = i < S ? pd[i] : 0.0f;
    }
    float M = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));
    M = wave_max(M);
    float o[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) o[e] = 0.0f;
    if (M == kNegInf) {
#pragma unroll
        for (int e = 0; e < NV; ++e) out[lane * NV + e] = 0.0f;
        if (lse && lane == 0) *lse = kNegInf;
        return;
    }
    float a[4], dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = mv[k] == kNegInf ? 0.0f : fexp2((mv[k] - M) * kLog2e);
        dsum += a[k] * dv[k];
    }
    dsum = wave_sum(dsum);
    // alpha_s is broadcast from lane s % 64 of register a[s / 64]
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const float alpha = u < S ? readlane(a[0], u) : 0.0f;
#pragma unroll
        for (int e = 0; e < NV; ++e) o[e] += alpha * x[u][e];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = min(64, S - 64 * k);
        for (int j0 = (k == 0 ? NB : 0); j0 < n; j0 += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                if (j0 + u < n) {
                    load_row(64 * k + j0 + u, x[u]);
                } else {
#pragma unroll
                    for (int e = 0; e < NV; ++e) x[u][e] = 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const float alpha = (j0 + u < n) ? readlane(a[k], min(j0 + u, 63)) : 0.0f;
#pragma unroll
                for (int e = 0; e < NV; ++e) o[e] += alpha * x[u][e];
            }
        }
    }
    const float inv = 1.0f / dsum;
    if constexpr (NV == 2) {
        *reinterpret_cast<float2 *>(out + lane * 2) = make_float2(o[0] * inv, o[1] * inv);
    } else {
#pragma unroll
        for (int e = 0; e < NV; ++e) out[lane * NV + e] = o[e] * inv;
    }
    if (lse && lane == 0) *lse = M + flog2(dsum) * kLn2;
}

}  // namespace fdec
