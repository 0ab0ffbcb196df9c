// Merge kernel: the FlashDecoding reduce stage (lpnh.cn FlashDecoding explainer
// §2 stage 2; tbr8.org "FlashDecoding 与 FlashInfer 深度解析" §2.1 step 3).
// Up to 32 states: one wave per (request, query head) merges them
// (merge_states_wave, shared with the single-kernel path). More states: one
// block per (request, query head), one wave per group of 32 states, each
// group's rows requested at once; the group sums meet in LDS and are added in
// group order, which gives the bits of merge_states_wave.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

// LSE slot of state row `row`. Rows are (request, token, head) with Hq heads
// and q tokens per request; the LSE is [request, head, token] (for q = 1 the
// row itself).
__device__ __forceinline__ int64_t lse_slot(int64_t row, int Hq, int q) {
    if (q <= 1) return row;
    const int64_t bi = row / Hq, h = row - bi * Hq, b = bi / q, i = bi - b * q;
    return (b * Hq + h) * q + i;
}

template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const float *__restrict__ po,
                                                                  const float *__restrict__ pm,
                                                                  const float *__restrict__ pd, int BH,
                                                                  int S, float *__restrict__ out,
                                                                  float *__restrict__ lse, int Hq, int q) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
    if (bh >= BH) return;
    merge_states_wave<D>(po + bh * S * D, pm + bh * S, pd + bh * S, S, out + bh * D,
                         lse ? lse + lse_slot(bh, Hq, q) : nullptr, lane);
}

template <int D>
__global__ __launch_bounds__(64 * (256 / kMergeGroup)) void merge_kernel_groups(
    const float *__restrict__ po, const float *__restrict__ pm, const float *__restrict__ pd, int S,
    float *__restrict__ out, float *__restrict__ lse, int Hq, int q) {
    __shared__ float gs[256 / kMergeGroup][D];
    const int lane = threadIdx.x & 63;
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's group
    const int64_t bh = blockIdx.x;
    const ContigStates<D> src{po + bh * S * D, pm + bh * S, pd + bh * S};
    merge_states_block<D>(src, S, out + bh * D, lse ? lse + lse_slot(bh, Hq, q) : nullptr, lane, k,
                          blockDim.x >> 6, gs);
}

// Balanced-split merge: one block per (b, token, h) (q tokens per request,
// rows token * Hq + h of the [q * Hq, nslots] states). The piece count is known
// only on the device, so the block has kSegWaves waves that take the groups in
// turn.
template <int D>
__global__ __launch_bounds__(64 * (256 / kMergeGroup)) void merge_kernel_segments(
    const float *__restrict__ po, const float *__restrict__ pm, const float *__restrict__ pd,
    const int *__restrict__ meta, int Hq, int q, int nslots, float *__restrict__ out, float *__restrict__ lse) {
    __shared__ float gs[256 / kMergeGroup][D];
    const int lane = threadIdx.x & 63;
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / ((int64_t)q * Hq)), row = (int)(bh - (int64_t)b * q * Hq);
    const int64_t base = (int64_t)row * nslots + meta[2 * b];
    const ContigStates<D> src{po + base * D, pm + base, pd + base};
    merge_states_block<D>(src, meta[2 * b + 1], out + bh * D, lse ? lse + lse_slot(bh, Hq, q) : nullptr, lane, k,
                          blockDim.x >> 6, gs);
}

// Cascade with a balanced suffix: per (b, h) the sp prefix states [B, Hq, sp]
// come first, then the request's suffix pieces as in merge_kernel_segments.
template <int D>
__global__ __launch_bounds__(64 * (256 / kMergeGroup)) void merge_kernel_cascade(
    const float *__restrict__ ppo, const float *__restrict__ ppm, const float *__restrict__ ppd, int sp,
    const float *__restrict__ po, const float *__restrict__ pm, const float *__restrict__ pd,
    const int *__restrict__ meta, int Hq, int nslots, float *__restrict__ out, float *__restrict__ lse) {
    __shared__ float gs[256 / kMergeGroup][D];
    const int lane = threadIdx.x & 63;
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / Hq), h = (int)(bh % Hq);
    const int64_t base = (int64_t)h * nslots + meta[2 * b];
    const TwoRuns<D> src{ContigStates<D>{ppo + bh * sp * D, ppm + bh * sp, ppd + bh * sp},
                         ContigStates<D>{po + base * D, pm + base, pd + base}, sp};
    merge_states_block<D>(src, sp + meta[2 * b + 1], out + bh * D, lse ? lse + bh : nullptr, lane, k,
                          blockDim.x >> 6, gs);
}

// Waves per block of the merges whose state counts only the device knows:
// enough for the usual one or two groups of 32 in one memory round trip, few
// enough that idle waves cost little.
constexpr int kSegWaves = 2;

hipError_t launch_merge_segments(const float *po, const float *pm, const float *pd, const int *meta, int B, int Hq,
                                 int nslots, int max_count, int head_dim, float *out, float *lse,
                                 hipStream_t st, int q_len) {
    const int K = (max(max_count, 1) + kMergeGroup - 1) / kMergeGroup;
    if (K > 256 / kMergeGroup) return hipErrorInvalidValue;
    const dim3 grid((unsigned)B * q_len * Hq), block(64 * min(K, kSegWaves));
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel_segments<128>, grid, block, 0, st, po, pm, pd, meta, Hq, q_len, nslots, out,
                           lse);
    else if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel_segments<64>, grid, block, 0, st, po, pm, pd, meta, Hq, q_len, nslots, out,
                           lse);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_merge_cascade(const float *ppo, const float *ppm, const float *ppd, int sp, const float *po,
                                const float *pm, const float *pd, const int *meta, int B, int Hq, int nslots,
                                int max_count, float *out, float *lse, hipStream_t st) {
    const int K = (sp + max(max_count, 1) + kMergeGroup - 1) / kMergeGroup;
    if (K > 256 / kMergeGroup) return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_kernel_cascade<128>, dim3((unsigned)B * Hq), dim3(64 * min(K, kSegWaves)), 0, st, ppo,
                       ppm, ppd, sp, po,
                       pm, pd, meta, Hq, nslots, out, lse);
    return hipGetLastError();
}

hipError_t launch_merge(const float *po, const float *pm, const float *pd, int B, int Hq, int S,
                        int head_dim, float *out, float *lse, hipStream_t st, int q_len) {
    const int BH = B * q_len * Hq;
    if (S > kMergeGroup) {
        const int K = (S + kMergeGroup - 1) / kMergeGroup;  // <= 8 for S <= 256
        if (K > 256 / kMergeGroup) return hipErrorInvalidValue;
        if (head_dim == 128)
            hipLaunchKernelGGL(merge_kernel_groups<128>, dim3(BH), dim3(64 * K), 0, st, po, pm, pd, S, out, lse, Hq,
                               q_len);
        else if (head_dim == 64)
            hipLaunchKernelGGL(merge_kernel_groups<64>, dim3(BH), dim3(64 * K), 0, st, po, pm, pd, S, out, lse, Hq,
                               q_len);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    dim3 grid((BH + kMergeWaves - 1) / kMergeWaves);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64 * kMergeWaves), 0, st, po, pm, pd, BH, S, out, lse, Hq,
                           q_len);
    else if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64 * kMergeWaves), 0, st, po, pm, pd, BH, S, out, lse, Hq,
                           q_len);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

__global__ void zero_words_kernel(uint32_t *p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(void *ptr, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int bs = 256;
    dim3 grid((unsigned)((n + bs - 1) / bs));
    hipLaunchKernelGGL(zero_words_kernel, grid, dim3(bs), 0, st, reinterpret_cast<uint32_t *>(ptr), n);
    return hipGetLastError();
}

}  // namespace fdec
