// Merge kernel: the FlashDecoding reduce stage (lpnh.cn FlashDecoding explainer
// §2 stage 2; tbr8.org "FlashDecoding 与 FlashInfer 深度解析" §2.1 step 3).
// One wave per (request, query head) merges its S partial states; the
// arithmetic is merge_states_wave, shared with the single-kernel path.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const float *__restrict__ po,
                                                                  const float *__restrict__ pm,
                                                                  const float *__restrict__ pd, int BH,
                                                                  int S, float *__restrict__ out,
                                                                  float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
    if (bh >= BH) return;
    merge_states_wave<D>(po + bh * S * D, pm + bh * S, pd + bh * S, S, out + bh * D,
                         lse ? lse + bh : nullptr, lane);
}

hipError_t launch_merge(const float *po, const float *pm, const float *pd, int B, int Hq, int S,
                        int head_dim, float *out, float *lse, hipStream_t st) {
    const int BH = B * Hq;
    dim3 grid((BH + kMergeWaves - 1) / kMergeWaves);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64 * kMergeWaves), 0, st, po, pm, pd, BH, S, out, lse);
    else if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64 * kMergeWaves), 0, st, po, pm, pd, BH, S, out, lse);
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
