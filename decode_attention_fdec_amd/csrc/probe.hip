// Measurement probes: streaming read and plain copy with 16-byte accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fdec.h"
#include "../../include/fdec_probe.h"
#include "fdec_host.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ src, size_t n,
                                                        uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4 *__restrict__ dst, const uint4 *__restrict__ src,
                                                        size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int fdec_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    fdec_clear_error();
    if (!src || !sink || bytes == 0 || bytes % 16 || !al16(src))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_probe_read: need aligned non-NULL src/sink and bytes %% 16 == 0");
    hipLaunchKernelGGL(read_kernel, dim3(FDEC_PROBE_BLOCKS), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), bytes / 16, sink);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? FDEC_OK : fdec_fail(FDEC_ERR_HIP, "fdec_probe_read: %s", hipGetErrorString(e));
}

extern "C" int fdec_probe_copy(void *dst, const void *src, size_t bytes, void *stream) {
    fdec_clear_error();
    if (!src || !dst || bytes == 0 || bytes % 16 || !al16(src) || !al16(dst))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_probe_copy: need aligned non-NULL pointers and bytes %% 16 == 0");
    hipLaunchKernelGGL(copy_kernel, dim3(FDEC_PROBE_BLOCKS), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4 *>(dst), static_cast<const uint4 *>(src), bytes / 16);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? FDEC_OK : fdec_fail(FDEC_ERR_HIP, "fdec_probe_copy: %s", hipGetErrorString(e));
}
