// Measurement probes: streaming reads (the attainable read bandwidth) and a
// plain copy with 16-byte accesses (the counters' scale).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/fdec.h"
#include "../../include/fdec_probe.h"
#include "device_common.h"
#include "fdec_host.h"

namespace {

constexpr int kThreads = 256;

// Best-effort streaming read: block b reads one contiguous chunk of the source
// with non-temporal 16-byte loads, kReadUnroll of them in flight per thread.
// Measured on MI355X against other load forms at a 512 MiB footprint (plain
// loads without the non-temporal policy, 2-16 loads in flight, 1-8 blocks per
// compute unit, LDS-DMA rings): this form, two blocks per compute unit, streams
// fastest (~6.8 TB/s).
constexpr int kReadUnroll = 4;
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ src, size_t n,
                                                        uint32_t *__restrict__ sink) {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v *s = reinterpret_cast<const u4v *>(src);
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per, b1 = b0 + per < n ? b0 + per : n;
    uint32_t acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kThreads * kReadUnroll) {
        u4v v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            v[u] = j < b1 ? __builtin_nontemporal_load(s + j) : u4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int st = kThreads / 2; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) red[threadIdx.x] ^= red[threadIdx.x + st];
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

// ---- LDS-DMA streaming reads (the map kernels' load path, without compute)
// A wave moves 4 KB per ring slot: four global_load_lds_dwordx4 of 1 KB each
// (64 lanes x 16 bytes) into its LDS ring, kRing slots deep, with explicit
// vmcnt waits; it then reads one dword per lane of the slot, so the data is
// consumed as the map kernels consume their tiles.
constexpr int kStreamWaves = 4;  // waves per block (one per SIMD)
constexpr int kSlotBytes = 4096;
constexpr int kRing = 4;         // slots per wave: three in flight ahead

// Stream slots [0, n) of `base` (wave-uniform), folding one dword per lane per slot into acc.
__device__ __forceinline__ uint32_t stream_slots(const char *base, int64_t n, uint8_t *ring, int lane) {
    const uint32_t r0 = fdec::lds_addr(ring);
    auto issue = [&](int64_t i) {
        const char *b = base + i * kSlotBytes;
        const uint32_t l = r0 + (uint32_t)(i % kRing) * kSlotBytes;
#pragma unroll
        for (int c = 0; c < 4; ++c) fdec::dma16_kv(b, (uint32_t)(c * 1024 + lane * 16), l + c * 1024);
    };
    const int64_t pro = n < kRing - 1 ? n : kRing - 1;
    for (int64_t i = 0; i < pro; ++i) issue(i);
    uint32_t acc = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (i + kRing - 1 < n) issue(i + kRing - 1);
        const int64_t left = n - 1 - i;
        fdec::wait_vm_n<4>((int)(left < kRing - 1 ? left : kRing - 1));
        acc ^= *reinterpret_cast<const uint32_t *>(ring + (i % kRing) * kSlotBytes + lane * 16);
    }
    return acc;
}

// Static: wave w of W streams slots [w n / W, (w + 1) n / W).
__global__ __launch_bounds__(64 * kStreamWaves) void stream_static_kernel(const char *__restrict__ src, int64_t nslots,
                                                                          uint32_t *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStreamWaves][kRing * kSlotBytes];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t W = (int64_t)gridDim.x * kStreamWaves, w = (int64_t)blockIdx.x * kStreamWaves + wv;
    const int64_t s0 = w * nslots / W, s1 = (w + 1) * nslots / W;
    const uint32_t acc = stream_slots(src + s0 * kSlotBytes, s1 - s0, ring[wv], lane);
    if (lane == 0 && blockIdx.x < FDEC_PROBE_BLOCKS) atomicXor(sink + blockIdx.x, acc);
}

// Ticketed items: the bytes are cut into nitems equal items of ipb slots per
// wave (kStreamWaves * ipb slots per item). Blocks below `first` take item
// blockIdx.x; every later block takes the next ticket from *ticket, item
// first + ticket, and ends at once when that is past the last item. Blocks are
// dispatched to the dies of the GPU in a fixed rotation, but a die that
// streams faster frees its compute units sooner, so its later blocks take more
// of the tickets. The block with the last ticket puts the counter back to 0.
__global__ __launch_bounds__(64 * kStreamWaves) void stream_ticket_kernel(const char *__restrict__ src, int nitems,
                                                                          int ipb, int first, int *ticket,
                                                                          uint32_t *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStreamWaves][kRing * kSlotBytes];
    __shared__ int s_item;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int)blockIdx.x < first) {
        if (threadIdx.x == 0) s_item = blockIdx.x;
    } else if (threadIdx.x == 0) {
        const int t = atomicAdd(ticket, 1);
        if (t == (int)gridDim.x - first - 1) atomicExch(ticket, 0);  // every later block has taken its ticket
        s_item = first + t;
    }
    __syncthreads();
    const int item = s_item;
    if (item >= nitems) return;
    const int64_t s0 = ((int64_t)item * kStreamWaves + wv) * ipb;
    const uint32_t acc = stream_slots(src + s0 * kSlotBytes, ipb, ring[wv], lane);
    if (lane == 0 && blockIdx.x < FDEC_PROBE_BLOCKS) atomicXor(sink + blockIdx.x, acc);
}

int device_cu_count() {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
        cu = 256;
    return cu;
}

}  // namespace

extern "C" int fdec_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    fdec_clear_error();
    if (!src || !sink || bytes == 0 || bytes % 16 || !al16(src))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_probe_read: need aligned non-NULL src/sink and bytes %% 16 == 0");
    const int blocks = std::min(FDEC_PROBE_BLOCKS, 2 * device_cu_count());
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
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

extern "C" int fdec_probe_stream(const void *src, size_t bytes, uint32_t *sink, int mode, int per_cu, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_probe_stream";
    if (!src || !sink || bytes == 0 || bytes % kSlotBytes || (reinterpret_cast<uintptr_t>(src) & 255u))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: need 256-byte aligned src, non-NULL sink, bytes %% 4096 == 0", fn);
    if (per_cu < 1 || per_cu > 4) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: per_cu %d outside [1, 4]", fn, per_cu);
    const int64_t nslots = (int64_t)(bytes / kSlotBytes);
    const int cus = device_cu_count();
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == FDEC_PROBE_STATIC) {
        const int64_t blocks = (int64_t)cus * per_cu;
        if (nslots < blocks * kStreamWaves) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: too few bytes", fn);
        hipLaunchKernelGGL(stream_static_kernel, dim3((unsigned)blocks), dim3(64 * kStreamWaves), 0, st,
                           static_cast<const char *>(src), nslots, sink);
    } else if (mode == FDEC_PROBE_TICKETS) {
        // items of 16 slots (64 KB) per wave, 256 KB per block; the first round of
        // blocks takes items by index, later blocks by ticket; enough later blocks
        // that a die may take half again its share of the ticketed items
        const int ipb = 16;
        const int64_t per_item = (int64_t)ipb * kStreamWaves;
        if (nslots % per_item) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: bytes must be a multiple of 256 KB", fn);
        const int64_t nitems = nslots / per_item;
        const int64_t first = std::min<int64_t>(nitems, (int64_t)cus * per_cu);
        const int64_t later = (nitems - first) + (nitems - first) / 2 + 8;
        if (nitems + later > (int64_t)1 << 30) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: too many bytes", fn);
        hipLaunchKernelGGL(stream_ticket_kernel, dim3((unsigned)(first + later)), dim3(64 * kStreamWaves), 0, st,
                           static_cast<const char *>(src), (int)nitems, ipb, (int)first,
                           reinterpret_cast<int *>(sink + FDEC_PROBE_BLOCKS), sink);
    } else {
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: unknown mode %d", fn, mode);
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? FDEC_OK : fdec_fail(FDEC_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}
