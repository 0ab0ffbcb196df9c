// fdec_decode_noalloc: fdec_decode without a workspace argument, for callers
// that cannot allocate device memory at the call (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc). The partial states and
// arrival counters live in a file-scope device array, `scratch`, one copy per
// GPU, which the library holds until the process ends. Host code never passes
// the array's name to a kernel: it resolves each device's address once with
// hipGetSymbolAddress (with that device current) and passes that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fdec.h"
#include "fdec_host.h"
#include "fdec_internal.h"

static __device__ __align__(256) unsigned char scratch[FDEC_NOALLOC_SCRATCH_BYTES];

namespace {

// The first kCounterBytes hold the fused path's arrival counters (cleared by a
// kernel before every fused call); the states start after them, so no call's
// states ever overlap another call's counters.
constexpr size_t kCounterBytes = 64 * 1024;
static_assert(FDEC_NOALLOC_SCRATCH_BYTES > kCounterBytes, "scratch holds the counters and some states");

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    char *ptr = nullptr;        // this device's copy of `scratch`
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's scratch address (resolved on the first call on it).
int current_scratch(const char *fn, char **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fdec_fail(FDEC_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev, kMaxDevices);
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) d.ptr = static_cast<char *>(p);
    });
    if (d.err != hipSuccess || !d.ptr)
        return fdec_fail(FDEC_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                         hipGetErrorString(d.err));
    *ptr = d.ptr;
    return FDEC_OK;
}

}  // namespace

extern "C" int fdec_decode_noalloc(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                                   int num_splits, float softmax_scale, const fdec_append *append, int fused,
                                   float *out, float *lse, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_decode_noalloc";
    int S = 0;
    int rc = fdec_decode_validate(fn, q, B, Hq, kv, seq_lens, num_splits, softmax_scale, append, fused, out, lse, &S);
    if (rc || B == 0) return rc;
    const size_t counters = (size_t)B * kv->num_kv_heads * sizeof(int32_t);
    const size_t states = fdec_decode_state_bytes(B, Hq, kv->head_dim, S);
    if (counters > kCounterBytes || states > FDEC_NOALLOC_SCRATCH_BYTES - kCounterBytes)
        return fdec_fail(FDEC_ERR_WORKSPACE,
                         "%s: %zu bytes of states (%d splits) and %zu of counters exceed the library's scratch of "
                         "%zu and %zu bytes; use fdec_decode with a workspace",
                         fn, states, S, counters, (size_t)FDEC_NOALLOC_SCRATCH_BYTES - kCounterBytes, kCounterBytes);
    char *base = nullptr;
    if ((rc = current_scratch(fn, &base))) return rc;
    int *cnt = reinterpret_cast<int *>(base);
    if (fused) {
        // the counters must start at zero: a kernel clears this call's (no memset
        // node, so a captured graph stays correct on every replay)
        hipError_t e = fdec::launch_zero_words(cnt, counters / sizeof(int32_t), static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fdec_fail(FDEC_ERR_HIP, "%s: counter clear: %s", fn, hipGetErrorString(e));
    }
    return fdec_decode_launch(fn, q, B, Hq, kv, seq_lens, S, softmax_scale, append, fused, out, lse, cnt,
                              base + kCounterBytes, stream);
}
