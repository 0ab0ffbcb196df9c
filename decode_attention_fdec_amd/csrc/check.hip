// Device-data checks: the debug mode of the library. In the fast path the
// kernels trust the lengths, page ids, row indices and positions on the device
// (reading a page id past the pool is an out-of-bounds access). The check
// kernel reads them -- never past what the shapes the caller declared allow --
// and reports what is out of range in a word per device, which the host reads
// back; with the debug mode on, every decode entry point runs it first and
// refuses to launch on bad data. The failure modes follow the vLLM notes
// "FlashAttention 與 FlashInfer" (its list of backend failure modes) and the
// paging rules of "Inference Cookbook / 推理優化" §4.2 (page table rows padded
// with -1 past a request's pages).
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fdec.h"
#include "fdec_host.h"
#include "fdec_internal.h"

// [0]: the OR of the FDEC_CHECK_* flags; [1]: the smallest flagged request
// (B for the shared prefix), INT_MAX when none. One copy per GPU.
static __device__ __align__(16) int check_words[2];

namespace fdec {
namespace {

struct CheckParams {
    int B;
    const int32_t *seq_lens;
    int extra_rows;  // rows an append adds
    int capacity;    // rows a request may address
    const int32_t *page_table;
    int max_pages, page_size;
    int num_blocks;  // pages of the pool / rows of a contiguous cache; 0 = unknown
    const int32_t *batch_idx, *leftpad;
    int rope_max_pos;  // 0 = no rotary
    const int32_t *prefix_pages;
    int prefix_len;
};

__global__ void check_init_kernel(int *w) {
    if (threadIdx.x == 0) {
        w[0] = 0;
        w[1] = INT_MAX;
    }
}

__device__ __forceinline__ bool bad_block(int id, int nb) { return id < 0 || (nb > 0 && id >= nb); }

// One thread per request b < B; thread B checks the shared prefix's pages.
__global__ void check_inputs_kernel(const CheckParams c, int *w) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b > c.B) return;
    int f = 0;
    if (b == c.B) {
        if (c.prefix_len > 0) {
            const int n = (c.prefix_len + c.page_size - 1) / c.page_size;
            for (int j = 0; j < n; ++j)
                if (bad_block(c.prefix_pages[j], c.num_blocks)) f |= FDEC_CHECK_PREFIX_PAGE;
        }
    } else {
        const int L = c.seq_lens[b];
        const int64_t rows = (int64_t)L + c.extra_rows;  // rows the call addresses
        if (L < 0 || rows > c.capacity) f |= FDEC_CHECK_LENGTH;
        int lp = 0;
        if (c.leftpad) {
            lp = c.leftpad[b];
            if (lp < 0 || lp > L) f |= FDEC_CHECK_LEFTPAD;
        }
        if (c.batch_idx && bad_block(c.batch_idx[b], c.num_blocks)) f |= FDEC_CHECK_BATCH_IDX;
        if (c.page_table) {
            // only the entries the kernels read: from the page holding the 16-row
            // tile of the first valid row (left padding below it is never read) to
            // the page of the last row, and never past the request's table row
            const int64_t need = rows > 0 ? (rows + c.page_size - 1) / c.page_size : 0;
            const int n = (int)(need < c.max_pages ? need : c.max_pages);
            const int j0 = (lp > 0 && lp <= L) ? (lp & ~15) / c.page_size : 0;
            const int32_t *row = c.page_table + (int64_t)b * c.max_pages;
            for (int j = j0; j < n; ++j)
                if (bad_block(row[j], c.num_blocks)) f |= FDEC_CHECK_PAGE;
        }
        if (c.rope_max_pos > 0 && L >= 0 && (L - lp < 0 || L - lp >= c.rope_max_pos)) f |= FDEC_CHECK_ROPE_POS;
    }
    if (f) {
        atomicOr(&w[0], f);
        atomicMin(&w[1], b);
    }
}

constexpr int kMaxDevices = 64;
struct DeviceWords {
    std::once_flag once;
    int *ptr = nullptr;
    hipError_t err = hipSuccess;
    std::mutex mu;  // one check at a time per device: the words are shared
};
DeviceWords g_words[kMaxDevices];

std::once_flag g_debug_once;
std::atomic<int> g_debug{0};

int debug_on() {
    std::call_once(g_debug_once, [] {
        const char *e = std::getenv("FDEC_DEBUG");
        if (e && *e && std::strcmp(e, "0") != 0) g_debug.store(1);
    });
    return g_debug.load();
}

}  // namespace
}  // namespace fdec

extern "C" void fdec_set_debug(int on) {
    fdec::debug_on();  // the environment is read first, so a later call wins
    fdec::g_debug.store(on ? 1 : 0);
}

extern "C" int fdec_debug_enabled(void) { return fdec::debug_on(); }

extern "C" int fdec_check_inputs(int B, const fdec_kv *kv, const int32_t *seq_lens, const fdec_append *append,
                                 const int32_t *prefix_pages, int prefix_len, int *flags_out, int *first_out,
                                 void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_check_inputs";
    if (!kv || !flags_out) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: kv and flags_out must be non-NULL", fn);
    if (B < 0 || prefix_len < 0) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: B and prefix_len must be >= 0", fn);
    if (B > 0 && !seq_lens) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: seq_lens is NULL", fn);
    if (kv->page_size < 0 || kv->page_size % 16 || (kv->page_size > 0 && (!kv->page_table || kv->max_pages_per_seq < 1)))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: page_size must be 0 or a multiple of 16 with a page table", fn);
    if (prefix_len > 0 && (kv->page_size == 0 || !prefix_pages))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: a prefix needs a paged pool and prefix_pages", fn);
    if (kv->num_blocks < 0) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: num_blocks < 0", fn);
    fdec::CheckParams c;
    std::memset(&c, 0, sizeof(c));
    c.B = B;
    c.seq_lens = seq_lens;
    c.extra_rows = append ? 1 : 0;
    c.capacity = kv->page_size ? kv->max_pages_per_seq * kv->page_size : kv->capacity;
    c.page_table = kv->page_size ? kv->page_table : nullptr;
    c.max_pages = kv->max_pages_per_seq;
    c.page_size = kv->page_size ? kv->page_size : 1;
    c.num_blocks = kv->num_blocks;
    c.batch_idx = kv->page_size ? nullptr : kv->cache_batch_idx;
    c.leftpad = kv->cache_leftpad;
    c.rope_max_pos = append && append->rotary_dim > 0 ? append->rope_max_pos : 0;
    c.prefix_pages = prefix_pages;
    c.prefix_len = prefix_len;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fdec_fail(FDEC_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= fdec::kMaxDevices)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev,
                         fdec::kMaxDevices);
    fdec::DeviceWords &d = fdec::g_words[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(check_words));
        if (d.err == hipSuccess) d.ptr = static_cast<int *>(p);
    });
    if (d.err != hipSuccess || !d.ptr)
        return fdec_fail(FDEC_ERR_HIP, "%s: hipGetSymbolAddress(check_words): %s", fn, hipGetErrorString(d.err));

    std::lock_guard<std::mutex> lock(d.mu);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int words[2] = {0, INT_MAX};
    hipLaunchKernelGGL(fdec::check_init_kernel, dim3(1), dim3(64), 0, st, d.ptr);
    const int threads = 256, blocks = (B + 1 + threads - 1) / threads;
    hipLaunchKernelGGL(fdec::check_inputs_kernel, dim3(blocks), dim3(threads), 0, st, c, d.ptr);
    if ((e = hipGetLastError()) != hipSuccess ||
        (e = hipMemcpyAsync(words, d.ptr, sizeof(words), hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess)
        return fdec_fail(FDEC_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    *flags_out = words[0];
    if (first_out) *first_out = words[0] ? words[1] : -1;
    return FDEC_OK;
}

// With the debug mode on: check the call's device data first, and refuse the
// call (FDEC_ERR_INVALID_ARG, nothing launched) when any of it is out of range.
int fdec_debug_gate(const char *fn, int B, const fdec_kv *kv, const int32_t *seq_lens, const fdec_append *append,
                    const int32_t *prefix_pages, int prefix_len, void *stream) {
    if (!fdec::debug_on()) return FDEC_OK;
    // the check waits for its result on the host, which a stream under graph
    // capture cannot do: captured calls go unchecked
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
        return FDEC_OK;
    int flags = 0, first = -1;
    int rc = fdec_check_inputs(B, kv, seq_lens, append, prefix_pages, prefix_len, &flags, &first, stream);
    if (rc) return rc;
    if (flags)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: device data out of range (check flags 0x%x, first at request %d)",
                         fn, flags, first);
    return FDEC_OK;
}
