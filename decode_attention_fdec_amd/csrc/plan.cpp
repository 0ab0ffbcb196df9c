// Split planners for libfdec. Host-only C++: no HIP calls, so it runs (and is
// tested) on machines without a GPU.
//
// fdec_plan is the MI355X planner: a cost model over the batch's lengths, the
// KV-head count and the compute-unit count, in the spirit of the runtime split
// cost model of the lpnh.cn FlashDecoding explainer (§3, dynamic split: short
// sequences split little, long ones a lot). fdec_plan_rules restates the
// four-rule heuristic of the flash-attn "Inference Cookbook / 推理优化" page
// (§6.3, with §8.2's block count) for comparison with that page's examples.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "../../include/fdec.h"
#include "fdec_host.h"

namespace {

// Model constants for one MI355X (gfx950: 256 CUs, 8 TB/s HBM3E), fitted to
// measurements of this library's map kernels (two-kernel path). A model block
// is one launched block: heads_per_block KV heads over one split.
struct CostModel {
    double bw_total;              // sustained aggregate KV read rate, bytes/s
    double bw_block;              // one map block's ceiling, bytes/s
    int blocks_per_cu;            // map blocks worth running per CU at once
    int heads_per_block;          // KV heads one block reads
    double t_block;               // fixed cost of a non-empty block (q load, epilogue), s
    double t_empty = 0.1e-6;      // an empty block, s
    double t_merge = 3.0e-6;      // merge kernel launch and latency, s
    double bytes_per_token = 2.0 * 128 * 2;  // K + V row of one KV head (D = 128, 2-byte)
    int fill_per_cu = 1;          // (KV head, split) pairs per CU a bandwidth-bound launch needs
};

// G = 4 runs on the matrix-core kernel: blocks of up to 4 KV heads, one block
// per CU (a second resident block adds no bandwidth), about 42 GB/s per block
// below saturation and 5.9 TB/s in aggregate (128k-token GQA: 93 us at 256
// blocks, 107 us at 128). G = 8 runs on its matrix-core kernel with the same
// blocks (128k tokens: 98 us at 256 blocks). Other shapes run on the vector
// kernel, modelled per KV head (its blocks stream each head independently).
// kv8: a float8 cache. A vector-kernel wave then streams the same tokens per
// second as over a 16-bit cache, at half the bytes, so more waves are needed to
// reach the aggregate rate (one 128k-token request, 8 KV heads, G = 1 or 2:
// 54-55 us at 128 splits against 60-75 at 64).
CostModel model_for(int Hq, int Hkv, bool kv8) {
    CostModel cm;
    if (Hq == 4 * Hkv || Hq == 8 * Hkv) {
        int hpb = 1;
        for (int w = 4; w > 1; --w)
            if (Hkv % w == 0) {
                hpb = w;
                break;
            }
        cm.bw_total = 5.9e12;
        cm.bw_block = 42.0e9;
        cm.blocks_per_cu = 1;
        cm.heads_per_block = hpb;
        cm.t_block = 2.0e-6;
        cm.fill_per_cu = 1;
    } else {
        cm.bw_total = 5.4e12;
        cm.bw_block = 35.0e9;
        cm.blocks_per_cu = 2;
        cm.heads_per_block = 1;
        cm.t_block = 3.0e-6;
        cm.fill_per_cu = 2;
        if (kv8) {
            cm.bw_block *= 0.5;
            cm.bytes_per_token *= 0.5;
            cm.fill_per_cu = 4;
        }
    }
    return cm;
}

// Fluid model of one launch: blocks enter free slots in dispatch order (split
// fastest, then KV head, then request); the active blocks share the aggregate
// bandwidth equally, each capped at bw_block. A block's fixed cost is charged
// as bytes at its capped rate. Every active block advances at the same rate, so
// completions happen in order of (progress at entry + bytes): a min-heap of
// those thresholds gives the schedule in O(n log n).
double makespan(const CostModel &cm, const std::vector<double> &bytes, int slots) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> heap;
    size_t next = 0;
    double progress = 0.0, t = 0.0;
    while (next < bytes.size() && (int)heap.size() < slots) heap.push(progress + bytes[next++]);
    while (!heap.empty()) {
        const double n = (double)heap.size();
        const double rate = std::min(cm.bw_block, cm.bw_total / n);
        const double target = heap.top();
        heap.pop();
        t += (target - progress) / rate;
        progress = target;
        if (next < bytes.size()) heap.push(progress + bytes[next++]);
    }
    return t;
}

double estimate(const CostModel &cm, int B, int Hq, int Hkv, const std::vector<int> &lens, int cap,
                int S, int cu_count) {
    const int64_t chunk = fdec_split_chunk(cap, S);
    const int groups = Hkv / cm.heads_per_block;
    const double block_bytes_per_token = cm.bytes_per_token * cm.heads_per_block;
    std::vector<double> bytes;
    bytes.reserve((size_t)B * groups * S);
    // dispatch order of the launch: split fastest, then request, then head group
    for (int g = 0; g < groups; ++g) {
        for (int b = 0; b < B; ++b) {
            for (int s = 0; s < S; ++s) {
                int64_t lo = s * chunk, hi = std::min<int64_t>((int64_t)lens[b], lo + chunk);
                if (hi > lo)
                    bytes.push_back((double)(hi - lo) * block_bytes_per_token + cm.t_block * cm.bw_block);
                else
                    bytes.push_back(cm.t_empty * cm.bw_block);
            }
        }
    }
    double t = makespan(cm, bytes, cu_count * cm.blocks_per_cu);
    // Merge: partial states written and read once more (fp32, D + 2 values).
    if (S > 1) t += cm.t_merge + 2.0 * (double)B * Hq * S * (128 + 2) * 4.0 / cm.bw_total;
    return t;
}

}  // namespace

extern "C" int fdec_plan(int B, int Hq, int Hkv, const int32_t *seq_lens_host, int capacity,
                         int page_size, int cu_count, int *num_splits_out) {
    return fdec_plan_kv(B, Hq, Hkv, seq_lens_host, capacity, page_size, FDEC_BF16, cu_count, num_splits_out);
}

extern "C" int fdec_plan_kv(int B, int Hq, int Hkv, const int32_t *seq_lens_host, int capacity,
                            int page_size, int kv_dtype, int cu_count, int *num_splits_out) {
    fdec_clear_error();
    if (!num_splits_out) return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: num_splits_out is NULL");
    if (kv_dtype != FDEC_F16 && kv_dtype != FDEC_BF16 && kv_dtype != FDEC_FP8_E4M3)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: kv_dtype %d is not an fdec_dtype", kv_dtype);
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: need B >= 0, Hq >= 1, Hkv >= 1, Hq %% Hkv == 0");
    if (capacity < 1) return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: capacity must be >= 1");
    if (page_size < 0 || page_size % 16 != 0)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: page_size must be 0 or a multiple of 16");
    if (cu_count <= 0) cu_count = 256;
    std::vector<int> lens(B > 0 ? B : 0, capacity);
    if (seq_lens_host) {
        for (int b = 0; b < B; ++b) {
            if (seq_lens_host[b] < 0 || seq_lens_host[b] > capacity)
                return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan: seq_lens_host[%d] = %d outside [0, capacity]",
                                 b, seq_lens_host[b]);
            lens[b] = seq_lens_host[b];
        }
    }
    if (B == 0) {
        *num_splits_out = 1;
        return FDEC_OK;
    }
    const CostModel cm = model_for(Hq, Hkv, kv_dtype == FDEC_FP8_E4M3);
    // Candidate split counts: every distinct chunk size, up to 64 blocks per slot.
    const int max_s =
        (int)std::min<int64_t>(FDEC_MAX_SPLITS, ((int64_t)capacity + FDEC_CHUNK_ALIGN - 1) / FDEC_CHUNK_ALIGN);
    const int64_t block_cap = (int64_t)64 * cu_count * cm.blocks_per_cu;
    // The matrix-core kernel reaches its aggregate rate only with a block on
    // every CU (measured: 128 or 192 blocks of a 256-CU part stream at ~5.0
    // TB/s, 256 at 5.9), which the fluid model does not capture: when the
    // launch is bandwidth-bound (its bytes take over 20 us at the aggregate
    // rate), candidates start at one block per CU. Short work keeps the model's
    // choice, which splits little.
    // The vector kernel likewise: a (KV head, split) pair is one wave, and the
    // measured rate needs about two of them per CU (one request, 8 KV heads,
    // 128k tokens: 137 us at 19 splits, 97 us at 64; G = 2: 208 against 100;
    // eight 8k requests at G = 2: 90 us at 3 splits, 53 at 8), so its
    // candidates start at two pairs per CU (four over a float8 cache).
    const int groups = Hkv / cm.heads_per_block;
    // the work in 16-bit bytes: a float8 cache has the same tokens per wave
    double work_bytes = 0.0;
    for (int b = 0; b < B; ++b) work_bytes += (double)lens[b] * (2.0 * 128 * 2) * Hkv;
    // (the vector kernel already from 5 us of reading: 4k tokens x 32 KV heads,
    // 64 MB, 18.3 us at 16 splits against 23.4 at the fluid model's 5)
    const double work_s = work_bytes / cm.bw_total;
    const bool bw_bound = work_s > (cm.blocks_per_cu == 1 ? 20.0e-6 : 5.0e-6);
    // Long vector-kernel launches gain from four pairs per CU over 16-bit caches
    // too (over 20 us of reading; µs at two → four pairs per CU: one 128k-token
    // request with 8 KV heads, G = 1: 101.4 → 98.6, G = 2: 103.6 → 100.1; 32 4k
    // requests, G = 1: 101.1 → 98.0; two 64k requests: 53.1 → 50.7), while
    // shorter ones do not (4 2k requests, G = 2: 14.8 → 15.2).
    const int fill_per_cu = (cm.blocks_per_cu != 1 && work_s > 20.0e-6) ? std::max(cm.fill_per_cu, 4) : cm.fill_per_cu;
    const int64_t fill = (int64_t)fill_per_cu * cu_count;
    const int s_min = bw_bound ? (int)std::max<int64_t>(1, std::min<int64_t>(max_s, (fill + (int64_t)B * groups - 1) /
                                                                                         ((int64_t)B * groups)))
                               : 1;
    double best = 1e30;
    std::vector<std::pair<int, double>> est;
    int64_t last_chunk = -1;
    for (int S = s_min; S <= max_s; ++S) {
        int64_t chunk = fdec_split_chunk(capacity, S);
        if (chunk == last_chunk) continue;
        last_chunk = chunk;
        if ((int64_t)B * groups * S > block_cap && S > s_min) break;
        double t = estimate(cm, B, Hq, Hkv, lens, capacity, S, cu_count);
        est.push_back({S, t});
        best = std::min(best, t);
    }
    // The smallest split count whose estimate is within 2% of the best: fewer
    // splits means fewer partial states to write and merge.
    int pick = s_min;
    for (auto &e : est) {
        if (e.second <= best * 1.02) {
            pick = e.first;
            break;
        }
    }
    *num_splits_out = pick;
    return FDEC_OK;
}

extern "C" int fdec_plan_rules(int B, int Hkv, int sm_count, int max_splits, int *num_splits_out) {
    fdec_clear_error();
    if (!num_splits_out) return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan_rules: num_splits_out is NULL");
    if (B < 1 || Hkv < 1 || sm_count < 1 || max_splits < 1)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_plan_rules: arguments must be >= 1");
    const int64_t blocks = (int64_t)B * Hkv;
    // Rule 1: the blocks already cover 80% of the SMs.
    if ((double)blocks >= 0.8 * sm_count) {
        *num_splits_out = 1;
        return FDEC_OK;
    }
    // Rule 3: SM efficiency of every split count; rule 4: the smallest within 85% of the best.
    std::vector<double> eff(max_splits + 1, 0.0);
    double best = 0.0;
    for (int s = 1; s <= max_splits; ++s) {
        int64_t n = blocks * s;
        int64_t waves = (n + sm_count - 1) / sm_count;
        eff[s] = (double)n / (double)(waves * sm_count);
        best = std::max(best, eff[s]);
    }
    for (int s = 1; s <= max_splits; ++s) {
        if (eff[s] >= 0.85 * best) {
            *num_splits_out = s;
            return FDEC_OK;
        }
    }
    *num_splits_out = 1;
    return FDEC_OK;
}

extern "C" int64_t fdec_split_chunk(int capacity, int num_splits) {
    if (capacity < 1 || num_splits < 1) return 0;
    int64_t per = ((int64_t)capacity + num_splits - 1) / num_splits;
    return (per + FDEC_CHUNK_ALIGN - 1) / FDEC_CHUNK_ALIGN * FDEC_CHUNK_ALIGN;
}
