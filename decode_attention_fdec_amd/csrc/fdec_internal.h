// Launch parameters shared between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdec {

constexpr int kMapMaxWaves = 8;     // split-KV block: one wave per KV head, up to 8
constexpr int kMapMaxWavesBig = 4;  // ... up to 4 when G * D needs more than 256 registers per lane
constexpr int kMergeWaves = 4;                // (b, h) pairs per merge block
#ifndef FDEC_MFMA_WAVES
#define FDEC_MFMA_WAVES 4
#endif
constexpr int kMapMfmaWaves = FDEC_MFMA_WAVES;  // matrix-core map block (G = 4, D = 128): KV heads

// What happens around the attention itself.
enum MapMode : int {
    kPlain = 0,       // attend to seq_lens[b] tokens
    kAppend = 1,      // write k_new / v_new at row seq_lens[b], attend to seq_lens[b] + 1
    kAppendRope = 2,  // as kAppend, with NeoX rotary of q and k_new
};

struct MapParams {
    const void *q;              // [B, Hq, D]
    const char *k, *v;          // cache base pointers (bytes)
    int64_t s_outer, s_token, s_head;  // element strides
    const int32_t *page_table;  // [B, max_pages] or nullptr (contiguous)
    int max_pages;
    int page_size;
    int page_shift;             // log2(page_size) when a power of two, else -1
    const int32_t *seq_lens;    // [B]
    int B, Hq, Hkv;
    int heads_per_block;        // KV heads (= waves) per block: the largest divisor of Hkv <= 8 (4 for G = 8, D = 128)
    int chunk;                  // tokens per split (multiple of 16)
    float scale_log2;           // softmax scale * log2(e)
    // partial states [B, Hq, s_total, D] / [B, Hq, s_total]; this launch fills
    // split slots [s_offset, s_offset + gridDim.x)
    float *po, *pm, *pd;
    int s_total, s_offset;
    // single-kernel merge: counters [B * Hkv / heads_per_block] (nullptr = no merge in this kernel)
    int *counters;
    float *out, *lse;
    // append
    const void *k_new, *v_new;  // [B, Hkv, D]
    const float *rope_cos, *rope_sin;  // [max_pos, rotary_dim / 2]
    int rotary_dim;
    int mode;                   // MapMode
    int dtype;                  // 0 fp16, 1 bf16
    int head_dim;
    int mfma;                   // 1: matrix-core kernel (map_mfma_eligible)
    // float8 e4m3fn cache (dtype is then the queries' bf16): [B, Hkv] factors or nullptr
    int kv_fp8;
    const float *k_descale, *v_descale;
    // balanced split: states [Hq, nslots] and per-request (first slot, count)
    int *seg_meta;
    int nslots;
    // [B] int32 or nullptr: cache row of request b (contiguous caches), first valid row
    const int32_t *batch_idx, *leftpad;
    // query tokens per request (q [B, q_len, Hq, D], causal) and groups of them along
    // the grid (matrix-core kernel); 1 and 1 for a single query
    int q_len, q_groups;
};

// Whether the matrix-core map kernel can take these parameters (mfma aside).
inline bool map_mfma_eligible(const MapParams &p) {
    return (p.Hq == 4 * p.Hkv || p.Hq == 8 * p.Hkv) && p.head_dim == 128 &&
           (p.page_table == nullptr || p.page_size % 16 == 0) && p.s_token > 0 &&
           p.s_token < (int64_t(1) << 26);  // 16 rows of a tile as 32-bit byte offsets
}

// Grid: (num_splits, B, Hkv / heads_per_block), 64 * heads_per_block threads.
// Runs the matrix-core kernel when p.mfma is set (heads_per_block <= 4).
hipError_t launch_map(const MapParams &p, int num_splits, hipStream_t stream);
hipError_t launch_map_mfma_g4(const MapParams &p, int num_splits, hipStream_t stream);
// Query tokens per wave of the matrix-core map kernels for q_len tokens per
// request: up to 4 in registers, more in groups of 4 along the grid's y axis.
inline int mfma_tokens_per_wave(int q_len) { return q_len <= 1 ? 1 : q_len == 2 ? 2 : 4; }
// Multi-token map kernel on 16x16x32 matrix cores (16-bit or float8 caches,
// head_dim 128, any G): one wave per (split, request, KV head, 16 or 32 query
// rows), kMtWaves waves per block.
constexpr int kMtWaves = 4;
hipError_t launch_map_mt16(const MapParams &p, int num_splits, hipStream_t stream);
// Whether several query tokens (q_len >= 2) take the 16x16x32 kernel: from 8
// query rows per (request, KV head), so every G from two tokens (G = 4 with two
// tokens pads 8 rows into its 16-row block and measured as fast as the 4x4x4
// kernel on bf16 caches, 53 against 70 us on float8 ones, on the 128k request).
inline bool mt16_eligible(int q_len, int G, int head_dim) {
    return head_dim == 128 && (q_len * G >= 8 || (G != 4 && G != 8));
}
// Blocks along z of the 16x16x32 kernels: kMtWaves waves per block, one per
// (KV head, chunk of 16 or 32 query rows).
inline int mt16_row_blocks(int rows) { return rows <= 16 ? 1 : 2; }
inline int mt16_z_blocks(int q_len, int G, int Hkv) {
    const int rows = q_len * G, per = 16 * mt16_row_blocks(rows);
    return (Hkv * ((rows + per - 1) / per) + kMtWaves - 1) / kMtWaves;
}
// Balanced split of the 16x16x32 multi-token kernel: grid (nblocks, 1, z blocks).
hipError_t launch_map_mt16_balanced(const MapParams &p, int nblocks, hipStream_t stream);
// Balanced split over nblocks blocks per group of KV heads (matrix-core kernel).
hipError_t launch_map_mfma_g4_balanced(const MapParams &p, int nblocks, hipStream_t stream);

// Cascade prefix: partial states of every query row over the shared prefix.
constexpr int kPrefixPagesPerBlock = 1024;  // prefix page ids one prefix block stages in LDS
struct CascadeParams {
    const void *q;                  // [B, Hq, D]
    const void *k, *v;              // page pool
    int64_t s_outer, s_token, s_head;
    const int32_t *prefix_pages;    // pages of the shared prefix
    int prefix_len;
    int page_size, page_shift;
    int B, Hq, Hkv;
    int chunk;                      // prefix tokens per split (multiple of 64)
    float scale_log2;
    float *po, *pm, *pd;            // states, slots [s_offset, s_offset + splits)
    int s_total, s_offset;
    int dtype;                      // the queries' (and matrix cores') type: 0 fp16, 1 bf16
    // float8 e4m3fn pool (queries bf16): [B, Hkv] descales of the querying request, or nullptr (1)
    int kv_fp8;
    const float *k_descale, *v_descale;
};
// Grid: (splits, Hkv, ceil(B * Hq / Hkv / 256)).
hipError_t launch_cascade_prefix(const CascadeParams &p, int splits, hipStream_t stream);
// Shared prefix and balanced suffixes (G = 4, four KV heads per suffix block) in
// one launch: sp prefix splits of 128-row chunks and ss suffix blocks per group of
// four KV heads; cascade_fused_blocks gives the two block counts (0 on overflow).
int cascade_fused_blocks(const CascadeParams &cp, int sp, int ss, int *nprefix, int *nsuffix);
hipError_t launch_cascade_fused(const CascadeParams &cp, const MapParams &pb, int sp, int ss, hipStream_t stream);

// One wave per (b, h): merges S states into out / lse.
hipError_t launch_merge(const float *po, const float *pm, const float *pd, int B, int Hq, int S,
                        int head_dim, float *out, float *lse, hipStream_t stream, int q_len = 1);
// Merge of balanced-split states: request b's states are slots
// [meta[2b], meta[2b] + meta[2b+1]) of [Hq, nslots]; max_count bounds the counts.
hipError_t launch_merge_segments(const float *po, const float *pm, const float *pd, const int *meta, int B, int Hq,
                                 int nslots, int max_count, int head_dim, float *out, float *lse,
                                 hipStream_t stream, int q_len = 1);

// Cascade merge with a balanced suffix: per (b, h) the prefix states
// [B, Hq, sp] then request b's suffix pieces (as launch_merge_segments).
hipError_t launch_merge_cascade(const float *ppo, const float *ppm, const float *ppd, int sp, const float *po,
                                const float *pm, const float *pd, const int *meta, int B, int Hq, int nslots,
                                int max_count, float *out, float *lse, hipStream_t stream);

// Zero n 32-bit words with a kernel (no memset node, so graph capture stays safe).
hipError_t launch_zero_words(void *ptr, size_t n_words, hipStream_t stream);

}  // namespace fdec
