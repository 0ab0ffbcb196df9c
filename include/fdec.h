/*
 * libfdec: split-KV (FlashDecoding) decode attention for AMD Instinct MI355X (gfx950).
 *
 * One query token per request attends to a long, optionally paged KV cache.
 * The KV sequence of every (request, KV head) is cut into splits; each split
 * produces a partial state (O~, m, d) (unnormalised output, local max, local
 * sum of exponentials), and an exact log-sum-exp merge combines the states into
 * the output and its LSE.
 *
 * Pages this interface follows (extracted web text on FlashDecoding):
 *   [tbr8]     "FlashDecoding 与 FlashInfer 深度解析" (tbr8.org): §2.1 the three-step
 *              split / partial / merge method; §3.2 paged KV with plan/run.
 *   [lpnh]     lpnh.cn/news/1601758 FlashDecoding explainer: §2 stage 1 (map: per
 *              split (O~_i, m_i, d_i)) and stage 2 (reduce: alpha merge); §3 the
 *              runtime split cost model, the unified map+reduce kernel, GQA reuse.
 *   [cookbook] "Inference Cookbook / 推理优化" (inference.lei6393.com):
 *              §3.2-3.3 cache_seqlens and KV append (lengths are not advanced by the
 *              library), §3.4 fused NeoX rotary, §3.5 softmax LSE of shape
 *              (batch, heads), §4.2 page table with -1 padding, §6.2 num_splits
 *              (0 = automatic), §6.3 the split heuristic, §8.2 block arithmetic.
 *   [vllm-arch] "FlashAttention 與 FlashInfer:兩大 GPU 注意力後端" (vLLM notes): page
 *              sizes must be multiples of 16; cascade attention computes a shared
 *              prefix once and merges it with per-request suffix attention.
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned (for example torch tensors). The library
 *     never allocates device memory, never synchronises, and launches only on
 *     the caller's stream (`stream` is a hipStream_t; NULL = the null stream).
 *   - Argument validation is host-only and happens before any launch: a failing
 *     call returns a status, launches nothing and records a message readable
 *     with fdec_last_error() on the calling thread.
 *   - Device data is trusted: page ids, lengths and positions out of range are
 *     undefined behaviour (the kernels never read page-table entries past
 *     ceil(L_b / page_size), so -1 padding is safe). The debug mode
 *     (fdec_set_debug, or FDEC_DEBUG=1 in the environment) checks them first in
 *     every decode call, which then waits for that check on its stream.
 *   - Lengths are never modified. With an append, the new token goes to row
 *     seq_lens[b] and attention covers seq_lens[b] + 1 tokens; the caller bumps
 *     the lengths afterwards ([cookbook] §3.2).
 *   - Scores are s_j = scale * q . k_j; lse = ln sum_j exp(s_j) (natural log);
 *     out = sum_j exp(s_j - lse) v_j. A request with no tokens gives out = 0,
 *     lse = -inf.
 *   - Query head h reads KV head h / (Hq / Hkv) (consecutive GQA groups).
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by events).
 */
#ifndef FDEC_H
#define FDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FDEC_OK = 0,
    FDEC_ERR_INVALID_ARG = 1, /* malformed arguments (NULL, negative, misaligned, page size) */
    FDEC_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, dtype, GQA group size */
    FDEC_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than fdec_workspace_size() */
    FDEC_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} fdec_status;

/* Cache element types. FDEC_FP8_E4M3: float8 e4m3fn (OCP) K/V with bf16
 * queries and per-(request, KV head) descales ([cookbook] §7.1-7.2 FP8 KV cache). */
typedef enum { FDEC_F16 = 0, FDEC_BF16 = 1, FDEC_FP8_E4M3 = 2 } fdec_dtype;

/* Largest num_splits accepted by any call. */
#define FDEC_MAX_SPLITS 256
/* Largest q_len of fdec_decode_multi. */
#define FDEC_MAX_QLEN 16
/* Split chunks are whole multiples of this many tokens. */
#define FDEC_CHUNK_ALIGN 16

/*
 * One KV cache; K and V share geometry and element type. Rows are head_dim
 * contiguous elements (D stride 1). Layout (NHD, [cookbook] §3.1, §4.2):
 *   page_size == 0: contiguous, element (b, t, g, d) at b*s_outer + t*s_token + g*s_head + d,
 *                   t < capacity (the per-request row count, max_seqlen);
 *   page_size  > 0: a page pool, element (p, slot, g, d) at
 *                   p*s_outer + slot*s_token + g*s_head + d; logical token j of
 *                   request b is in page page_table[b*max_pages_per_seq + j/page_size],
 *                   slot j % page_size. page_size must be a multiple of 16
 *                   ([vllm-arch] block size rule). capacity must be 0 or
 *                   max_pages_per_seq * page_size.
 * k and v must be 16-byte aligned and every stride a multiple of 16 bytes (8
 * 16-bit or 16 float8 elements). They are written only by an append (one row
 * per request and KV head). Other layouts are described by their strides
 * ([vllm-arch] KV cache shapes), e.g. HND pages [pages, Hkv, page, D]:
 * s_outer = Hkv*page*D, s_token = D, s_head = page*D; one pool
 * [blocks, 2, page, Hkv, D] holding K and V: k = pool, v = pool + page*Hkv*D,
 * s_outer = 2*page*Hkv*D, s_token = Hkv*D, s_head = D (HND pool
 * [blocks, 2, Hkv, page, D] likewise). page_size has no upper bound beyond
 * capacity < 2^31.
 * Float8 caches (dtype FDEC_FP8_E4M3): element (b, t, g, d) stands for its
 * e4m3 value times k_descale[b*Hkv + g] (K) or v_descale[b*Hkv + g] (V); a NULL
 * descale is 1. Queries are bf16. Built for page_size a multiple of 16 (or
 * contiguous): every GQA group size and head_dim in fdec_decode and
 * fdec_decode_partials (the matrix-core map kernel for Hq = 4 or 8 Hkv at
 * head_dim 128, with or without append, the vector kernel otherwise); head_dim 128 for every Hq / Hkv in fdec_decode_balanced, and in
 * fdec_decode_multi and fdec_decode_multi_balanced with q_len > 1 (the 16x16x32 matrix-core kernel widens float8 tiles to
 * bf16 as it reads them); fdec_decode_multi with q_len = 1 takes every shape
 * fdec_decode does; other calls and shapes return FDEC_ERR_UNSUPPORTED. The partial states then
 * already include V's descale.
 */
typedef struct fdec_kv {
    void *k;
    void *v;
    int dtype;        /* fdec_dtype: fp16 or bf16 (q has the same dtype), or float8 (q bf16) */
    int num_kv_heads; /* Hkv */
    int head_dim;     /* D: 128 (64 is also built) */
    int page_size;    /* 0 = contiguous */
    int capacity;     /* contiguous: rows per request; paged: 0 or max_pages_per_seq*page_size */
    int64_t s_outer, s_token, s_head; /* element strides */
    const int32_t *page_table;        /* device [B, max_pages_per_seq] int32, -1 = unused */
    int max_pages_per_seq;
    const float *k_descale;           /* float8 only: device [B, Hkv] fp32, or NULL (1) */
    const float *v_descale;           /* float8 only: device [B, Hkv] fp32, or NULL (1) */
    /* contiguous caches only: device [B] int32, request b reads (and appends
     * to) cache row cache_batch_idx[b] ([cookbook] §5.2); NULL = row b. The
     * cache then has any number of rows >= max(cache_batch_idx) + 1. */
    const int32_t *cache_batch_idx;
    /* device [B] int32 or NULL (0): request b's valid rows start at
     * cache_leftpad[b] ([cookbook] §5.3); it attends to rows
     * [cache_leftpad[b], L_b) with L_b counted from row 0 (seq_lens[b], +1
     * with an append), and an appended row is rotated at its position among
     * the valid rows, seq_lens[b] - cache_leftpad[b]. Requires
     * 0 <= cache_leftpad[b] <= seq_lens[b] (device data, not checked). Split
     * boundaries then count from the 16-row tile holding row cache_leftpad[b]
     * (cache_leftpad[b] rounded down to a multiple of 16), whose rows above the
     * padding are masked. Not in fdec_cascade_decode. */
    const int32_t *cache_leftpad;
    /* pages in a paged pool, or rows (the outer index) of a contiguous cache; 0 =
     * not given. Read only by fdec_check_inputs and the debug mode, to bound
     * page ids and cache_batch_idx. */
    int num_blocks;
} fdec_kv;

/*
 * Optional KV append with fused GPT-NeoX rotary ([cookbook] §3.3-3.4). For each
 * request b with c = seq_lens[b]: k row c of every KV head <- rope(k_new[b,g], p)
 * with p = c - cache_leftpad[b] (p = c without left padding), rounded once
 * (nearest-even) to the cache dtype; v row c <- v_new[b,g] bit copy; the query
 * is rotated by the same position in fp32 before attention. Only q and
 * k are rotated, never v. rotary_dim == 0 appends without rotation. Pairs are
 * (i, i + rotary_dim/2) for i < rotary_dim/2; dims >= rotary_dim are untouched.
 * Float8 caches ([cookbook] §7.2 FP8 KV cache): k_new and v_new are bf16 (the
 * queries' dtype) and each element of the new rows is stored as the e4m3fn
 * code of (value / descale), the k value rotated in fp32 first; the division
 * is fp32, the code the nearest one (ties to even), magnitudes from 448 up
 * saturate to +-448 and NaN stays NaN. Attention then reads the stored codes.
 */
typedef struct fdec_append {
    const void *k_new;    /* device [B, Hkv, D], the queries' dtype, contiguous */
    const void *v_new;    /* device [B, Hkv, D] */
    const float *rope_cos; /* device [rope_max_pos, rotary_dim/2] fp32, or NULL if rotary_dim == 0 */
    const float *rope_sin;
    int rotary_dim;       /* 0 or even, <= head_dim */
    int rope_max_pos;     /* rows of the tables; seq_lens[b] < rope_max_pos (device data, trusted) */
} fdec_append;

/* Short text for a status code. Never NULL. The codes follow the failure
 * modes the vLLM notes list under "邊界與失敗" (an unsupported head size, cache
 * type or block size makes the selector fall back to another backend): a shape
 * this library does not build returns FDEC_ERR_UNSUPPORTED before any launch,
 * so the caller can route it elsewhere; a workspace that is too small returns
 * FDEC_ERR_WORKSPACE with the size it needs in fdec_last_error() instead of
 * allocating (the out-of-memory case of [tbr8] §6.2 problem 1). */
const char *fdec_status_string(int status);

/* Detail message of the most recent failing call on this thread ("" if none). */
const char *fdec_last_error(void);

/*
 * Split planner, MI355X cost model ([lpnh] §3 dynamic split: a runtime cost
 * model over batch, heads, lengths and compute-unit count). Host only, no HIP
 * calls. seq_lens_host: [B] attended lengths on the host, or NULL to assume
 * every request uses the full capacity. cu_count: compute units to fill (256
 * on MI355X; <= 0 means 256). Writes num_splits in [1, FDEC_MAX_SPLITS].
 */
int fdec_plan(int B, int Hq, int Hkv, const int32_t *seq_lens_host, int capacity, int page_size,
              int cu_count, int *num_splits_out);

/*
 * fdec_plan for a cache of element type kv_dtype (an fdec_dtype). fdec_plan is
 * this call with a 16-bit cache. A float8 cache on the vector map kernel
 * (shapes other than Hq = 4 or 8 Hkv) reads half the bytes per token at the
 * same token rate per wave, so it is planned with more splits; the other
 * shapes plan as for 16-bit caches. FDEC_ERR_INVALID_ARG for an unknown
 * kv_dtype, else as fdec_plan. Host only, no HIP calls.
 */
int fdec_plan_kv(int B, int Hq, int Hkv, const int32_t *seq_lens_host, int capacity, int page_size,
                 int kv_dtype, int cu_count, int *num_splits_out);

/*
 * The four-rule split heuristic as the flash-attn cookbook states it
 * ([cookbook] §6.3 with §8.2's block count B*Hkv*num_splits): no split when the
 * blocks already cover 80% of the SMs; otherwise the SM efficiency
 * n/(ceil(n/SMs)*SMs) of n = B*Hkv*s blocks is computed for s = 1..max_splits
 * and the smallest s within 85% of the best is chosen. Kept for comparison
 * with the page's examples; fdec_plan is the MI355X planner. Host only.
 */
int fdec_plan_rules(int B, int Hkv, int sm_count, int max_splits, int *num_splits_out);

/*
 * Tokens per split for a call with this capacity and num_splits:
 * chunk = 16 * ceil(ceil(capacity / num_splits) / 16). Split s of request b
 * covers tokens [s*chunk, min((s+1)*chunk, L_b)) and is empty past L_b
 * ([cookbook] §6.1: equal contiguous KV ranges). Returns 0 on bad arguments.
 */
int64_t fdec_split_chunk(int capacity, int num_splits);

/*
 * Bytes of workspace fdec_decode needs for these sizes (num_splits >= 1); 0 on
 * bad arguments. The workspace is one caller-owned contiguous device buffer
 * that holds the partial states between the map and merge stages, as the
 * workspace buffer handed to FlashInfer's decode wrapper ([tbr8] §3.1-3.2, and
 * §6.2 problem 1 on sizing it for large batches and long sequences). Layout:
 * the fused path's arrival counters [B * Hkv] int32 first, then m, d
 * [B, Hq, S] and O~ [B, Hq, S, D] fp32, each 256-byte aligned.
 * With num_splits = 0 in fdec_decode, a C caller sizes the workspace for the
 * split count the call will use: fdec_plan_kv(B, Hq, Hkv, NULL, capacity,
 * page_size, kv->dtype, 256, &S), then fdec_workspace_size(B, Hq, Hkv, D, S).
 */
size_t fdec_workspace_size(int B, int Hq, int Hkv, int head_dim, int num_splits);

/*
 * Prepare a fresh workspace: zeroes it (in particular the arrival counters the
 * single-kernel (fused) path uses) with a kernel on `stream`. Every call lays
 * out its data after the first B * Hkv 32-bit words of the workspace (rounded
 * up to 256 bytes), which are those counters, and a completed fused call
 * leaves them at zero; so one initialisation serves every later call of any
 * kind with the same or a smaller B * Hkv. Before a fused call whose B * Hkv
 * (B * q_len * Hkv for fdec_decode_multi) exceeds that of a call made since the
 * last initialisation, initialise again. No allocation ([tbr8] §3.1 workspace).
 */
int fdec_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention for B requests ([tbr8] §2.1; [lpnh] §2).
 *   q          device [B, Hq, D], kv->dtype, contiguous, 16-byte aligned.
 *   seq_lens   device [B] int32: attended lengths, or (with append) cache_seqlens
 *              before the append. Never modified.
 *   num_splits >= 1 splits per (request, KV head); 0 = planned from capacity alone
 *              with fdec_plan_kv for kv->dtype (no device read), as num_splits=0
 *              in [cookbook] §6.2.
 *   softmax_scale 0 => 1/sqrt(D).
 *   append     NULL or an fdec_append (the caches in *kv are then written).
 *   fused      0 = map kernel + merge kernel; 1 = one kernel whose last-arriving
 *              block per (request, KV head) merges ([lpnh] §3 unified kernel).
 *              Both give bitwise identical results.
 *   out        device [B, Hq, D] fp32.  lse: device [B, Hq] fp32, or NULL.
 *   workspace  device, >= fdec_workspace_size(B, Hq, Hkv, D, splits used) bytes,
 *              initialised once with fdec_workspace_init when fused = 1.
 */
int fdec_decode(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                int num_splits, float softmax_scale, const fdec_append *append, int fused,
                float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fdec_decode without a workspace, for callers that cannot allocate device
 * memory at the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and results as
 * fdec_decode (bitwise), minus the workspace: the partial states and arrival
 * counters live in the library's own device array of
 * FDEC_NOALLOC_SCRATCH_BYTES, one per GPU, held from the first call on that GPU
 * until the process ends (the first call on a device resolves its address).
 * Calls needing more than that (the states of B * Hq * S splits,
 * fdec_workspace_size minus the counters, beyond FDEC_NOALLOC_SCRATCH_BYTES -
 * 64 KiB, or B * Hkv > 16384) return FDEC_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that array and leaves it holding its own
 * states: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. With fused = 1 a kernel
 * first clears the call's counters. Allocates nothing, never synchronises.
 */
#define FDEC_NOALLOC_SCRATCH_BYTES (16u << 20)
int fdec_decode_noalloc(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens, int num_splits,
                        float softmax_scale, const fdec_append *append, int fused, float *out, float *lse,
                        void *stream);

/*
 * The map stage alone ([lpnh] §2 stage 1): writes every split's partial state
 * for each (b, h) and split s < num_splits (num_splits >= 1 here):
 *   part_o [B, Hq, num_splits, D] fp32  O~ = sum_j exp(s_j - m) v_j over the split,
 *   part_m [B, Hq, num_splits]    fp32  m  = max_j s_j (natural-log units),
 *   part_d [B, Hq, num_splits]    fp32  d  = sum_j exp(s_j - m);
 * an empty split is (0, -inf, 0). Splits follow fdec_split_chunk. Feeding the
 * states to fdec_merge_states gives fdec_decode's result; a caller may also
 * merge states from several devices (decode context parallelism).
 */
int fdec_decode_partials(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                         int num_splits, float softmax_scale, const fdec_append *append,
                         float *part_o, float *part_m, float *part_d, void *stream);

/*
 * The reduce stage ([lpnh] §2 stage 2; [tbr8] §2.1 step 3): for each (b, h),
 * m = max_i m_i, alpha_i = exp(m_i - m) (0 for an empty state), d = sum alpha_i d_i,
 * out = sum alpha_i O~_i / d, lse = m + ln d; all states empty gives out = 0,
 * lse = -inf. Inputs as written by fdec_decode_partials ([B, Hq, S, D], [B, Hq, S],
 * [B, Hq, S], fp32, contiguous); states need not use a true local max: any
 * reference m_i with O~_i, d_i scaled to it merges identically. lse may be NULL.
 * 1 <= S <= FDEC_MAX_SPLITS.
 */
int fdec_merge_states(const float *part_o, const float *part_m, const float *part_d, int B, int Hq,
                      int S, int head_dim, float *out, float *lse, void *stream);

/*
 * Multi-token decode: q_len query tokens per request, e.g. the draft tokens of
 * speculative decoding ([vllm-arch] spec-decode batches), under the causal mask
 * the pages' calls pass. Query token i of request b is the request's row
 * L_b - q_len + i (L_b = seq_lens[b], counted from row 0; the new tokens' K and
 * V are already in the cache) and attends to rows [cache_leftpad[b],
 * L_b - q_len + i]; a token with no rows gives out = 0, lse = -inf. The q_len
 * tokens share each KV tile: the cache is read once per request, as for one
 * query.
 *   q    device [B, q_len, Hq, D], the cache's 16-bit dtype (bf16 for float8)
 *   out  device [B, q_len, Hq, D] fp32; lse device [B, Hq, q_len] fp32 or NULL
 *        ([cookbook] §3.5 softmax_lse shape (batch, heads, seqlen_q))
 *   num_splits, softmax_scale as in fdec_decode (splits over the request's rows)
 *   1 <= q_len <= FDEC_MAX_QLEN. q_len = 1 runs fdec_decode's map and merge
 *   kernels: every shape fdec_decode takes without append, and the result is
 *   fdec_decode's two-kernel result bitwise. q_len > 1 is built for head_dim
 *   128, page_size a multiple of 16 or contiguous, every Hq / Hkv and every
 *   cache dtype (FDEC_ERR_UNSUPPORTED otherwise): the 16x16x32 matrix-core
 *   kernel over 16-row blocks of the q_len * Hq / Hkv query rows of a (request,
 *   KV head); no append. workspace >= fdec_workspace_size(B * q_len, Hq, Hkv,
 *   head_dim, S).
 */
int fdec_decode_multi(const void *q, int B, int q_len, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                      int num_splits, float softmax_scale, float *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Decode with a balanced split ([lpnh] §3: the work cut to fill every compute
 * unit whatever the mix of lengths). Per group of KV heads, the 16-token tiles
 * of all B requests, taken in request order, are cut into num_blocks equal
 * contiguous ranges, one block each; a range may cover the end of one request
 * and the start of the next, and its block writes one partial state per
 * request piece. A merge then combines each request's pieces; the result is
 * fdec_decode's up to rounding. The ranges are computed on the device from
 * seq_lens (no host copy of the lengths), so the call may be captured in a
 * graph whose lengths change between replays.
 *   Supported for every G = Hq/Hkv (G = 4 and 8 on their single-query
 *   matrix-core kernels, G = 1 and 2 on the 16x16x32 kernel with its 16-row
 *   block padded), head_dim 128, page_size a multiple of 16 (or contiguous), no
 *   append: FDEC_ERR_UNSUPPORTED otherwise.
 *   num_blocks  blocks per group of KV heads, 1..256; 0 = per compute unit of
 *               the current device over all groups, one block for fp16/bf16
 *               caches and two for float8 caches (measured best on MI355X).
 *   Requires B * ceil(capacity / 16) < 2^31 (FDEC_ERR_INVALID_ARG otherwise).
 *   out / lse as in fdec_decode. workspace >= fdec_balanced_workspace_size()
 *   bytes (no initialisation needed).
 */
int fdec_decode_balanced(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                         int num_blocks, float softmax_scale, float *out, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Workspace bytes for fdec_decode_balanced (num_blocks as there; 0 = enough for
 * the default of every cache dtype). fdec_decode_multi_balanced takes
 * fdec_balanced_workspace_size(B, q_len * Hq, Hkv, head_dim, num_blocks). */
size_t fdec_balanced_workspace_size(int B, int Hq, int Hkv, int head_dim, int num_blocks);

/*
 * fdec_decode_multi on the balanced split: q_len query tokens per request
 * (q [B, q_len, Hq, D], out [B, q_len, Hq, D], lse [B, Hq, q_len], causal as in
 * fdec_decode_multi) with the work of all requests cut into num_blocks equal
 * tile ranges per group of KV heads as in fdec_decode_balanced (0 = one block
 * per compute unit over all groups). 1 <= q_len <= FDEC_MAX_QLEN. q_len = 1: the
 * shapes and errors of fdec_decode_balanced, and its result bitwise; q_len > 1:
 * the shapes of fdec_decode_multi.
 */
int fdec_decode_multi_balanced(const void *q, int B, int q_len, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                               int num_blocks, float softmax_scale, float *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Cascade decode with a shared prefix ([vllm-arch] cascade attention): all B
 * requests share the first prefix_len tokens, stored once in the pages
 * prefix_pages[0 .. ceil(prefix_len/page_size)); request b then has
 * suffix_lens[b] tokens of its own in kv->page_table row b. The prefix is read
 * once for all requests (matrix-core kernel over the B*G query rows of each KV
 * head), the suffixes by the split-KV kernel, and one merge combines both:
 * the result equals fdec_decode over the concatenated [prefix; suffix]
 * sequence. kv must be paged, head_dim 128. splits_prefix / splits_suffix >= 1
 * (0 = fdec_cascade_plan_kv's choice for the pool's type, a planned count
 * reduced to fit beside a count the caller gave); the prefix is cut into chunks of
 * 64 * ceil(ceil(prefix_len / splits_prefix) / 64) tokens, each of at most 1022
 * pages. With G = Hq/Hkv = 4 the suffixes run on the balanced split (as
 * fdec_decode_balanced) and splits_suffix is its block count per group of KV
 * heads; otherwise splits_suffix splits every suffix (as fdec_decode). With
 * G = 4 and Hkv a multiple of 4, the prefix blocks (128 query rows each) and
 * the suffix blocks share one launch, so that the matrix-core prefix work and
 * the streaming suffix work run side by side on every compute unit (two
 * launches, prefix then suffix, when FDEC_CASCADE_PATH=two is set in the
 * environment); the states and the merge are the same either way. At most
 * FDEC_MAX_SPLITS states merge per request: splits_prefix + splits_suffix
 * <= FDEC_MAX_SPLITS. Workspace: fdec_cascade_workspace_size().
 */
int fdec_cascade_decode(const void *q, int B, int Hq, const fdec_kv *kv,
                        const int32_t *prefix_pages, int prefix_len, const int32_t *suffix_lens,
                        int splits_prefix, int splits_suffix, float softmax_scale, float *out,
                        float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split counts for fdec_cascade_decode (host only), with at least 256 prefix
 * tokens per prefix split. When prefix and suffix share one launch (G = 4, Hkv
 * a multiple of 4), each role gets at most one block per compute unit: prefix
 * blocks of 128 query rows on three quarters of the units for 16-bit pools and
 * on all of them for float8 pools (measured on MI355X, the 64-request
 * shared-prefix workload: 70 against 76 us, and 61 against 68 us), and one
 * balanced-split suffix block per unit. Otherwise the prefix kernel (256 query
 * rows per block) gets about one block per compute unit, and the suffix count
 * is, for G = 4, the balanced split's block count per group of KV heads (one
 * block per compute unit; two for float8 pools) and else fdec_plan's split count
 * over the suffix page table's capacity. prefix_len >= 0; capacity =
 * max_pages_per_seq * page_size of the suffix table. fdec_cascade_plan_kv plans
 * for a pool of element type kv_dtype (an fdec_dtype; fdec_cascade_plan is it
 * with a 16-bit pool), within splits_prefix + splits_suffix <= FDEC_MAX_SPLITS.
 */
int fdec_cascade_plan_kv(int B, int Hq, int Hkv, int prefix_len, int capacity, int page_size, int kv_dtype,
                         int cu_count, int *splits_prefix_out, int *splits_suffix_out);
int fdec_cascade_plan(int B, int Hq, int Hkv, int prefix_len, int capacity, int page_size, int cu_count,
                      int *splits_prefix_out, int *splits_suffix_out);

/* Workspace bytes for fdec_cascade_decode with these split counts (both >= 1). */
size_t fdec_cascade_workspace_size(int B, int Hq, int Hkv, int head_dim, int splits_prefix,
                                   int splits_suffix);

/*
 * Stage timing (tracing). After fdec_trace_start(max_events), every call the
 * calling thread makes records a HIP event on its stream before its first
 * kernel and after each kernel it launches, up to max_events events in all
 * (2..2^20; the events are the library's own). fdec_trace_stop ends the trace,
 * waits for the last event, and writes for i = 1 .. n-1 the interval between
 * event i-1 and event i to intervals_ms[i-1] (ms, at most `capacity` of them)
 * and the kind of event i to kinds[i-1]: k >= 1 for the end of a call's k-th
 * kernel (so the interval is that kernel's time on the stream, launches queued
 * back to back), 0 for the start of a call (the interval is the gap since the
 * previous call's last kernel). *count_out = n, the events recorded. Either
 * array may be NULL. Tracing adds an event record per kernel; it is for
 * measurement, off by default. Host-side; no device memory is allocated.
 */
int fdec_trace_start(int max_events);
int fdec_trace_stop(float *intervals_ms, int *kinds, int capacity, int *count_out);

/*
 * Device-data check ([vllm-arch] the backend's failure modes; [cookbook] §4.2 page
 * tables padded with -1 past a request's pages). Reads, on `stream`, what a
 * decode call with these arguments would trust: seq_lens[b] (plus one row with an
 * append) within [0, capacity]; page-table entries covering those rows (never
 * past max_pages_per_seq) in [0, num_blocks); cache_batch_idx[b] in
 * [0, num_blocks) (contiguous caches); 0 <= cache_leftpad[b] <= seq_lens[b];
 * with a rotary append, the position seq_lens[b] - cache_leftpad[b] below
 * rope_max_pos; the ceil(prefix_len / page_size) prefix_pages in [0, num_blocks).
 * Page entries below the one holding the 16-row tile of cache_leftpad[b] are
 * not read (the kernels never read them). Upper bounds on ids apply only when
 * kv->num_blocks > 0. Writes the OR of the
 * FDEC_CHECK_* flags of what is out of range to *flags_out (0: nothing) and the
 * smallest request flagged (B for the prefix, -1 for none) to *first_out (may be
 * NULL). Waits for the check (hipStreamSynchronize): not for graph capture. The
 * check uses one device word per GPU, guarded by a host lock. FDEC_ERR_INVALID_ARG
 * for NULL or malformed arguments, FDEC_ERR_HIP if a HIP call fails.
 */
enum {
    FDEC_CHECK_LENGTH = 1,       /* seq_lens[b] < 0, or its rows past the capacity */
    FDEC_CHECK_PAGE = 2,         /* a page id the request's rows cover is < 0 or >= num_blocks */
    FDEC_CHECK_LEFTPAD = 4,      /* cache_leftpad[b] < 0 or > seq_lens[b] */
    FDEC_CHECK_BATCH_IDX = 8,    /* cache_batch_idx[b] < 0 or >= num_blocks */
    FDEC_CHECK_ROPE_POS = 16,    /* the appended row's rotary position outside the tables */
    FDEC_CHECK_PREFIX_PAGE = 32  /* a shared-prefix page id < 0 or >= num_blocks */
};
int fdec_check_inputs(int B, const fdec_kv *kv, const int32_t *seq_lens, const fdec_append *append,
                      const int32_t *prefix_pages, int prefix_len, int *flags_out, int *first_out, void *stream);

/*
 * The debug mode: with it on, fdec_decode, fdec_decode_noalloc,
 * fdec_decode_partials, fdec_decode_balanced, fdec_decode_multi,
 * fdec_decode_multi_balanced and fdec_cascade_decode run fdec_check_inputs on
 * their own arguments before any launch and return FDEC_ERR_INVALID_ARG (message
 * in fdec_last_error()) without launching when a flag is set. The check waits
 * for its result, which a stream under graph capture cannot: calls made while
 * their stream is capturing launch unchecked. Off by default; FDEC_DEBUG set to
 * anything but "0" in the environment turns it on at the first call;
 * fdec_set_debug overrides it (process-wide).
 */
void fdec_set_debug(int on);
int fdec_debug_enabled(void);

#ifdef __cplusplus
}
#endif

#endif /* FDEC_H */
