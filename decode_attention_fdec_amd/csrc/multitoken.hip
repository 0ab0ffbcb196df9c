// Multi-token decode map kernel on 16x16x32 matrix cores (gfx950).
//
// The split-KV map stage (lpnh.cn FlashDecoding explainer §2 stage 1) for q_len
// query tokens per request (speculative decode, vLLM notes spec-decode
// batches) under the causal mask of the pages' calls: query token i of request
// b is its row L_b - q_len + i and sees rows [leftpad, L_b - q_len + i]. The
// q_len * G query rows of one (request, KV head) -- G query heads per KV head --
// form the row blocks of v_mfma_f32_16x16x32_{bf16,f16}, so the contraction is
// dense for any G once q_len * G reaches 16; below that the row blocks are
// padded. It takes every call with two or more query tokens, and the balanced
// split's single-query calls at G = 1, 2 (the 4x4x4 kernel's multi-token tiles
// in split_kv_mfma.hip remain as the path FDEC_MULTI_PATH forces).
//
// One wave per (split, request, KV head, chunk of 32 query rows); a block
// holds kMtWaves such waves, each with a private LDS ring. Per 32-key tile:
//   - K and V rows go global -> LDS by LDS-DMA (no registers), 4 rows per
//     instruction (a page holds a multiple of 16 rows, so 4 rows lie on one
//     page), 16-byte pieces of row r in slot piece ^ (r mod 16); float8 caches
//     (the pages' FP8 KV cache, bf16 queries): 128-byte rows, 8 per instruction,
//     piece slots swizzled by fp8_row_swz, widened to bf16 in registers after
//     each LDS read (K: an 8-byte read; V: an 8-bit transpose read), the
//     request's descales applied to the scores and to the output;
//   - S^T = K Q^T: A = 16 keys x 32 d of K from LDS, B = Q^T held in registers,
//     so lane l's result column is query row l % 16 and its four values four
//     keys of that row: each lane applies its row's causal limit;
//   - online softmax per query row in the log2 domain (lazily moved reference),
//     P entering P V as hi + lo, two 16-bit parts (fp32-level accuracy);
//   - O += P V: A = P straight from the S^T registers (key order inside the K
//     dimension permuted alike for A and B), B = V^T from two ds_read_b64_tr_b16
//     of the row-major V tile.
// Layout of v_mfma_f32_16x16x32 (lane l, kq = l / 16): A holds row l % 16,
// k = 8 kq .. 8 kq + 7; B holds column l % 16, k = 8 kq .. 8 kq + 7; D holds
// rows 4 kq .. 4 kq + 3 of column l % 16.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;
typedef int i32x2_v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_v lds_i32x2;

template <int DT> struct Mfma16;
template <> struct Mfma16<0> {
    static __device__ __forceinline__ f32x4_v run(uint4 a, uint4 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a), __builtin_bit_cast(f16x8_v, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct Mfma16<1> {
    static __device__ __forceinline__ f32x4_v run(uint4 a, uint4 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                       __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
    }
};

// Two 16-bit values packed (lo, hi), rounded to nearest even by the hardware.
template <int DT> __device__ __forceinline__ uint32_t mt_pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t mt_pack2<0>(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t mt_pack2<1>(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2{(__bf16)a, (__bf16)b});
}

constexpr int kMtKeys = 32;                  // keys per tile
constexpr int kMtTileBytes = kMtKeys * 256;  // 32 rows of 128 16-bit elements (float8: the first half)
constexpr int kMtNS = 2;                     // ring slots per wave (one tile in flight ahead)
// DMA instructions per tile: K and V, 4 rows (16-bit) or 8 rows (float8) each
template <int KF> struct MtDma {
    static constexpr int kValue = 2 * kMtKeys / (KF ? 8 : 4);
};
constexpr float kMtTau = 8.0f;
constexpr float kMtFloor = -1.0e30f;

}  // namespace

// The running softmax of a wave's query rows (row 16 rb + li in the S^T
// layout; O rows 16 rb + 4 kq + r) and O as hi / lo accumulators.
template <int RB> struct Mt16State {
    float m[RB], tmax[RB], l[RB];
    f32x4_v o[RB][8], ol[RB][8];
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m[rb] = kMtFloor;
            tmax[rb] = kNegInf;
            l[rb] = 0.0f;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                o[rb][db] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
                ol[rb][db] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    }
};

// The query rows of a wave: per lane (S^T column li of row block rb) the Q^T
// B operand and the key limit lim (keys [t_lo, lim) count; t_lo for rows past
// R). Rows are (token i, head) = (r / G, r % G) of request b, KV head g.
template <int RB>
__device__ __forceinline__ void mt16_rows(const MapParams &p, int b, int g, int G, int R, int r0, int L, int t_lo,
                                          int lane, uint4 (&qb)[RB][4], int (&lim)[RB]) {
    constexpr int D = 128;
    const int kq = lane >> 4, li = lane & 15;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = r0 + 16 * rb + li;
        const bool ok = r < R;
        const int i = ok ? r / G : 0, hh = ok ? r - (r / G) * G : 0;
        lim[rb] = ok ? L - p.q_len + i + 1 : t_lo;
        const uint16_t *qrow =
            reinterpret_cast<const uint16_t *>(p.q) + (((int64_t)b * p.q_len + i) * p.Hq + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[rb][ks] = ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * kq) : make_uint4(0, 0, 0, 0);
    }
}

// DMA of the 32-key tile at token t0 of request b (contiguous row crow), KV
// head g, into K / V tiles kt / vt: 8 groups of 4 rows (16-bit) or 4 groups of 8
// rows (float8); tile rows below lo and above hi (outside the valid rows) repeat
// the nearest valid row. t0 is a multiple of 16 and pages hold a multiple of 16
// rows, so each 16-row half of the tile lies in one page: at most two page ids
// per tile, both read before any address needs them.
template <bool PAGED, int KF>
__device__ __forceinline__ void mt16_issue(const MapParams &p, int b, int64_t crow, int g, int t0, int lo, int hi,
                                           uint8_t *kt, uint8_t *vt, int lane) {
    constexpr int ES = KF ? 1 : 2;   // bytes per element
    constexpr int RW = KF ? 8 : 4;   // rows per instruction (1 KB)
    constexpr int LPR = 64 / RW;     // lanes per row (16-byte pieces)
    const uint32_t stok = (uint32_t)(p.s_token * ES);
    int64_t half[2];  // element offset of token t0 + 16 h
    if constexpr (PAGED) {
        typedef const __attribute__((address_space(4))) int32_t *cpage_t;
        const cpage_t row = (cpage_t)(p.page_table + (int64_t)b * p.max_pages);
        const int t1 = t0 + 16;
        const int i0 = p.page_shift >= 0 ? (t0 >> p.page_shift) : (t0 / p.page_size);
        // the second half's page exists only when a valid row lies there
        const int i1 = hi >= 16 ? (p.page_shift >= 0 ? (t1 >> p.page_shift) : (t1 / p.page_size)) : i0;
        const int64_t pg0 = row[i0], pg1 = row[min(i1, p.max_pages - 1)];
        half[0] = pg0 * p.s_outer + (int64_t)(t0 - i0 * p.page_size) * p.s_token + (int64_t)g * p.s_head;
        half[1] = pg1 * p.s_outer + (int64_t)(t1 - i1 * p.page_size) * p.s_token + (int64_t)g * p.s_head;
    } else {
        half[0] = crow * p.s_outer + (int64_t)t0 * p.s_token + (int64_t)g * p.s_head;
        half[1] = half[0] + 16 * p.s_token;
    }
#pragma unroll
    for (int gi = 0; gi < kMtKeys / RW; ++gi) {
        const int g0 = RW * gi;
        const int rs = min(max(g0, lo), hi);  // the group's first source row
        const int h = rs >> 4;                // its half of the tile
        const int base = rs & ~(RW - 1);      // the RW-aligned block holding every source row
        const int64_t eoff = half[h] + (int64_t)(base - 16 * h) * p.s_token;
        const int r = g0 + lane / LPR;
        const int src = min(max(r, lo), hi) - base;  // 0 .. RW - 1
        const int sw = KF ? fp8_row_swz(r) : (r & 15);
        const uint32_t voff = (uint32_t)src * stok + 16u * (uint32_t)((lane % LPR) ^ sw);
        dma16_kv(reinterpret_cast<const char *>(p.k) + eoff * ES, voff, lds_addr(kt) + (uint32_t)(128 * ES * g0));
        dma16_kv(reinterpret_cast<const char *>(p.v) + eoff * ES, voff, lds_addr(vt) + (uint32_t)(128 * ES * g0));
    }
}

// One 32-key tile at token t0: S^T = K Q^T, online softmax per query row (keys
// [t_lo, lim[rb]) count), O += P V. srow: the wave's LDS row factors. Float8
// tiles (KF = 1, bf16 queries) are widened to bf16 as they are read; scale_log2
// then carries the K descale.
template <int DT, int RB, int KF>
__device__ __forceinline__ void mt16_tile(const uint8_t *K, const uint8_t *V, const uint4 (&qb)[RB][4], int t0,
                                          int t_lo, const int (&lim)[RB], float scale_log2, int lane,
                                          Mt16State<RB> &st, float (*srow)[16 * RB]) {
    const int kq = lane >> 4, li = lane & 15;
    // ---- S^T = K Q^T: s[kb][rb] holds keys 16kb + 4kq + r of row 16rb + li
    f32x4_v s[2][RB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kr = 16 * kb + li;
            uint4 a;
            if constexpr (KF == 1) {
                // elements d = 32ks + 8kq .. + 7: half kq & 1 of piece 2ks + kq / 2
                const uint2 k8 = *reinterpret_cast<const uint2 *>(
                    K + kr * 128 + 16 * ((2 * ks + (kq >> 1)) ^ fp8_row_swz(kr)) + 8 * (kq & 1));
                const uint2 lo = fp8x4_to_bf16(k8.x), hi = fp8x4_to_bf16(k8.y);
                a = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
                a = *reinterpret_cast<const uint4 *>(K + kr * 256 + 16 * ((4 * ks + kq) ^ (kr & 15)));
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[kb][rb] = Mfma16<DT>::run(a, qb[rb][ks], s[kb][rb]);
        }
    }

    // ---- online softmax per query row
    bool move = false;
    float mx[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float x = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 16 * kb + 4 * kq + r;
                float v = s[kb][rb][r] * scale_log2;
                if (t < t_lo || t >= lim[rb]) v = kNegInf;
                s[kb][rb][r] = v;
                x = fmaxf(x, v);
            }
        x = fmaxf(x, shfl_xor(x, 16));
        x = fmaxf(x, shfl_xor(x, 32));
        mx[rb] = x;
        st.tmax[rb] = fmaxf(st.tmax[rb], x);
        move |= x > st.m[rb] + kMtTau;
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
        // move the reference; O rows live in lanes by (kq, r), so the per-row
        // factors go through LDS
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float mn = fmaxf(st.m[rb], mx[rb]);
            const float alpha = fexp2(st.m[rb] - mn);
            st.m[rb] = mn;
            st.l[rb] *= alpha;
            if (kq == 0) srow[0][16 * rb + li] = alpha;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float alpha = srow[0][16 * rb + 4 * kq + r];
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    st.o[rb][db][r] *= alpha;
                    st.ol[rb][db][r] *= alpha;
                }
            }
        __builtin_amdgcn_wave_barrier();
    }
    // P as hi + lo, packed as the A operand of P V: K-slot 8kq + e is key
    // 4kq + e (e < 4) or 16 + 4kq + (e - 4) (e >= 4)
    uint4 pah[RB], pal[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        uint32_t wh[4], wl[4];
        float ps = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pv[r] = fexp2(s[kb][rb][r] - st.m[rb]);
                ps += pv[r];
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t h = mt_pack2<DT>(pv[2 * e], pv[2 * e + 1]);
                wh[2 * kb + e] = h;
                wl[2 * kb + e] = mt_pack2<DT>(pv[2 * e] - Elem<DT>::lo(h), pv[2 * e + 1] - Elem<DT>::hi(h));
            }
        }
        pah[rb] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        pal[rb] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
        st.l[rb] += ps;
    }

    // ---- O += P V: B operand of K-slots 8kq .. 8kq + 7 at d = 16db + li from two
    // transpose reads whose lane m (of 16) addresses key row 4kq + m / 4 (+ 16),
    // d 16db + 4 (m % 4) .. + 3. Float8: one 8-bit transpose read (in each group
    // of 16 lanes, lane j gets byte j % 8 of the 8-byte pieces of lanes j / 8 + 2k,
    // k = 0..7) whose lane m addresses the (m / 2)-th of the same 8 keys, bytes
    // 16db + 8 (m & 1) .. + 7.
    if constexpr (KF == 1) {
        const int k8 = li >> 1;
        const int rv0 = k8 < 4 ? 4 * kq + k8 : 16 + 4 * kq + (k8 - 4);
        const uint8_t *vrow = V + rv0 * 128 + 8 * (li & 1);
        const int vsw = fp8_row_swz(rv0);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const i32x2_v x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(vrow + 16 * (db ^ vsw)));
            const uint2 v0 = fp8x4_to_bf16((uint32_t)x[0]), v1 = fp8x4_to_bf16((uint32_t)x[1]);
            const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                st.o[rb][db] = Mfma16<DT>::run(pah[rb], bop, st.o[rb][db]);
                st.ol[rb][db] = Mfma16<DT>::run(pal[rb], bop, st.ol[rb][db]);
            }
        }
    } else {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int ra = 4 * kq + (li >> 2), rb2 = ra + 16;
            const int piece = 2 * db + ((li & 3) >> 1), half = 8 * (li & 1);
            const s16x4_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(V + ra * 256 + 16 * (piece ^ (ra & 15)) + half));
            const s16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(V + rb2 * 256 + 16 * (piece ^ (rb2 & 15)) + half));
            const uint2 v0 = __builtin_bit_cast(uint2, x0), v1 = __builtin_bit_cast(uint2, x1);
            const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                st.o[rb][db] = Mfma16<DT>::run(pah[rb], bop, st.o[rb][db]);
                st.ol[rb][db] = Mfma16<DT>::run(pal[rb], bop, st.ol[rb][db]);
            }
        }
    }
}

// The rows' states against their true maximum T: O~ = O 2^(m - T) vdesc,
// d = l 2^(m - T), m = T ln 2 (empty: (0, -inf, 0)). Query row rr = r0 + local row (rows < R)
// goes to state index slot(i, head) of po / pm / pd.
template <int RB, class SlotOf>
__device__ __forceinline__ void mt16_write(const MapParams &p, const Mt16State<RB> &st, float (*srow)[16 * RB],
                                           int r0, int R, int G, int lane, float vdesc, SlotOf slot) {
    constexpr int D = 128;
    const int kq = lane >> 4, li = lane & 15;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = st.l[rb];
        lt += shfl_xor(lt, 16);
        lt += shfl_xor(lt, 32);
        const float T = st.tmax[rb];
        const float f = (T == kNegInf) ? 0.0f : fexp2(st.m[rb] - T);
        if (kq == 0) {
            srow[0][16 * rb + li] = f;
            srow[1][16 * rb + li] = lt * f;
            srow[2][16 * rb + li] = (T == kNegInf) ? kNegInf : T * kLn2;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 16 * rb + 4 * kq + r;
            const int rr = r0 + rl;
            if (rr >= R) continue;
            const int i = rr / G, hh = rr - i * G;
            const int64_t sidx = slot(i, hh);
            const float f = srow[0][rl] * vdesc;  // V's descale (1 for 16-bit caches)
            float *dst = p.po + sidx * D;
#pragma unroll
            for (int db = 0; db < 8; ++db) dst[16 * db + li] = (st.o[rb][db][r] + st.ol[rb][db][r]) * f;
            if (li == 0) {
                p.pd[sidx] = srow[1][rl];
                p.pm[sidx] = srow[2][rl];
            }
        }
    }
    __builtin_amdgcn_wave_barrier();  // srow is reused by the next piece
}

template <int DT, bool PAGED, int RB, int KF>
__global__ __launch_bounds__(64 * kMtWaves, 1) void map_kernel_mt16(const MapParams p) {
    static_assert(!KF || DT == 1, "float8 caches take bf16 queries");
    constexpr int ROWS = 16 * RB;  // query rows of a wave
    __shared__ __attribute__((aligned(16))) uint8_t ring[kMtWaves][kMtNS][2][kMtTileBytes];
    __shared__ float srow[kMtWaves][3][ROWS];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x, b = blockIdx.y;
    const int G = p.Hq / p.Hkv;
    const int R = p.q_len * G;               // query rows per (request, KV head)
    const int nchunk = (R + ROWS - 1) / ROWS;
    const int u = blockIdx.z * kMtWaves + w;  // (KV head, row chunk) of this wave
    if (u >= p.Hkv * nchunk) return;
    const int g = u / nchunk, r0 = (u - g * nchunk) * ROWS;

    const int L = p.seq_lens[b];
    const int lp = p.leftpad ? p.leftpad[b] : 0;
    const int64_t crow = p.batch_idx ? p.batch_idx[b] : b;
    // split boundaries: multiples of the chunk from the 16-row tile holding the first valid row
    const int t_begin = (lp & ~15) + split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    const int t_lo = max(t_begin, lp);
    // the last query row of this wave sees rows up to L - q_len + its token
    const int t_stop = min(t_end, L - p.q_len + (min(r0 + ROWS, R) - 1) / G + 1);
    const int ntiles = t_stop > t_lo ? (t_stop - t_begin + kMtKeys - 1) / kMtKeys : 0;

    uint4 qb[RB][4];
    int lim[RB];
    mt16_rows<RB>(p, b, g, G, R, r0, L, t_lo, lane, qb, lim);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lim[rb] = min(lim[rb], t_end);
    // float8 caches: the request's descales for this KV head (scalar loads)
    const float kd = KF ? kv_descale(p.k_descale, p, b, g) : 1.0f;
    const float vd = KF ? kv_descale(p.v_descale, p, b, g) : 1.0f;
    // the loads above are done before any DMA is issued: a wait the compiler
    // models keeps it from waiting on them (and so on the DMA) later
    __builtin_amdgcn_s_waitcnt(0);

    const int nskip0 = t_lo - t_begin;
    auto issue = [&](int tile) {
        const int t0 = t_begin + tile * kMtKeys;
        const int slot = tile % kMtNS;
        mt16_issue<PAGED, KF>(p, b, crow, g, t0, tile == 0 ? nskip0 : 0, t_stop - t0 - 1, ring[w][slot][0],
                              ring[w][slot][1], lane);
    };
    Mt16State<RB> st;
    st.reset();
    if (ntiles > 0) issue(0);
    for (int tile = 0; tile < ntiles; ++tile) {
        if (tile + 1 < ntiles) issue(tile + 1);
        // this tile's loads have landed once only the next tile's remain
        if (tile + 1 < ntiles)
            wait_vm<MtDma<KF>::kValue>();
        else
            wait_vm<0>();
        mt16_tile<DT, RB, KF>(ring[w][tile % kMtNS][0], ring[w][tile % kMtNS][1], qb, t_begin + tile * kMtKeys,
                              t_lo, lim, p.scale_log2 * kd, lane, st, srow[w]);
    }
    // state rows (request, token, head) of [B * q_len * Hq, s_total]
    mt16_write<RB>(p, st, srow[w], r0, R, G, lane, vd, [&](int i, int hh) -> int64_t {
        return (((int64_t)b * p.q_len + i) * p.Hq + g * G + hh) * p.s_total + p.s_offset + split;
    });
}

// Balanced split (as map_kernel_mfma_g4_bal, in 32-key tiles): the tiles of all
// requests, in request order, cut into gridDim.x equal ranges; a wave streams
// its range across request boundaries, writing each request piece's states to
// slot (block + request) of rows (token, head) of [q_len * Hq, nslots], and the
// block holding a request's first tile records (first slot, piece count) in
// seg_meta. Q of each request is loaded into registers when its piece starts.
template <int DT, bool PAGED, int RB, int KF>
__global__ __launch_bounds__(64 * kMtWaves, 1) void map_kernel_mt16_bal(const MapParams p) {
    static_assert(!KF || DT == 1, "float8 caches take bf16 queries");
    constexpr int ROWS = 16 * RB;
    __shared__ __attribute__((aligned(16))) uint8_t ring[kMtWaves][kMtNS][2][kMtTileBytes];
    __shared__ float srow[kMtWaves][3][ROWS];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = p.Hq / p.Hkv;
    const int R = p.q_len * G;
    const int nchunk = (R + ROWS - 1) / ROWS;
    const int u = blockIdx.z * kMtWaves + w;
    const bool active = u < p.Hkv * nchunk;
    const int g = active ? u / nchunk : 0, r0 = active ? (u - g * nchunk) * ROWS : 0;
    const int NB = gridDim.x, blk = blockIdx.x;

    // ---- the block's tile range: rows [lp & ~15, L) of each request in 32-key tiles
    const bool one_pass = p.B <= 64;
    auto tiles_of = [&](int j) -> int {
        if (j >= p.B) return 0;
        const int L = p.seq_lens[j], lp = p.leftpad ? p.leftpad[j] : 0;
        return L > lp ? (L - (lp & ~15) + kMtKeys - 1) / kMtKeys : 0;
    };
    const int T0l = tiles_of(lane);
    int NT = 0;
    for (int c = 0; c < p.B; c += 64) NT += wave_sum_int(one_pass ? T0l : tiles_of(c + lane));
    const int NBe = min(NB, NT);
    auto block_of = [&](int x) -> int {
        return x >= NT ? NBe - 1 : (int)((((int64_t)x + 1) * NBe - 1) / NT);
    };
    const bool working = blk < NBe;
    const int start = working ? (int)((int64_t)blk * NT / NBe) : 0;
    const int end = working ? (int)((int64_t)(blk + 1) * NT / NBe) : 0;
    const bool meta_writer = blockIdx.z == 0 && w == 0;
    int b0 = -1, P0 = 0, T0 = 0;
    int carry = 0;
    for (int c = 0; c < p.B; c += 64) {
        const int j = c + lane;
        const int T = one_pass ? T0l : tiles_of(j);
        const int incl = wave_incl_scan(T, lane);
        const int P = carry + incl - T;
        if (meta_writer && j < p.B) {
            const int first = NT > 0 ? block_of(P) : 0;
            if (first == blk) {
                p.seg_meta[2 * j] = first + j;
                p.seg_meta[2 * j + 1] = T > 0 ? block_of(P + T - 1) - first + 1 : 0;
            }
        }
        const uint64_t mask = __builtin_amdgcn_ballot_w64(working && j < p.B && T > 0 && P <= start && start < P + T);
        if (b0 < 0 && mask) {
            const int l = __builtin_ctzll(mask);
            b0 = c + l;
            P0 = __builtin_amdgcn_readlane(P, l);
            T0 = __builtin_amdgcn_readlane(T, l);
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (!working || !active) return;
    __builtin_amdgcn_s_waitcnt(0);

    // ---- stream tiles [start, end): a cursor per side walks the requests
    typedef const __attribute__((address_space(4))) int32_t *ci_t;
    struct Cursor {
        int b, P, T, L, lp;
        int64_t crow;
    };
    auto load = [&](Cursor &c) {
        c.b = __builtin_amdgcn_readfirstlane(c.b);
        c.L = __builtin_amdgcn_readfirstlane(((ci_t)p.seq_lens)[c.b]);
        c.lp = p.leftpad ? __builtin_amdgcn_readfirstlane(((ci_t)p.leftpad)[c.b]) : 0;
        c.crow = p.batch_idx ? __builtin_amdgcn_readfirstlane(((ci_t)p.batch_idx)[c.b]) : c.b;
    };
    auto advance = [&](Cursor &c) {  // to the next request with tiles
        do {
            c.P += c.T;
            c.b += 1;
            load(c);
            c.T = c.L > c.lp ? (c.L - (c.lp & ~15) + kMtKeys - 1) / kMtKeys : 0;
        } while (c.T == 0);
    };
    // uniform by construction; said so, the cursor's loads are scalar
    b0 = __builtin_amdgcn_readfirstlane(b0);
    P0 = __builtin_amdgcn_readfirstlane(P0);
    T0 = __builtin_amdgcn_readfirstlane(T0);
    Cursor prod{b0, P0, T0, 0, 0, 0}, cons{b0, P0, T0, 0, 0, 0};
    load(prod);
    load(cons);
    auto issue = [&](int x) {
        if (x >= prod.P + prod.T) advance(prod);
        const int k = x - prod.P;
        const int t0 = (prod.lp & ~15) + k * kMtKeys;
        const int lo = k == 0 ? prod.lp - (prod.lp & ~15) : 0;
        mt16_issue<PAGED, KF>(p, prod.b, prod.crow, g, t0, lo, prod.L - t0 - 1, ring[w][x % kMtNS][0],
                              ring[w][x % kMtNS][1], lane);
    };
    // float8 caches: the current request's descales for this KV head
    float kd = KF ? kv_descale(p.k_descale, p, cons.b, g) : 1.0f;
    float vd = KF ? kv_descale(p.v_descale, p, cons.b, g) : 1.0f;
    // the states of request b's piece: slot blk + b of rows (token, head)
    auto flush = [&](const Mt16State<RB> &st, int b) {
        mt16_write<RB>(p, st, srow[w], r0, R, G, lane, vd, [&](int i, int hh) -> int64_t {
            return ((int64_t)i * p.Hq + g * G + hh) * p.nslots + blk + b;
        });
    };

    uint4 qb[RB][4];
    int lim[RB];
    mt16_rows<RB>(p, cons.b, g, G, R, r0, cons.L, cons.lp, lane, qb, lim);
    __builtin_amdgcn_s_waitcnt(0);
    Mt16State<RB> st;
    st.reset();
    issue(start);
    for (int x = start; x < end; ++x) {
        if (x >= cons.P + cons.T) {
            flush(st, cons.b);
            st.reset();
            advance(cons);
            mt16_rows<RB>(p, cons.b, g, G, R, r0, cons.L, cons.lp, lane, qb, lim);
            if constexpr (KF == 1) {
                kd = kv_descale(p.k_descale, p, cons.b, g);
                vd = kv_descale(p.v_descale, p, cons.b, g);
            }
            // before the next tile's DMA: this wait (on tile x, needed anyway)
            // tells the compiler the Q loads are done, so it adds no wait of
            // its own in the loop, which would also wait on the DMA ahead
            __builtin_amdgcn_s_waitcnt(0);
        }
        if (x + 1 < end) issue(x + 1);
        if (x + 1 < end)
            wait_vm<MtDma<KF>::kValue>();
        else
            wait_vm<0>();
        const int t0 = (cons.lp & ~15) + (x - cons.P) * kMtKeys;
        mt16_tile<DT, RB, KF>(ring[w][x % kMtNS][0], ring[w][x % kMtNS][1], qb, t0, cons.lp, lim,
                              p.scale_log2 * kd, lane, st, srow[w]);
    }
    flush(st, cons.b);
}

// Row blocks per wave for q_len * G query rows per (request, KV head).
hipError_t launch_map_mt16(const MapParams &p, int S, hipStream_t st) {
    const int G = p.Hq / p.Hkv, R = p.q_len * G;
    const int rb = mt16_row_blocks(R);
    const int nchunk = (R + 16 * rb - 1) / (16 * rb);
    const int units = p.Hkv * nchunk;
    dim3 grid(S, p.B, (units + kMtWaves - 1) / kMtWaves), block(64 * kMtWaves);
    if (p.head_dim != 128 || p.mode != kPlain || (p.kv_fp8 && p.dtype != 1)) return hipErrorInvalidValue;
#define FDEC_MT16(DT, PG, RBV) hipLaunchKernelGGL((map_kernel_mt16<DT, PG, RBV, 0>), grid, block, 0, st, p)
#define FDEC_MT16F8(PG, RBV) hipLaunchKernelGGL((map_kernel_mt16<1, PG, RBV, 1>), grid, block, 0, st, p)
    if (p.kv_fp8) {
        if (rb == 1) {
            if (p.page_table) FDEC_MT16F8(true, 1); else FDEC_MT16F8(false, 1);
        } else {
            if (p.page_table) FDEC_MT16F8(true, 2); else FDEC_MT16F8(false, 2);
        }
    } else if (rb == 1) {
        if (p.dtype == 0) {
            if (p.page_table) FDEC_MT16(0, true, 1); else FDEC_MT16(0, false, 1);
        } else {
            if (p.page_table) FDEC_MT16(1, true, 1); else FDEC_MT16(1, false, 1);
        }
    } else {
        if (p.dtype == 0) {
            if (p.page_table) FDEC_MT16(0, true, 2); else FDEC_MT16(0, false, 2);
        } else {
            if (p.page_table) FDEC_MT16(1, true, 2); else FDEC_MT16(1, false, 2);
        }
    }
#undef FDEC_MT16
#undef FDEC_MT16F8
    return hipGetLastError();
}

hipError_t launch_map_mt16_balanced(const MapParams &p, int nblocks, hipStream_t st) {
    const int G = p.Hq / p.Hkv, R = p.q_len * G;
    const int rb = mt16_row_blocks(R);
    const int nchunk = (R + 16 * rb - 1) / (16 * rb);
    const int units = p.Hkv * nchunk;
    dim3 grid(nblocks, 1, (units + kMtWaves - 1) / kMtWaves), block(64 * kMtWaves);
    if (p.head_dim != 128 || p.mode != kPlain || (p.kv_fp8 && p.dtype != 1)) return hipErrorInvalidValue;
#define FDEC_MT16B(DT, PG, RBV) hipLaunchKernelGGL((map_kernel_mt16_bal<DT, PG, RBV, 0>), grid, block, 0, st, p)
#define FDEC_MT16BF8(PG, RBV) hipLaunchKernelGGL((map_kernel_mt16_bal<1, PG, RBV, 1>), grid, block, 0, st, p)
    if (p.kv_fp8) {
        if (rb == 1) {
            if (p.page_table) FDEC_MT16BF8(true, 1); else FDEC_MT16BF8(false, 1);
        } else {
            if (p.page_table) FDEC_MT16BF8(true, 2); else FDEC_MT16BF8(false, 2);
        }
    } else if (rb == 1) {
        if (p.dtype == 0) {
            if (p.page_table) FDEC_MT16B(0, true, 1); else FDEC_MT16B(0, false, 1);
        } else {
            if (p.page_table) FDEC_MT16B(1, true, 1); else FDEC_MT16B(1, false, 1);
        }
    } else {
        if (p.dtype == 0) {
            if (p.page_table) FDEC_MT16B(0, true, 2); else FDEC_MT16B(0, false, 2);
        } else {
            if (p.page_table) FDEC_MT16B(1, true, 2); else FDEC_MT16B(1, false, 2);
        }
    }
#undef FDEC_MT16B
#undef FDEC_MT16BF8
    return hipGetLastError();
}

}  // namespace fdec
