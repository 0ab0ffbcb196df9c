// Multi-token decode map kernel on 16x16x32 matrix cores (gfx950).
//
// The split-KV map stage (lpnh.cn FlashDecoding explainer §2 stage 1) for q_len
// query tokens per request (speculative decode, vLLM notes spec-decode
// batches) under the causal mask of the pages' calls: query token i of request
// b is its row L_b - q_len + i and sees rows [leftpad, L_b - q_len + i]. The
// q_len * G query rows of one (request, KV head) -- G query heads per KV head --
// form the row blocks of v_mfma_f32_16x16x32_{bf16,f16}, so the contraction is
// dense for any G once q_len * G reaches 16 (the 4x4x4 kernel in
// split_kv_mfma.hip covers short q_len).
//
// One wave per (split, request, KV head, chunk of 32 query rows); a block
// holds kMtWaves such waves, each with a private LDS ring. Per 32-key tile:
//   - K and V rows go global -> LDS by LDS-DMA (no registers), 4 rows per
//     instruction (a page holds a multiple of 16 rows, so 4 rows lie on one
//     page), 16-byte pieces of row r in slot piece ^ (r mod 16);
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
constexpr int kMtTileBytes = kMtKeys * 256;  // 32 rows of 128 16-bit elements
constexpr int kMtNS = 2;                     // ring slots per wave (one tile in flight ahead)
constexpr int kMtDma = 2 * kMtKeys / 4;      // DMA instructions per tile (K and V, 4 rows each)
constexpr float kMtTau = 8.0f;
constexpr float kMtFloor = -1.0e30f;

}  // namespace

template <int DT, bool PAGED, int RB>
__global__ __launch_bounds__(64 * kMtWaves, 1) void map_kernel_mt16(const MapParams p) {
    constexpr int D = 128;
    constexpr int ROWS = 16 * RB;  // query rows of a wave
    __shared__ __attribute__((aligned(16))) uint8_t ring[kMtWaves][kMtNS][2][kMtTileBytes];
    __shared__ float srow[kMtWaves][3][ROWS];

    const int lane = threadIdx.x & 63, kq = lane >> 4, li = lane & 15;
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
    // the last query row of this wave sees rows up to L - q_len + i_last
    const int i_last = min(r0 + ROWS, R) - 1;
    const int t_stop = min(t_end, L - p.q_len + i_last / G + 1);
    const int ntiles = t_stop > t_lo ? (t_stop - t_begin + kMtKeys - 1) / kMtKeys : 0;

    // this lane's query rows (S^T column li of row block rb): limits and Q^T
    int lim[RB];       // keys [t_lo, lim) count for the row
    uint4 qb[RB][4];   // B operand of S^T per (rb, ks)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = r0 + 16 * rb + li;
        const bool ok = r < R;
        const int i = ok ? r / G : 0, hh = ok ? r - (r / G) * G : 0;
        lim[rb] = ok ? min(t_end, L - p.q_len + i + 1) : t_lo;
        const uint16_t *qrow =
            reinterpret_cast<const uint16_t *>(p.q) + (((int64_t)b * p.q_len + i) * p.Hq + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[rb][ks] = ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * kq) : make_uint4(0, 0, 0, 0);
    }
    // the loads above are done before any DMA is issued: a wait the compiler
    // models keeps it from waiting on them (and so on the DMA) later
    __builtin_amdgcn_s_waitcnt(0);

    // DMA of tile `tile` into ring slot tile % kMtNS: 8 groups of 4 rows for K
    // and for V; rows below t_lo and from t_stop on repeat the nearest valid row
    const uint32_t stok = (uint32_t)(p.s_token * 2);
    const int nskip0 = t_lo - t_begin;
    auto issue = [&](int tile) {
        const int t0 = t_begin + tile * kMtKeys;
        const int lo = tile == 0 ? nskip0 : 0, hi = t_stop - t0 - 1;  // valid tile rows [lo, hi]
        const int slot = tile % kMtNS;
#pragma unroll
        for (int gi = 0; gi < kMtKeys / 4; ++gi) {
            const int g0 = 4 * gi;
            const int rs = min(max(g0, lo), hi);  // the group's first source row
            int64_t eoff;
            const int t = t0 + (rs & ~3);  // the 4-row group holding rs: one page
            if constexpr (PAGED) {
                const int pidx = p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
                typedef const __attribute__((address_space(4))) int32_t *cpage_t;
                const int64_t page = ((cpage_t)(p.page_table + (int64_t)b * p.max_pages))[pidx];
                eoff = page * p.s_outer + (int64_t)(t - pidx * p.page_size) * p.s_token + (int64_t)g * p.s_head;
            } else {
                eoff = crow * p.s_outer + (int64_t)t * p.s_token + (int64_t)g * p.s_head;
            }
            const int r = g0 + (lane >> 4);
            const int src = min(max(r, lo), hi) - (rs & ~3);  // 0..3 within the group
            const uint32_t voff = (uint32_t)src * stok + 16u * (uint32_t)((lane & 15) ^ (r & 15));
            dma16(reinterpret_cast<const char *>(p.k) + eoff * 2, voff, lds_addr(ring[w][slot][0]) + 256u * g0);
            dma16(reinterpret_cast<const char *>(p.v) + eoff * 2, voff, lds_addr(ring[w][slot][1]) + 256u * g0);
        }
    };

    float m[RB], tmax[RB], l[RB];
    f32x4_v o[RB][8], ol[RB][8];
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

    const int npro = min(kMtNS - 1, ntiles);
    for (int t = 0; t < npro; ++t) issue(t);
    for (int tile = 0; tile < ntiles; ++tile) {
        if (tile + kMtNS - 1 < ntiles) issue(tile + kMtNS - 1);
        // this tile's loads have landed once only the later tile's remain
        static_assert(kMtNS == 2 && kMtDma <= 63, "one tile in flight ahead");
        if (tile + 1 < ntiles)
            wait_vm<kMtDma>();
        else
            wait_vm<0>();
        const int t0 = t_begin + tile * kMtKeys;
        const uint8_t *K = ring[w][tile % kMtNS][0];
        const uint8_t *V = ring[w][tile % kMtNS][1];

        // ---- S^T = K Q^T: s[kb][rb] holds keys 16kb + 4kq + r of row 16rb + li
        f32x4_v s[2][RB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kr = 16 * kb + li;
                const uint4 a = *reinterpret_cast<const uint4 *>(K + kr * 256 + 16 * ((4 * ks + kq) ^ (kr & 15)));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) s[kb][rb] = Mfma16<DT>::run(a, qb[rb][ks], s[kb][rb]);
            }
        }

        // ---- online softmax per query row (its keys: [t_lo, lim))
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
                    float v = s[kb][rb][r] * p.scale_log2;
                    if (t < t_lo || t >= lim[rb]) v = kNegInf;
                    s[kb][rb][r] = v;
                    x = fmaxf(x, v);
                }
            x = fmaxf(x, shfl_xor(x, 16));
            x = fmaxf(x, shfl_xor(x, 32));
            mx[rb] = x;
            tmax[rb] = fmaxf(tmax[rb], x);
            move |= x > m[rb] + kMtTau;
        }
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            // move the reference; O rows live in lanes by (kq, r), so the
            // per-row factors go through LDS
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float mn = fmaxf(m[rb], mx[rb]);
                const float alpha = fexp2(m[rb] - mn);
                m[rb] = mn;
                l[rb] *= alpha;
                if (kq == 0) srow[w][0][16 * rb + li] = alpha;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float alpha = srow[w][0][16 * rb + 4 * kq + r];
#pragma unroll
                    for (int db = 0; db < 8; ++db) {
                        o[rb][db][r] *= alpha;
                        ol[rb][db][r] *= alpha;
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
                    pv[r] = fexp2(s[kb][rb][r] - m[rb]);
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
            l[rb] += ps;
        }

        // ---- O += P V: B operand of K-slots 8kq .. 8kq + 7 at d = 16db + li from two
        // transpose reads whose lane m (of 16) addresses key row 4kq + m / 4 (+ 16),
        // d 16db + 4 (m % 4) .. + 3
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int ra = 4 * kq + (li >> 2), rb2 = ra + 16;
            const int piece = 2 * db + ((li & 3) >> 1), half = 8 * (li & 1);
            const s16x4_v x0 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(V + ra * 256 + 16 * (piece ^ (ra & 15)) + half));
            const s16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(V + rb2 * 256 + 16 * (piece ^ (rb2 & 15)) + half));
            const uint2 v0 = __builtin_bit_cast(uint2, x0), v1 = __builtin_bit_cast(uint2, x1);
            const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                o[rb][db] = Mfma16<DT>::run(pah[rb], bop, o[rb][db]);
                ol[rb][db] = Mfma16<DT>::run(pal[rb], bop, ol[rb][db]);
            }
        }
    }

    // ---- states against the true maximum: O~ = O 2^(m - T), d = l 2^(m - T)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = l[rb];
        lt += shfl_xor(lt, 16);
        lt += shfl_xor(lt, 32);
        const float T = tmax[rb];
        const float f = (T == kNegInf) ? 0.0f : fexp2(m[rb] - T);
        if (kq == 0) {
            srow[w][0][16 * rb + li] = f;
            srow[w][1][16 * rb + li] = lt * f;
            srow[w][2][16 * rb + li] = (T == kNegInf) ? kNegInf : T * kLn2;
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
            // state row (request, token, head) of [B * q_len * Hq, s_total]
            const int64_t row = ((int64_t)b * p.q_len + i) * p.Hq + g * G + hh;
            const int64_t st = row * p.s_total + p.s_offset + split;
            const float f = srow[w][0][rl];
            float *dst = p.po + st * D;
#pragma unroll
            for (int db = 0; db < 8; ++db) dst[16 * db + li] = (o[rb][db][r] + ol[rb][db][r]) * f;
            if (li == 0) {
                p.pd[st] = srow[w][1][rl];
                p.pm[st] = srow[w][2][rl];
            }
        }
    }
}

// Row blocks per wave for q_len * G query rows per (request, KV head).
int mt16_row_blocks(int rows) { return rows <= 16 ? 1 : 2; }

hipError_t launch_map_mt16(const MapParams &p, int S, hipStream_t st) {
    const int G = p.Hq / p.Hkv, R = p.q_len * G;
    const int rb = mt16_row_blocks(R);
    const int nchunk = (R + 16 * rb - 1) / (16 * rb);
    const int units = p.Hkv * nchunk;
    dim3 grid(S, p.B, (units + kMtWaves - 1) / kMtWaves), block(64 * kMtWaves);
    if (p.head_dim != 128 || p.kv_fp8 || p.mode != kPlain) return hipErrorInvalidValue;
#define FDEC_MT16(DT, PG, RBV) hipLaunchKernelGGL((map_kernel_mt16<DT, PG, RBV>), grid, block, 0, st, p)
    if (rb == 1) {
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
    return hipGetLastError();
}

}  // namespace fdec
