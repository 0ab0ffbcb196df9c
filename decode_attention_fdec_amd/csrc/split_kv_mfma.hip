// Split-KV map kernel on matrix cores for GQA groups of four query heads
// (gfx950). Same contract as map_kernel in split_kv.hip (the FlashDecoding map
// stage: per split the local max m_i, the local sum of exponentials d_i and the
// unnormalised output O~_i -- lpnh.cn explainer §2 stage 1), for G = Hq/Hkv = 4,
// D = 128; K/V in fp16/bf16 or in float8 e4m3fn (bf16 queries); the in-kernel
// append with NeoX rotary on fp16/bf16 caches (map_kernel_mfma_g4_app).
//
// Packing the four query heads of a KV head makes q.K^T a dense contraction for
// the 16-block v_mfma_f32_4x4x4_16b_{bf16,f16} (M = 4 = G, no padding; lpnh §3
// "KV-Reused layout" for GQA). Layout facts used (lane L, block b = L / 4,
// i = L % 4), verified on the GPU:
//   A: lane holds row i of block b's 4x4 A, four K values;
//   B: lane holds column i of block b's B, four K values;
//   D: lane holds column i of block b's result, rows 0..3 in its four registers;
//   cbsz = 4, abid = q: every block uses block q's A.
// And of ds_read_b64_tr_b16 (the LDS transpose read): in each group of 16
// lanes, lane j receives element j % 4 of the 64-bit chunks addressed by lanes
// j/4, 4 + j/4, 8 + j/4, 12 + j/4.
//
// One wave per KV head. Per wave and 16-token tile:
//   - K and V rows go global -> LDS with global_load_lds_dwordx4 (no registers)
//     into a ring of kNbuf tiles per wave, rows XOR-swizzled in 16-byte slots;
//   - S^T = K Q^T with the 16 blocks as 4 token groups x 4 quarters of D:
//     block b = 4 dq + tg takes tokens 4 tg .. 4 tg + 3 over d in
//     [32 dq, 32 dq + 32); two lane swaps add the quarters, after which lane
//     4 tg + j (j = head) holds the scores of tokens 4 tg .. 4 tg + 3 for head
//     j -- exactly the A operand of P.V for those tokens;
//   - online softmax in the log2 domain with a lazily moved reference per head;
//   - O += P V: A = P broadcast from block q (tokens 4q..4q+3), B = V^T from the
//     transpose read of the row-major V tile; lane L accumulates O[head 0..3]
//     at d = L and 64 + L.
// Float8 caches (the pages' FP8 KV cache: e4m3fn values with one fp32 descale
// per (request, KV head) for K and one for V): tiles arrive at half the bytes;
// K is converted to bf16 in registers after its LDS read, V after an 8-bit
// transpose read (ds_read_b64_tr_b8: in each group of 16 lanes, lane j receives
// byte j % 8 of the 8-byte chunks addressed by lanes j/8 + 2k, k = 0..7, also
// verified on the GPU), both by v_cvt_scalef32_pk_bf16_fp8 at scale 1 (every
// e4m3 value is a bf16 value: exact). K's descale multiplies the score scale
// and V's the written state.
#include "cascade_prefix.h"
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_v __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef int i32x2_v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;
typedef __attribute__((address_space(3))) i32x2_v lds_i32x2;

template <int DT> struct Mfma4;
template <> struct Mfma4<0> {
    template <int CBSZ, int ABID>
    static __device__ __forceinline__ f32x4_v run(uint2 a, uint2 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4_v, a), __builtin_bit_cast(f16x4_v, b), c,
                                                  CBSZ, ABID, 0);
    }
};
template <> struct Mfma4<1> {
    template <int CBSZ, int ABID>
    static __device__ __forceinline__ f32x4_v run(uint2 a, uint2 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_v, a), __builtin_bit_cast(s16x4_v, b),
                                                      c, CBSZ, ABID, 0);
    }
};

// Two 16-bit values packed (lo, hi), rounded to nearest even by the hardware
// conversion.
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<0>(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t pack2<1>(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2{(__bf16)a, (__bf16)b});
}

// x summed over lanes L, L ^ 16, L ^ 32, L ^ 48 (the same order in every lane).
__device__ __forceinline__ float sum_quarters(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// KV element formats: KF = 0 for fp16/bf16, KF = 1 for float8 e4m3fn.
template <int KF> struct KvFmt {
    static constexpr int kElem = KF ? 1 : 2;  // bytes per element
    static constexpr int kDma = KF ? 4 : 8;   // DMA instructions per tile (K + V)
};

constexpr int kMT = 16;                 // tokens per tile
constexpr int kMTileBytes = kMT * 256;  // one tile of K (or V) rows of one KV head
#ifndef FDEC_MFMA_NBUF
#define FDEC_MFMA_NBUF 2
#endif
#ifndef FDEC_MFMA_NBUF8
#define FDEC_MFMA_NBUF8 3
#endif
constexpr int kNbuf = FDEC_MFMA_NBUF;   // ring slots per wave: kNbuf - 1 tiles in flight ahead
constexpr int kNbuf8 = FDEC_MFMA_NBUF8; // the same for float8 tiles (half the bytes: a deeper ring)
static_assert(kNbuf >= 2 && kNbuf <= 8 && kNbuf8 >= 2 && kNbuf8 <= 8, "rings of 2..8 tiles");

// One wave's LDS ring: slots of [K tile | V tile], kNbuf of them for 16-bit
// tiles, kNbuf8 for float8 tiles (half the size).
template <int KF> struct Ring {
    static constexpr int kSlots = KF ? kNbuf8 : kNbuf;
    static constexpr int kTileBytes = KF ? kMTileBytes / 2 : kMTileBytes;
    static constexpr int kBytes = kSlots * 2 * kTileBytes;
    static __device__ __forceinline__ uint8_t *k_tile(uint8_t *w, int slot) { return w + slot * 2 * kTileBytes; }
    static __device__ __forceinline__ uint8_t *v_tile(uint8_t *w, int slot) { return k_tile(w, slot) + kTileBytes; }
};
static_assert(kMapMfmaWaves * Ring<0>::kBytes <= 128 * 1024, "16-bit K/V rings fit in LDS");
static_assert(kMapMfmaWaves * (Ring<1>::kBytes + kNbuf8 * 1024) <= 128 * 1024, "float8 K/V rings fit in LDS");
constexpr float kTau = 8.0f;            // the softmax reference moves when a score exceeds it by 2^kTau
constexpr float kFloor = -1.0e30f;      // initial reference (finite: masked scores give p = 0, no NaN)

// Global -> LDS staging of one 16-token tile of one KV head.
// 16-bit elements (256-byte rows): instruction i (0..3) writes rows 4i..4i+3:
// lane l fills slot (l & 15) of row r = 4i + l / 16 with 16-byte piece
// (l & 15) ^ swz(r) of that row; piece c of row r therefore sits in slot
// c ^ swz(r). K rows use swz = r (an S^T read takes one piece of each of the 16
// rows per quarter wave), V rows swz = 4 (r & 3) (a transpose read takes 4
// pieces of 4 consecutive rows per half wave).
// float8 (128-byte rows): instruction i (0..1) writes rows 8i..8i+7, lane l
// slot (l & 7) of row r = 8i + l / 8 with piece (l & 7) ^ swz(r): for K
// swz = (r >> 1) & 7 (the 16 rows of a quarter-wave S^T read cover all 64
// banks), for V swz = 2 ((r >> 1) & 3) (the 8 rows x 2 pieces of a half-wave
// transpose read take 16 distinct (row parity, slot) pairs: all 64 banks).
// kb / vb address the tile's first row; rows below nskip (left padding) and
// past nrows (the end) repeat rows nskip and nrows - 1, valid rows whose scores
// are masked.
template <int KF>
__device__ __forceinline__ void stage_tile(const char *kb, const char *vb, uint32_t kl, uint32_t vl, int nskip,
                                           int nrows, uint32_t stok, int lane) {
    if constexpr (KF == 0) {
        const int srow = lane >> 4, sslot = lane & 15;
#pragma unroll
        for (int i = 0; i < kMT / 4; ++i) {
            const int r = 4 * i + srow;
            const uint32_t row = (uint32_t)min(max(r, nskip), nrows - 1) * stok;
            dma16_kv(kb, row + 16u * (uint32_t)(sslot ^ r), kl + 1024u * i);
            dma16_kv(vb, row + 16u * (uint32_t)(sslot ^ (4 * (r & 3))), vl + 1024u * i);
        }
    } else {
        const int srow = lane >> 3, sslot = lane & 7;
#pragma unroll
        for (int i = 0; i < kMT / 8; ++i) {
            const int r = 8 * i + srow;
            const uint32_t row = (uint32_t)min(max(r, nskip), nrows - 1) * stok;
            dma16_kv(kb, row + 16u * (uint32_t)(sslot ^ ((r >> 1) & 7)), kl + 1024u * i);
            dma16_kv(vb, row + 16u * (uint32_t)(sslot ^ (2 * ((r >> 1) & 3))), vl + 1024u * i);
        }
    }
}

// Byte offset of token t of request b, KV head g (uniform); crow is the
// request's row of a contiguous cache. A tile of a paged cache lies on one page
// (page_size and tile starts are multiples of 16); the page id comes from a
// scalar load.
template <bool PAGED, int KF>
__device__ __forceinline__ int64_t token_offset(const MapParams &p, int b, int64_t crow, int g, int t) {
    constexpr int ES = KvFmt<KF>::kElem;
    if constexpr (PAGED) {
        typedef const __attribute__((address_space(4))) int32_t *cpage_t;
        const cpage_t ptab = (cpage_t)(p.page_table + (int64_t)b * p.max_pages);
        const int pidx = p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
        const int64_t page = ptab[pidx];
        return (page * p.s_outer + (int64_t)(t - pidx * p.page_size) * p.s_token + (int64_t)g * p.s_head) * ES;
    } else {
        return (crow * p.s_outer + (int64_t)t * p.s_token + (int64_t)g * p.s_head) * ES;
    }
}

// Request b's first valid row (left padding) and its row of a contiguous cache,
// by scalar loads.
__device__ __forceinline__ int first_row(const MapParams &p, int b) {
    typedef const __attribute__((address_space(4))) int32_t *ci_t;
    return p.leftpad ? ((ci_t)p.leftpad)[b] : 0;
}
__device__ __forceinline__ int64_t cache_row(const MapParams &p, int b) {
    typedef const __attribute__((address_space(4))) int32_t *ci_t;
    return p.batch_idx ? ((ci_t)p.batch_idx)[b] : b;
}

// LDS addresses of ring slot `slot`: its K tile and V tile.
template <int KF>
__device__ __forceinline__ void slot_dma_addrs(uint8_t *wl, int slot, uint32_t &kl, uint32_t &vl) {
    kl = lds_addr(Ring<KF>::k_tile(wl, slot));
    vl = lds_addr(Ring<KF>::v_tile(wl, slot));
}

// Q of the four query heads of KV head g of query row qr (1 KB) to LDS, with
// the same DMA path, so that every vector load the waits count is a DMA load.
// qr = b * q_len + token (b for a single query).
__device__ __forceinline__ void stage_q(const MapParams &p, int qr, int g, uint8_t *qslot, int lane) {
    dma16(reinterpret_cast<const char *>(p.q) + ((int64_t)qr * p.Hq + 4 * g) * 128 * 2, (uint32_t)lane * 16u,
          lds_addr(qslot));
}

// Q^T as the B operand of S^T: K-step k of quarter dq = d 32 dq + 4k .. +3 of
// head lane & 3.
__device__ __forceinline__ void read_q(const uint8_t *qslot, int lane, uint2 qb[8]) {
    const int hme = lane & 3, dq = lane >> 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 u = *reinterpret_cast<const uint4 *>(qslot + hme * 256 + dq * 64 + 16 * c);
        qb[2 * c] = make_uint2(u.x, u.y);
        qb[2 * c + 1] = make_uint2(u.z, u.w);
    }
}

// The running softmax of one wave (four query heads; head lane & 3 in the S^T
// layout): reference m, true maximum t, sum l, and O as hi / lo accumulators
// (P enters P V as hi + lo, two 16-bit parts whose sum carries about 16
// significant bits, so O is accumulated from P at close to fp32 accuracy).
struct MfmaSoftmax {
    float m, t, l;
    f32x4_v o[2], ol[2];
    __device__ __forceinline__ void reset() {
        m = kFloor;
        t = kNegInf;
        l = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            o[h] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
            ol[h] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
};

// One tile: S^T = K Q^T, online softmax, O += P V, for QL query tokens of the
// same request (speculative decode; QL = 1 is the single query). Tile tokens
// [nskip, nvalid[j]) count for query token j (nskip < nvalid[j] for at least
// the last token); the rest are masked. The K pieces, their float8 conversion
// and the V^T reads are shared by the QL tokens. kl / vl: the K and V tiles in
// LDS.
template <int DT, int KF, int QL, bool QLO = false>
__device__ __forceinline__ void mfma_tile(const uint8_t *kl, const uint8_t *vl, const uint2 (&qb)[QL][8], int nskip,
                                          const int (&nvalid)[QL], float scale_log2, int lane, MfmaSoftmax (&st)[QL],
                                          const uint2 (*qlo)[8] = nullptr) {
    using E = Elem<DT>;
    const int dq = lane >> 4;
    const int rk = lane & 15;  // S^T reads: token L & 15, pieces 4 dq .. 4 dq + 3
    // transpose reads: lane L = 16 gq + 4 k + a takes token 4q + k, d = 64h + 16 gq + 4a
    const int tk = (lane & 15) >> 2, ta = lane & 3, tg = lane >> 4;

    // ---- S^T = K Q^T: this lane's quarter of D, 4 pieces of 8 d-values
    f32x4_v s[QL], s1[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
        s[j] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
        s1[j] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if constexpr (KF == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 kr = *reinterpret_cast<const uint4 *>(kl + rk * 256 + 16 * ((4 * dq + c) ^ rk));
#pragma unroll
            for (int j = 0; j < QL; ++j) {
                s[j] = Mfma4<DT>::template run<0, 0>(make_uint2(kr.x, kr.y), qb[j][2 * c], s[j]);
                s1[j] = Mfma4<DT>::template run<0, 0>(make_uint2(kr.z, kr.w), qb[j][2 * c + 1], s1[j]);
                if constexpr (QLO) {  // q = hi + lo: the second 16-bit part of an fp32 query
                    s[j] = Mfma4<DT>::template run<0, 0>(make_uint2(kr.x, kr.y), qlo[j][2 * c], s[j]);
                    s1[j] = Mfma4<DT>::template run<0, 0>(make_uint2(kr.z, kr.w), qlo[j][2 * c + 1], s1[j]);
                }
            }
        }
    } else {
        // float8 piece 2 dq + e holds d 32 dq + 16 e .. + 15: K-steps 4e .. 4e + 3
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint4 k8 = *reinterpret_cast<const uint4 *>(kl + rk * 128 + 16 * ((2 * dq + e) ^ ((rk >> 1) & 7)));
            const uint2 k0 = fp8x4_to_bf16(k8.x), k1 = fp8x4_to_bf16(k8.y);
            const uint2 k2 = fp8x4_to_bf16(k8.z), k3 = fp8x4_to_bf16(k8.w);
#pragma unroll
            for (int j = 0; j < QL; ++j) {
                s[j] = Mfma4<DT>::template run<0, 0>(k0, qb[j][4 * e], s[j]);
                s1[j] = Mfma4<DT>::template run<0, 0>(k1, qb[j][4 * e + 1], s1[j]);
                s[j] = Mfma4<DT>::template run<0, 0>(k2, qb[j][4 * e + 2], s[j]);
                s1[j] = Mfma4<DT>::template run<0, 0>(k3, qb[j][4 * e + 3], s1[j]);
                if constexpr (QLO) {
                    s[j] = Mfma4<DT>::template run<0, 0>(k0, qlo[j][4 * e], s[j]);
                    s1[j] = Mfma4<DT>::template run<0, 0>(k1, qlo[j][4 * e + 1], s1[j]);
                    s[j] = Mfma4<DT>::template run<0, 0>(k2, qlo[j][4 * e + 2], s[j]);
                    s1[j] = Mfma4<DT>::template run<0, 0>(k3, qlo[j][4 * e + 3], s1[j]);
                }
            }
        }
    }
    // float8 V^T for P V: lane L gets tokens 8c .. 8c + 7 at d = 64h + L from the
    // 8-bit transpose read whose lane m (of 16) addresses row 8c + m / 2, bytes
    // 64h + 16 (L / 16) + 8 (m & 1) .. + 7; its first four bytes are the B operand
    // of token group 2c, the last four that of group 2c + 1
    uint2 vb[2][2][2];  // [c][h][group within c]
    if constexpr (KF == 1) {
        const int m = lane & 15, gq = lane >> 4;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = 8 * c + (m >> 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int piece = 4 * h + gq;
                lds_i32x2 *src = (lds_i32x2 *)(vl + r * 128 + 16 * (piece ^ (2 * ((r >> 1) & 3))) + 8 * (m & 1));
                const i32x2_v w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(src);
                vb[c][h][0] = fp8x4_to_bf16((uint32_t)w[0]);
                vb[c][h][1] = fp8x4_to_bf16((uint32_t)w[1]);
            }
        }
    }

    // ---- softmax for head lane & 3, tokens 4 tg .. 4 tg + 3 of this tile
    // (lanes 0..15 carry the tile; the others hold copies and stay masked)
    uint2 pa[QL], pb[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
        float sv[4], mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = sum_quarters(s[j][r] + s1[j][r]);
            const int tok = 4 * ((lane >> 2) & 3) + r;
            sv[r] = (tok >= nskip && tok < nvalid[j] && lane < 16) ? x * scale_log2 : kNegInf;
            mx = fmax_nc(mx, sv[r]);
        }
        MfmaSoftmax &t = st[j];
        t.t = fmax_nc(t.t, mx);
        if (__builtin_amdgcn_ballot_w64(mx > t.m + kTau) != 0) {
            // move the reference of every head to its running maximum
            float hm = mx;
            hm = fmax_nc(hm, shfl_xor(hm, 4));
            hm = fmax_nc(hm, shfl_xor(hm, 8));
            hm = fmax_nc(hm, shfl_xor(hm, 16));
            hm = fmax_nc(hm, shfl_xor(hm, 32));
            const float mn = fmax_nc(t.m, hm);
            const float alpha = fexp2(t.m - mn);
            t.m = mn;
            t.l *= alpha;
            f32x4_v al;
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = readlane(alpha, i);  // lanes 0..3 carry heads 0..3
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                t.o[h] *= al;
                t.ol[h] *= al;
            }
        }
        uint32_t ph[2], pl[2];
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
            const float p0 = fexp2(sv[r] - t.m), p1 = fexp2(sv[r + 1] - t.m);
            t.l += p0 + p1;
            const uint32_t h = pack2<DT>(p0, p1);
            ph[r / 2] = h;
            pl[r / 2] = pack2<DT>(p0 - E::lo(h), p1 - E::hi(h));
        }
        pa[j] = make_uint2(ph[0], ph[1]);
        pb[j] = make_uint2(pl[0], pl[1]);
    }

    // ---- O += P V over the tile's 4 groups of 4 tokens
#define FDEC_PV_STEP(Q)                                                                                       \
    {                                                                                                         \
        const int row = 4 * (Q) + tk;                                                                         \
        _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                       \
            uint2 vt;                                                                                         \
            if constexpr (KF == 1) {                                                                          \
                vt = vb[(Q) >> 1][h][(Q) & 1];                                                                \
            } else {                                                                                          \
                const int piece = 8 * h + 2 * tg + (ta >> 1);                                                 \
                lds_s16x4 *src = (lds_s16x4 *)(vl + row * 256 + 16 * (piece ^ (4 * (row & 3))) + 8 * (ta & 1)); \
                vt = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(src));                 \
            }                                                                                                 \
            _Pragma("unroll") for (int j = 0; j < QL; ++j) {                                                  \
                st[j].o[h] = Mfma4<DT>::template run<4, (Q)>(pa[j], vt, st[j].o[h]);                          \
                st[j].ol[h] = Mfma4<DT>::template run<4, (Q)>(pb[j], vt, st[j].ol[h]);                        \
            }                                                                                                 \
        }                                                                                                     \
    }
    FDEC_PV_STEP(0)
    FDEC_PV_STEP(1)
    FDEC_PV_STEP(2)
    FDEC_PV_STEP(3)
#undef FDEC_PV_STEP
}

// The wave's state per head against the true maximum T: O~ = 2^(m - T) O,
// d = 2^(m - T) l, m = T ln 2 (an empty state is (0, -inf, 0)); head i's goes to
// po0 + i hs D, pm0 + i hs, pd0 + i hs.
__device__ __forceinline__ void write_state(const MfmaSoftmax &st, int lane, float *po0, float *pm0, float *pd0,
                                            int64_t hs, float vscale = 1.0f) {
    constexpr int D = 128;
    const float lt = sum_mod4(st.l), tt = max_mod4(st.t);
    const float f_own = (tt == kNegInf) ? 0.0f : fexp2(st.m - tt);
    f32x4_v fs;
#pragma unroll
    for (int i = 0; i < 4; ++i) fs[i] = readlane(f_own, i) * vscale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float *dst = po0 + i * hs * D;
        dst[lane] = (st.o[0][i] + st.ol[0][i]) * fs[i];
        dst[64 + lane] = (st.o[1][i] + st.ol[1][i]) * fs[i];
    }
    if (lane < 4) {
        pm0[lane * hs] = (tt == kNegInf) ? kNegInf : tt * kLn2;
        pd0[lane * hs] = lt * f_own;  // the weights are unscaled: V's descale is on O~ only
    }
}

// One wave's pass over tokens [t_lo, t_end) of request b for KV head g (its
// four query heads; with HG, its eight query heads as QL = 2 groups of four,
// each group taking the place of a query token with no causal limit), in 16-token tiles from t_begin (a multiple of 16, <= t_lo:
// tiles of a paged cache then stay on one page), for nq <= QL query tokens
// ti0 .. ti0 + nq - 1 of the request: token i sees rows up to
// L - q_len + i (causal), i.e. its part of the segment ends at
// min(t_end, L - q_len + i + 1). Token j's state goes to po0[j] / pm0[j] /
// pd0[j] (+ i hs per head). wl / qslot are the wave's LDS: its ring (Ring<KF>)
// and QL KB of Q.
template <int DT, bool PAGED, int KF, int QL, bool HG = false>
__device__ __forceinline__ void mfma_segment(const MapParams &p, uint8_t *wl, uint8_t *qslot, int b, int g, int lane,
                                             int t_begin, int t_lo, int t_end, int L, int ti0, int nq,
                                             float *const (&po0)[QL], float *const (&pm0)[QL],
                                             float *const (&pd0)[QL], int64_t hs) {
    int tend[QL];  // each token's end within this segment (t_begin: nothing)
#pragma unroll
    for (int j = 0; j < QL; ++j) tend[j] = j < nq ? min(t_end, L - p.q_len + ti0 + j + 1) : t_begin;
    const int t_stop = min(t_end, L - p.q_len + ti0 + nq);  // past the group's last token's last row
    const int ntiles = t_stop > t_lo ? (t_stop - t_begin + kMT - 1) / kMT : 0;
    const int nskip0 = t_lo - t_begin;  // left-padding rows of the first tile
    const uint32_t stok = (uint32_t)(p.s_token * KvFmt<KF>::kElem);
    constexpr int NS = Ring<KF>::kSlots;
    auto stage = [&](int tile, int64_t off) {
        uint32_t kl, vl;
        slot_dma_addrs<KF>(wl, tile % NS, kl, vl);
        stage_tile<KF>(p.k + off, p.v + off, kl, vl, tile == 0 ? nskip0 : 0, t_stop - (t_begin + tile * kMT), stok,
                       lane);
    };
    const int64_t crow = PAGED ? 0 : cache_row(p, b);
    auto tile_offset = [&](int tile) { return token_offset<PAGED, KF>(p, b, crow, g, t_begin + tile * kMT); };
    const float kd = KF ? kv_descale(p.k_descale, p, b, g) : 1.0f;
    const float vd = KF ? kv_descale(p.v_descale, p, b, g) : 1.0f;

    MfmaSoftmax st[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
        st[j].reset();
        if (j < nq) {
            if constexpr (HG)  // group j of 4 query heads of a G = 8 KV head: heads 8 g + 4 j ..
                stage_q(p, b, 2 * g + j, qslot + 1024 * j, lane);
            else
                stage_q(p, b * p.q_len + ti0 + j, g, qslot + 1024 * j, lane);
        }
    }
    // prologue: the first NS - 1 tiles
    const int npro = min(NS - 1, ntiles);
    for (int t = 0; t < npro; ++t) stage(t, tile_offset(t));
    int64_t noff = (NS - 1 < ntiles) ? tile_offset(NS - 1) : 0;  // next tile to stage
    wait_vm_n<KvFmt<KF>::kDma>(npro);  // Q has landed
    uint2 qb[QL][8];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
        if (j < nq) {
            read_q(qslot + 1024 * j, lane, qb[j]);
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) qb[j][c] = make_uint2(0u, 0u);
        }
    }

    for (int tile = 0; tile < ntiles; ++tile) {
        const int ahead = tile + NS - 1;
        if (ahead < ntiles) {
            stage(ahead, noff);
            if (ahead + 1 < ntiles) noff = tile_offset(ahead + 1);
        }
        // this tile's loads have landed once only the later tiles' remain
        wait_vm_n<KvFmt<KF>::kDma>(min(NS - 1, ntiles - 1 - tile));
        const int slot = tile % NS;
        const int t0 = t_begin + tile * kMT;
        int nv[QL];
#pragma unroll
        for (int j = 0; j < QL; ++j) nv[j] = tend[j] - t0;
        mfma_tile<DT, KF, QL>(Ring<KF>::k_tile(wl, slot), Ring<KF>::v_tile(wl, slot), qb, tile == 0 ? nskip0 : 0, nv,
                              p.scale_log2 * kd, lane, st);
    }
#pragma unroll
    for (int j = 0; j < QL; ++j)
        if (j < nq) write_state(st[j], lane, po0[j], pm0[j], pd0[j], hs, vd);
}

template <int DT, bool PAGED, int KF, int QL>
__global__ __launch_bounds__(64 * kMapMfmaWaves, 1) void map_kernel_mfma_g4(const MapParams p) {
    constexpr int D = 128, G = 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMapMfmaWaves][Ring<KF>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kMapMfmaWaves][QL][G * D * 2];
    __shared__ int sm_flag;

    // grid (split, request x token group, KV-head group); q_groups token groups of QL
    const int split = blockIdx.x;
    const int b = blockIdx.y / p.q_groups, tgrp = blockIdx.y - b * p.q_groups;
    const int ti0 = tgrp * QL, nq = min(QL, p.q_len - ti0);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.z * p.heads_per_block + wv;
    const int hq0 = g * G;
    const int L = p.seq_lens[b];
    // splits start at the 16-row tile holding the first valid row
    const int lp = first_row(p, b);
    const int t_begin = (lp & ~(kMT - 1)) + split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    float *po0[QL], *pm0[QL], *pd0[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
        // state rows (request, token, head) of [B * q_len * Hq, s_total]
        const int64_t st0 = (((int64_t)b * p.q_len + ti0 + min(j, nq - 1)) * p.Hq + hq0) * p.s_total + p.s_offset +
                            split;
        po0[j] = p.po + st0 * D;
        pm0[j] = p.pm + st0;
        pd0[j] = p.pd + st0;
    }
    mfma_segment<DT, PAGED, KF, QL>(p, lds[wv], &qlds[wv][0][0], b, g, lane, t_begin, max(t_begin, lp), t_end, L, ti0,
                                    nq, po0, pm0, pd0, p.s_total);

    if (QL > 1 || p.counters == nullptr) return;  // single-kernel merge: single-query decode only

    // ---- single-kernel merge (as in map_kernel)
    __syncthreads();
    if (threadIdx.x == 0) {
        int *cnt = p.counters + (int64_t)b * gridDim.z + blockIdx.z;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (int)gridDim.x - 1);
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_flag = last;
    }
    __syncthreads();
    if (!sm_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        merge_states_wave<D>(p.po + bh * p.s_total * D, p.pm + bh * p.s_total, p.pd + bh * p.s_total,
                             p.s_total, p.out + bh * D, p.lse ? p.lse + bh : nullptr, lane);
    }
}

// GQA groups of eight query heads (single query): one wave per KV head runs
// its eight heads as two groups of four through the same tiles (the
// multi-token path of mfma_tile with QL = 2, the groups in place of query
// tokens, no causal limit), so every staged K/V tile and every K piece read
// from LDS serves eight query heads.
template <int DT, bool PAGED, int KF>
__global__ __launch_bounds__(64 * kMapMfmaWaves, 1) void map_kernel_mfma_g8(const MapParams p) {
    constexpr int D = 128, G = 8;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMapMfmaWaves][Ring<KF>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kMapMfmaWaves][2][4 * D * 2];
    __shared__ int sm_flag;

    const int split = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.z * p.heads_per_block + wv;
    const int hq0 = g * G;
    const int L = p.seq_lens[b];
    const int lp = first_row(p, b);
    const int t_begin = (lp & ~(kMT - 1)) + split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    float *po0[2], *pm0[2], *pd0[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t st0 = ((int64_t)b * p.Hq + hq0 + 4 * j) * p.s_total + p.s_offset + split;
        po0[j] = p.po + st0 * D;
        pm0[j] = p.pm + st0;
        pd0[j] = p.pd + st0;
    }
    mfma_segment<DT, PAGED, KF, 2, true>(p, lds[wv], &qlds[wv][0][0], b, g, lane, t_begin, max(t_begin, lp), t_end,
                                         L, 0, 2, po0, pm0, pd0, p.s_total);

    if (p.counters == nullptr) return;

    // ---- single-kernel merge (as in map_kernel_mfma_g4)
    __syncthreads();
    if (threadIdx.x == 0) {
        int *cnt = p.counters + (int64_t)b * gridDim.z + blockIdx.z;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (int)gridDim.x - 1);
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_flag = last;
    }
    __syncthreads();
    if (!sm_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        merge_states_wave<D>(p.po + bh * p.s_total * D, p.pm + bh * p.s_total, p.pd + bh * p.s_total,
                             p.s_total, p.out + bh * D, p.lse ? p.lse + bh : nullptr, lane);
    }
}

// Decode with an in-kernel append (flash-attn "Inference Cookbook / 推理优化"
// page §3.3-3.4: the new token's k / v are written at row cache_seqlens[b] and
// attended to, with GPT-NeoX rotary of q and k_new at the new token's position
// when tables are given),
// uniform splits, single query, fp16 / bf16 caches, G = 4 or 8 (NG = 1 or 2
// groups of four query heads through the same tiles). Every block rotates q in
// fp32 (in LDS) and feeds it to S^T = K Q^T as two 16-bit parts, hi + lo (the
// low part is q - hi rounded again: about 16 significant bits together); the
// block owning row cache_seqlens[b] rounds the rotated k_new once to the cache
// type, writes it and v_new into the cache, and waits for those stores before
// its first DMA, which may read the row back.
template <int DT, bool PAGED, int NG, int KF>
__global__ __launch_bounds__(64 * kMapMfmaWaves, 1) void map_kernel_mfma_g4_app(const MapParams p) {
    constexpr int D = 128, G = 4 * NG;  // NG groups of four query heads per KV head
    static_assert(!KF || DT == 1, "float8 caches take bf16 queries and new rows");
    constexpr int NS = Ring<KF>::kSlots;
    using E = Elem<DT>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMapMfmaWaves][Ring<KF>::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kMapMfmaWaves][2][G * D * 2];  // hi, lo
    __shared__ float fl[kMapMfmaWaves][(G + 1) * D];                                      // q, then k_new (fp32)
    __shared__ int sm_flag;

    const int split = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.z * p.heads_per_block + wv;
    const int hq0 = g * G;
    const int c_app = p.seq_lens[b];
    const int L = c_app + 1;
    const int lp = first_row(p, b);
    const int t_begin = (lp & ~(kMT - 1)) + split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    const bool owner = t_begin <= c_app && c_app < t_begin + p.chunk;
    const int64_t crow = PAGED ? 0 : cache_row(p, b);

    // ---- q (and k_new in the owner) in fp32, rotated
    float *qs = fl[wv];
    float *ks = qs + G * D;
    const uint16_t *qsrc = reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hq + hq0) * D;
    const uint16_t *ksrc = reinterpret_cast<const uint16_t *>(p.k_new) + ((int64_t)b * p.Hkv + g) * D;
    for (int i = lane; i < G * D; i += 64) qs[i] = E::lo((uint32_t)qsrc[i]);
    if (owner)
        for (int i = lane; i < D; i += 64) ks[i] = E::lo((uint32_t)ksrc[i]);
    __builtin_amdgcn_wave_barrier();
    if (p.mode == kAppendRope) {
        const int half = p.rotary_dim >> 1;
        // the new row's position among the valid rows
        const float *cs = p.rope_cos + (int64_t)(c_app - lp) * half;
        const float *sn = p.rope_sin + (int64_t)(c_app - lp) * half;
        const int nvec = owner ? G + 1 : G;
        for (int i = lane; i < nvec * half; i += 64) {
            const int h = i / half, j = i - h * half;
            float *x = qs + h * D;
            const float c = cs[j], sv = sn[j];
            const float x0 = x[j], x1 = x[j + half];
            x[j] = x0 * c - x1 * sv;
            x[j + half] = x0 * sv + x1 * c;
        }
        __builtin_amdgcn_wave_barrier();
    }
    // q as hi + lo in the layout read_q expects ([head][d], 16-bit)
    uint16_t *qh = reinterpret_cast<uint16_t *>(qlds[wv][0]);
    uint16_t *ql = reinterpret_cast<uint16_t *>(qlds[wv][1]);
    for (int i = lane; i < G * D; i += 64) {
        const float x = qs[i];
        const uint16_t h = E::from_float(x);
        qh[i] = h;
        ql[i] = E::from_float(x - E::lo((uint32_t)h));
    }
    if (owner) {
        const int64_t off = token_offset<PAGED, KF>(p, b, crow, g, c_app);
        uint16_t *kd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.k) + off);
        uint16_t *vd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.v) + off);
        const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(p.v_new) + ((int64_t)b * p.Hkv + g) * D;
        const bool rotated = p.mode == kAppendRope;
        if constexpr (KF == 1) {
            // float8: the codes of value / descale (the k value rotated in fp32, or
            // k_new's bf16 value), as the vector kernel stores them
            uint8_t *k8 = reinterpret_cast<uint8_t *>(const_cast<char *>(p.k)) + off;
            uint8_t *v8 = reinterpret_cast<uint8_t *>(const_cast<char *>(p.v)) + off;
            const float kds = kv_descale(p.k_descale, p, b, g), vds = kv_descale(p.v_descale, p, b, g);
            for (int i = lane; i < D; i += 64) {
                const float kx = rotated ? ks[i] : E::lo((uint32_t)ksrc[i]);
                k8[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(kx, kds));
                v8[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(E::lo((uint32_t)vsrc[i]), vds));
            }
        } else {
            for (int i = lane; i < D; i += 64) {
                kd[i] = rotated ? E::from_float(ks[i]) : ksrc[i];  // unrotated: the bits of k_new
                vd[i] = vsrc[i];
            }
        }
    }
    // every load and store above is done (the owner's row is in L2 before its
    // DMA reads it back; no earlier load of this kernel cached the row), and a
    // wait the compiler models keeps it from waiting on the DMA loads below
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    uint2 qb[NG][8], qlo[NG][8];
#pragma unroll
    for (int j = 0; j < NG; ++j) {  // group j: query heads 4 j .. 4 j + 3 of the KV head
        read_q(qlds[wv][0] + 1024 * j, lane, qb[j]);
        read_q(qlds[wv][1] + 1024 * j, lane, qlo[j]);
    }

    // ---- stream the split's tiles (as mfma_segment, one query token)
    const int t_lo = max(t_begin, lp);
    const int ntiles = t_end > t_lo ? (t_end - t_begin + kMT - 1) / kMT : 0;
    const int nskip0 = t_lo - t_begin;
    const uint32_t stok = (uint32_t)(p.s_token * KvFmt<KF>::kElem);
    // float8 caches: the request's descales for this KV head
    const float kd8 = KF ? kv_descale(p.k_descale, p, b, g) : 1.0f;
    const float vd8 = KF ? kv_descale(p.v_descale, p, b, g) : 1.0f;
    auto tile_offset = [&](int tile) { return token_offset<PAGED, KF>(p, b, crow, g, t_begin + tile * kMT); };
    auto stage = [&](int tile, int64_t off) {
        uint32_t kl, vl;
        slot_dma_addrs<KF>(lds[wv], tile % NS, kl, vl);
        stage_tile<KF>(p.k + off, p.v + off, kl, vl, tile == 0 ? nskip0 : 0, t_end - (t_begin + tile * kMT), stok,
                       lane);
    };
    MfmaSoftmax st[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) st[j].reset();
    const int npro = min(NS - 1, ntiles);
    for (int t = 0; t < npro; ++t) stage(t, tile_offset(t));
    int64_t noff = (NS - 1 < ntiles) ? tile_offset(NS - 1) : 0;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int ahead = tile + NS - 1;
        if (ahead < ntiles) {
            stage(ahead, noff);
            if (ahead + 1 < ntiles) noff = tile_offset(ahead + 1);
        }
        wait_vm_n<KvFmt<KF>::kDma>(min(NS - 1, ntiles - 1 - tile));
        const int slot = tile % NS;
        int nv[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) nv[j] = t_end - (t_begin + tile * kMT);
        mfma_tile<DT, KF, NG, true>(Ring<KF>::k_tile(lds[wv], slot), Ring<KF>::v_tile(lds[wv], slot), qb,
                                    tile == 0 ? nskip0 : 0, nv, p.scale_log2 * kd8, lane, st, qlo);
    }
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int64_t st0 = ((int64_t)b * p.Hq + hq0 + 4 * j) * p.s_total + p.s_offset + split;
        write_state(st[j], lane, p.po + st0 * D, p.pm + st0, p.pd + st0, p.s_total, vd8);
    }

    if (p.counters == nullptr) return;

    // ---- single-kernel merge (as in map_kernel_mfma_g4)
    __syncthreads();
    if (threadIdx.x == 0) {
        int *cnt = p.counters + (int64_t)b * gridDim.z + blockIdx.z;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (int)gridDim.x - 1);
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_flag = last;
    }
    __syncthreads();
    if (!sm_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        merge_states_wave<D>(p.po + bh * p.s_total * D, p.pm + bh * p.s_total, p.pd + bh * p.s_total,
                             p.s_total, p.out + bh * D, p.lse ? p.lse + bh : nullptr, lane);
    }
}

// Balanced split: the 16-token tiles of all requests, in request order, are
// cut into gridDim.x equal ranges, one per block (per group of KV heads). A
// block streams its range as one sequence of tiles across request boundaries
// (the DMA ring never drains between requests): at each boundary it writes
// the finished piece's state to slot (block + request) of [Hq, nslots]
// (nslots = gridDim.x + B; the pieces of one request take consecutive slots)
// and resets its softmax. Q of each request is staged by DMA ahead of the
// request's first tile into one of the ring's Q slots. The block holding a
// request's first tile records (first slot, piece count) in seg_meta[2b..].
// With fewer tiles than blocks, only the first (tiles) blocks take work, so
// every working block has at least one tile and no slot of a request is left
// unwritten. Every wave scans seq_lens itself (no block barrier).
// The LDS of one balanced-split block: each wave's K/V ring, and the Q of the
// pieces in flight (at most one per ring slot), QL query tokens each (with HG:
// the two groups of four query heads of a G = 8 KV head, one query).
template <int KF, int QL> struct BalLds {
    __attribute__((aligned(16))) uint8_t ring[kMapMfmaWaves][Ring<KF>::kBytes];
    __attribute__((aligned(16))) uint8_t q[kMapMfmaWaves][Ring<KF>::kSlots][QL][4 * 128 * 2];
};

// Block blk of NB of the balanced split, grid row by (groups of QL query
// tokens) and group bz of KV heads.
template <int DT, bool PAGED, int KF, int QL, bool HG = false>
__device__ __forceinline__ void map_g4_bal_body(const MapParams &p, int blk, int NB, int by, int bz,
                                                BalLds<KF, QL> &sm) {
    constexpr int D = 128, G = 4;
    constexpr int NS = Ring<KF>::kSlots;
    static_assert(!HG || QL == 2, "groups of eight query heads run as two groups of four");
    auto &lds = sm.ring;
    auto &qlds = sm.q;
    // query tokens ti0 .. ti0 + nq - 1 of every request (grid y: groups of QL)
    const int ti0 = HG ? 0 : by * QL, nq = HG ? 2 : min(QL, p.q_len - ti0);

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = bz * p.heads_per_block + wv;
    const int hq0 = g * (HG ? 2 * G : G);
    const uint32_t stok = (uint32_t)(p.s_token * KvFmt<KF>::kElem);

    // ---- the block's tile range and its first request
    // With B <= 64 one scan does it all: lane j holds request j's length, first
    // row and tile count, the total is the scan's last lane, and the first
    // request's length and first row come from registers (no second load
    // before the first DMA).
    const bool one_pass = p.B <= 64;
    // rows [leftpad, seq_len) of a request, counted from the 16-row tile holding
    // the first (0 when there are none)
    auto valid_of = [](int L, int lp) -> int { return L > lp ? L - (lp & ~(kMT - 1)) : 0; };
    auto valid_rows = [&](int j) -> int {
        if (j >= p.B) return 0;
        return valid_of(p.seq_lens[j], p.leftpad ? p.leftpad[j] : 0);
    };
    int NT = 0;           // tiles of all requests
    int Lv = 0, lpv = 0;  // one pass: request `lane`'s length and first row
    int T1 = 0, incl1 = 0;  // one pass: its tiles and their inclusive scan
    if (one_pass) {
        if (lane < p.B) {
            Lv = p.seq_lens[lane];
            lpv = p.leftpad ? p.leftpad[lane] : 0;
        }
        T1 = (valid_of(Lv, lpv) + kMT - 1) / kMT;
        incl1 = wave_incl_scan(T1, lane);
        NT = __builtin_amdgcn_readlane(incl1, 63);
    } else {
        for (int c = 0; c < p.B; c += 64) NT += wave_sum_int((valid_rows(c + lane) + kMT - 1) / kMT);
    }
    const int NBe = min(NB, NT);  // working blocks
    // block holding tile x (x < NT), the last working block past the end
    auto block_of = [&](int x) -> int {
        return x >= NT ? NBe - 1 : (int)((((int64_t)x + 1) * NBe - 1) / NT);
    };
    const bool working = blk < NBe;
    const int start = working ? (int)((int64_t)blk * NT / NBe) : 0;
    const int end = working ? (int)((int64_t)(blk + 1) * NT / NBe) : 0;
    const bool meta_writer = bz == 0 && by == 0 && wv == 0;
    // (first slot, piece count) of request j, whose tiles are [P, P + T), when
    // its first tile lies in this block's range
    auto write_meta = [&](int j, int P, int T) {
        if (meta_writer && j < p.B) {
            const int first = NT > 0 ? block_of(P) : 0;
            if (first == blk) {
                p.seg_meta[2 * j] = first + j;
                p.seg_meta[2 * j + 1] = T > 0 ? block_of(P + T - 1) - first + 1 : 0;
            }
        }
    };

    int b0 = -1, P0 = 0, T0 = 0;  // first request of the range and its first tile
    int Lb0 = 0, lp0 = 0;         // its end row and first row
    if (one_pass) {
        const int P = incl1 - T1;
        const uint64_t mask =
            __builtin_amdgcn_ballot_w64(working && lane < p.B && T1 > 0 && P <= start && start < P + T1);
        if (mask) {
            const int l = __builtin_ctzll(mask);
            b0 = l;
            P0 = __builtin_amdgcn_readlane(P, l);
            T0 = __builtin_amdgcn_readlane(T1, l);
            Lb0 = __builtin_amdgcn_readlane(Lv, l);
            lp0 = __builtin_amdgcn_readlane(lpv, l);
        }
    } else {
        int carry = 0;  // tiles of the requests before this group of 64
        for (int c = 0; c < p.B; c += 64) {
            const int j = c + lane;
            const int T = (valid_rows(j) + kMT - 1) / kMT;
            const int incl = wave_incl_scan(T, lane);
            const int P = carry + incl - T;  // first tile of request j
            write_meta(j, P, T);
            const uint64_t mask =
                __builtin_amdgcn_ballot_w64(working && j < p.B && T > 0 && P <= start && start < P + T);
            if (b0 < 0 && mask) {
                const int l = __builtin_ctzll(mask);
                b0 = c + l;
                P0 = __builtin_amdgcn_readlane(P, l);
                T0 = __builtin_amdgcn_readlane(T, l);
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        if (b0 >= 0) {
            typedef const __attribute__((address_space(4))) int32_t *clen0_t;
            Lb0 = ((clen0_t)p.seq_lens)[b0];
            lp0 = first_row(p, b0);
        }
    }
    if (!working) {
        if (one_pass) write_meta(lane, incl1 - T1, T1);
        return;
    }
    // the scan's loads are done; saying so with a wait the compiler models
    // keeps it from waiting on them (and so on the DMA loads) further down
    __builtin_amdgcn_s_waitcnt(0);

    // ---- stream tiles [start, end): a cursor per side walks the requests
    struct Cursor {
        int b, P, T, L, lp, seg;  // request, its first tile, tiles, end row, first row; pieces begun so far
        int64_t crow;             // its contiguous-cache row
    };
    // lengths by scalar loads: a vector load here would make the compiler wait
    // for every outstanding load, DMA ones included
    typedef const __attribute__((address_space(4))) int32_t *clen_t;
    const clen_t slens = (clen_t)p.seq_lens;
    auto advance = [&](Cursor &c) {  // to the next request with tiles (one exists before tile NT)
        do {
            c.P += c.T;
            c.b += 1;
            c.L = slens[c.b];
            c.lp = first_row(p, c.b);
            c.T = c.L > c.lp ? (c.L - (c.lp & ~(kMT - 1)) + kMT - 1) / kMT : 0;
        } while (c.T == 0);
        c.crow = PAGED ? 0 : cache_row(p, c.b);
        c.seg += 1;
    };
    const int64_t crow0 = PAGED ? 0 : cache_row(p, b0);
    Cursor prod{b0, P0, T0, Lb0, lp0, 0, crow0}, cons{b0, P0, T0, Lb0, lp0, 0, crow0};
    uint8_t *wl = lds[wv];
    // Q of request b's query tokens into ring slot qs
    auto stage_qs = [&](int b, int qs) {
#pragma unroll
        for (int j = 0; j < QL; ++j) {
            if (j >= nq) continue;
            if constexpr (HG)
                stage_q(p, b, 2 * g + j, qlds[wv][qs][j], lane);
            else
                stage_q(p, b * p.q_len + ti0 + j, g, qlds[wv][qs][j], lane);
        }
    };
    auto read_qs = [&](int qs, uint2 (&qb)[QL][8]) {
#pragma unroll
        for (int j = 0; j < QL; ++j) {
            if (j < nq) {
                read_q(qlds[wv][qs][j], lane, qb[j]);
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) qb[j][c] = make_uint2(0u, 0u);
            }
        }
    };
    // the states of request b's piece in this block: rows (token, head) of [q_len * Hq, nslots]
    auto flush = [&](const MfmaSoftmax (&st)[QL], int b, float vd) {
#pragma unroll
        for (int j = 0; j < QL; ++j) {
            if (j >= nq) continue;
            const int64_t s0 = (HG ? (int64_t)(hq0 + 4 * j) : ((int64_t)(ti0 + j) * p.Hq + hq0)) * p.nslots + blk + b;
            write_state(st[j], lane, p.po + s0 * D, p.pm + s0, p.pd + s0, p.nslots, vd);
        }
    };
    auto produce = [&](int x) {  // stage tile x (and Q when it starts a new piece)
        if (x >= prod.P + prod.T) {
            advance(prod);
            stage_qs(prod.b, prod.seg % NS);
        }
        const int t0 = (prod.lp & ~(kMT - 1)) + (x - prod.P) * kMT;
        const int64_t off = token_offset<PAGED, KF>(p, prod.b, prod.crow, g, t0);
        uint32_t kl, vl;
        slot_dma_addrs<KF>(wl, x % NS, kl, vl);
        stage_tile<KF>(p.k + off, p.v + off, kl, vl, max(prod.lp - t0, 0), prod.L - t0, stok, lane);
    };

    stage_qs(b0, 0);
    const int npro = min(NS - 1, end - start);
    for (int i = 0; i < npro; ++i) produce(start + i);

    MfmaSoftmax st[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) st[j].reset();
    uint2 qb[QL][8];
    float kd = 1.0f, vd = 1.0f;  // the current request's float8 descales
    for (int x = start; x < end; ++x) {
        if (x + NS - 1 < end) produce(x + NS - 1);
        // tile x has landed once at most the later tiles' loads remain (a Q load
        // issued after it only makes this wait longer)
        wait_vm_n<KvFmt<KF>::kDma>(min(NS - 1, end - 1 - x));
        if (x == start) {
            read_qs(0, qb);
            if (KF) {
                kd = kv_descale(p.k_descale, p, cons.b, g);
                vd = kv_descale(p.v_descale, p, cons.b, g);
            }
        } else if (x >= cons.P + cons.T) {
            flush(st, cons.b, vd);
#pragma unroll
            for (int j = 0; j < QL; ++j) st[j].reset();
            advance(cons);
            read_qs(cons.seg % NS, qb);
            if (KF) {
                kd = kv_descale(p.k_descale, p, cons.b, g);
                vd = kv_descale(p.v_descale, p, cons.b, g);
            }
        }
        const int slot = x % NS;
        const int t0 = (cons.lp & ~(kMT - 1)) + (x - cons.P) * kMT;
        int nv[QL];  // token ti0 + j sees rows up to L - q_len + ti0 + j (causal)
#pragma unroll
        for (int j = 0; j < QL; ++j) nv[j] = j < nq ? (HG ? cons.L : cons.L - p.q_len + ti0 + j + 1) - t0 : 0;
        mfma_tile<DT, KF, QL>(Ring<KF>::k_tile(wl, slot), Ring<KF>::v_tile(wl, slot), qb, max(cons.lp - t0, 0), nv,
                              p.scale_log2 * kd, lane, st);
    }
    flush(st, cons.b, vd);
    // one pass: the request metadata goes out last, off the path to the first DMA
    if (one_pass) write_meta(lane, incl1 - T1, T1);
}

template <int DT, bool PAGED, int KF, int QL, bool HG = false>
__global__ __launch_bounds__(64 * kMapMfmaWaves, 1) void map_kernel_mfma_g4_bal(const MapParams p) {
    __shared__ BalLds<KF, QL> sm;
    map_g4_bal_body<DT, PAGED, KF, QL, HG>(p, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z, sm);
}

// Instantiations: q / compute type DT (0 fp16, 1 bf16), paged or not, KV
// format (float8 caches take bf16 queries); EXTRA: further template arguments.
#define FDEC_MFMA_DISPATCH(KERNEL, ...)                                                              \
    if (p.kv_fp8) {                                                                                  \
        if (p.page_table)                                                                            \
            hipLaunchKernelGGL((KERNEL<1, true, 1 __VA_ARGS__>), grid, block, 0, st, p);             \
        else                                                                                         \
            hipLaunchKernelGGL((KERNEL<1, false, 1 __VA_ARGS__>), grid, block, 0, st, p);            \
    } else if (p.dtype == 0) {                                                                       \
        if (p.page_table)                                                                            \
            hipLaunchKernelGGL((KERNEL<0, true, 0 __VA_ARGS__>), grid, block, 0, st, p);             \
        else                                                                                         \
            hipLaunchKernelGGL((KERNEL<0, false, 0 __VA_ARGS__>), grid, block, 0, st, p);            \
    } else {                                                                                         \
        if (p.page_table)                                                                            \
            hipLaunchKernelGGL((KERNEL<1, true, 0 __VA_ARGS__>), grid, block, 0, st, p);             \
        else                                                                                         \
            hipLaunchKernelGGL((KERNEL<1, false, 0 __VA_ARGS__>), grid, block, 0, st, p);            \
    }

hipError_t launch_map_mfma_g4_balanced(const MapParams &p, int nblocks, hipStream_t st) {
    if (p.Hq == 8 * p.Hkv) {  // two groups of four query heads per wave, single query
        if (p.q_len != 1 || p.q_groups != 1) return hipErrorInvalidValue;
        dim3 grid(nblocks, 1, p.Hkv / p.heads_per_block);
        dim3 block(64 * p.heads_per_block);
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4_bal, , 2, true)
        return hipGetLastError();
    }
    if (p.Hq != 4 * p.Hkv) return hipErrorInvalidValue;
    const int ql = mfma_tokens_per_wave(p.q_len);
    if (p.q_groups != (p.q_len + ql - 1) / ql) return hipErrorInvalidValue;
    dim3 grid(nblocks, p.q_groups, p.Hkv / p.heads_per_block);
    dim3 block(64 * p.heads_per_block);
    if (ql == 1) {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4_bal, , 1)
    } else if (ql == 2) {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4_bal, , 2)
    } else {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4_bal, , 4)
    }
    return hipGetLastError();
}

hipError_t launch_map_mfma_g4(const MapParams &p, int S, hipStream_t st) {
    if (p.mode != kPlain) {  // append (single query), G = 4 or 8
        if (p.q_len != 1 || (p.kv_fp8 && p.dtype != 1)) return hipErrorInvalidValue;
        dim3 grid(S, p.B, p.Hkv / p.heads_per_block), block(64 * p.heads_per_block);
#define FDEC_APP(NG)                                                                            \
    if (p.kv_fp8) {                                                                             \
        if (p.page_table)                                                                       \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<1, true, NG, 1>), grid, block, 0, st, p);  \
        else                                                                                    \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<1, false, NG, 1>), grid, block, 0, st, p); \
    } else if (p.dtype == 0) {                                                                  \
        if (p.page_table)                                                                       \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<0, true, NG, 0>), grid, block, 0, st, p);  \
        else                                                                                    \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<0, false, NG, 0>), grid, block, 0, st, p); \
    } else {                                                                                    \
        if (p.page_table)                                                                       \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<1, true, NG, 0>), grid, block, 0, st, p);  \
        else                                                                                    \
            hipLaunchKernelGGL((map_kernel_mfma_g4_app<1, false, NG, 0>), grid, block, 0, st, p); \
    }
        if (p.Hq == 8 * p.Hkv) {
            FDEC_APP(2)
        } else {
            FDEC_APP(1)
        }
#undef FDEC_APP
        return hipGetLastError();
    }
    if (p.Hq == 8 * p.Hkv) {  // groups of eight query heads: single query
        if (p.q_len != 1) return hipErrorInvalidValue;
        dim3 grid(S, p.B, p.Hkv / p.heads_per_block), block(64 * p.heads_per_block);
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g8, )
        return hipGetLastError();
    }
    const int ql = mfma_tokens_per_wave(p.q_len);
    if (p.q_groups != (p.q_len + ql - 1) / ql) return hipErrorInvalidValue;
    dim3 grid(S, p.B * p.q_groups, p.Hkv / p.heads_per_block);
    dim3 block(64 * p.heads_per_block);
    if (ql == 1) {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4, , 1)
    } else if (ql == 2) {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4, , 2)
    } else {
        FDEC_MFMA_DISPATCH(map_kernel_mfma_g4, , 4)
    }
    return hipGetLastError();
}
#undef FDEC_MFMA_DISPATCH

// ---- Single-launch cascade (shared prefix + balanced suffixes, G = 4).
// The prefix blocks are compute-bound (matrix cores and the softmax, HBM mostly
// idle) and the balanced suffix blocks stream; run one after the other, each
// leaves the other's resource idle. Here one grid holds both: prefix blocks of
// four waves (128 query rows) take the suffix blocks' shape, so a
// block of each fits on one compute unit (LDS and VGPRs), and the roles are
// dealt so that every compute unit gets one of each. Blocks go to the eight XCDs
// in turn (block b to XCD b % 8) and, within an XCD, one per compute unit before
// any gets a second: within each run of 256 blocks, the XCDs of one parity take
// one role, and the next run swaps the parities. Pairs beyond whole runs
// alternate, and the count left over goes to whichever role has more blocks.
// The roles change only where blocks run, not what they compute: a prefix block
// is the prefix kernel's work on its row chunk, a suffix block the balanced
// kernel's block `blk` of `ss`, both with the same arithmetic.
__device__ __forceinline__ void cascade_role(int b, int NPf, int NSf, bool &prefix, int &v) {
    const int npair = min(NPf, NSf);
    const int runs = (2 * npair) / 256;  // whole runs of 256 blocks, 128 of each role
    if (b < 256 * runs) {
        const int run = b >> 8, x = b & 7, j = (b & 255) >> 3;
        prefix = ((x + run) & 1) == 0;
        v = run * 128 + j * 4 + (x >> 1);
        return;
    }
    const int b_alt = 256 * runs + 2 * (npair - 128 * runs);
    if (b < b_alt) {
        const int k = b - 256 * runs;
        prefix = (k & 1) == 0;
        v = 128 * runs + (k >> 1);
        return;
    }
    prefix = NPf > NSf;
    v = npair + (b - b_alt);
}

// Prefix ring slots: two for 16-bit pools (the union is then the suffix's 72 KB),
// three for float8 pools (half-size tiles: 52 KB, inside the suffix's 60 KB).
template <int KF> struct CascadeFusedSlots {
    static constexpr int kValue = KF ? 3 : 2;
};
template <int KF> union CascadeFusedLds {
    PfxLds<KF, CascadeFusedSlots<KF>::kValue> pf;
    BalLds<KF, 1> sf;
};

template <int DT, int KF>
__global__ __launch_bounds__(64 * kMapMfmaWaves, 2) void cascade_fused_kernel(const CascadeParams cp,
                                                                                const MapParams pb, int NPf,
                                                                                int NSf, int sp, int ss) {
    __shared__ CascadeFusedLds<KF> sm;
    bool prefix;
    int v;
    cascade_role((int)blockIdx.x, NPf, NSf, prefix, v);
    // Float8 pools: a suffix block's waves win issue over the prefix block's waves
    // on a shared SIMD, so their tile loads go out without waiting behind the
    // prefix's conversions and products (a wave's priority only orders issue;
    // no wave waits on another block). 16-bit pools keep equal priority, which
    // measured no slower.
    if (KF && !prefix) __builtin_amdgcn_s_setprio(3);
    if (prefix)
        cascade_prefix_body<DT, KF, kMapMfmaWaves, CascadeFusedSlots<KF>::kValue>(cp, v % sp, (v / sp) % cp.Hkv,
                                                                               v / (sp * cp.Hkv), sm.pf);
    else
        map_g4_bal_body<DT, true, KF, 1, false>(pb, v % ss, ss, 0, v / ss, sm.sf);
}

int cascade_fused_blocks(const CascadeParams &cp, int sp, int ss, int *nprefix, int *nsuffix) {
    constexpr int kRows = kMapMfmaWaves * kPfxRowsPerWave;
    const int R = cp.B * (cp.Hq / cp.Hkv);
    const int64_t np = (int64_t)sp * cp.Hkv * ((R + kRows - 1) / kRows);
    const int64_t ns = (int64_t)ss * (cp.Hkv / kMapMfmaWaves);
    if (np + ns > INT32_MAX) return 0;
    *nprefix = (int)np;
    *nsuffix = (int)ns;
    return 1;
}

hipError_t launch_cascade_fused(const CascadeParams &cp, const MapParams &pb, int sp, int ss, hipStream_t st) {
    if (pb.heads_per_block != kMapMfmaWaves || cp.Hq != 4 * cp.Hkv || pb.Hq != cp.Hq || pb.Hkv != cp.Hkv ||
        pb.q_len != 1 || pb.q_groups != 1 || !pb.page_table || pb.kv_fp8 != cp.kv_fp8 || sp < 1 || ss < 1)
        return hipErrorInvalidValue;
    int np = 0, ns = 0;
    if (!cascade_fused_blocks(cp, sp, ss, &np, &ns)) return hipErrorInvalidValue;
    const dim3 grid(np + ns), block(64 * kMapMfmaWaves);
    if (cp.kv_fp8) {
        if (cp.dtype != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((cascade_fused_kernel<1, 1>), grid, block, 0, st, cp, pb, np, ns, sp, ss);
    } else if (cp.dtype == 0) {
        hipLaunchKernelGGL((cascade_fused_kernel<0, 0>), grid, block, 0, st, cp, pb, np, ns, sp, ss);
    } else {
        hipLaunchKernelGGL((cascade_fused_kernel<1, 0>), grid, block, 0, st, cp, pb, np, ns, sp, ss);
    }
    return hipGetLastError();
}

}  // namespace fdec
