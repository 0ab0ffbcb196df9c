// Cascade prefix block: device code shared by the prefix kernel and the
// single-launch cascade kernel (the design is described in cascade.hip).
#pragma once
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

template <int DT> struct Mfma;
template <> struct Mfma<0> {
    static __device__ __forceinline__ f32x4_v run(uint4 a, uint4 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a), __builtin_bit_cast(f16x8_v, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct Mfma<1> {
    static __device__ __forceinline__ f32x4_v run(uint4 a, uint4 b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                       __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
    }
};

constexpr int kPfxKeys = 64;            // keys per tile
constexpr int kPfxRowsPerWave = 32;     // query rows per wave
constexpr int kRB = kPfxRowsPerWave / 16;

// Two 16-bit values packed (lo, hi), rounded to nearest even by the hardware.
template <int DT> __device__ __forceinline__ uint32_t pfx_pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pfx_pack2<0>(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t pfx_pack2<1>(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2{(__bf16)a, (__bf16)b});
}
typedef short pfx_s16x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pfx_s16x4_v pfx_lds_s16x4;
typedef int pfx_i32x2_v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) pfx_i32x2_v pfx_lds_i32x2;
typedef __attribute__((address_space(3))) const uint8_t pfx_lds_u8;
typedef unsigned int pfx_u32x2_v __attribute__((ext_vector_type(2)));
typedef unsigned int pfx_u32x4_v __attribute__((ext_vector_type(4)));
// An LDS pointer from an LDS byte address (reads through it are ds_* instructions
// on that address, with constant offsets folded into the instruction).
__device__ __forceinline__ pfx_lds_u8 *pfx_lds(uint32_t a) { return (pfx_lds_u8 *)(size_t)a; }

// The LDS of one prefix block: rings of NSL K tiles and NSL V tiles, and the
// split's page ids.
template <int KF, int NSL> struct PfxLds {
    __attribute__((aligned(16))) uint8_t kring[NSL][kPfxKeys * (KF ? 128 : 256)];
    __attribute__((aligned(16))) uint8_t vring[NSL][kPfxKeys * (KF ? 128 : 256)];
    int spages[kPrefixPagesPerBlock];
};

// One prefix block of W waves (W * 32 query rows) with a ring of NSL tiles:
// prefix split `split` of KV head g, row chunk rc. Every thread of the block
// calls it (it has block barriers).
template <int DT, int KF, int W, int NSL>
__device__ __forceinline__ void cascade_prefix_body(const CascadeParams &p, int split, int g, int rc,
                                                    PfxLds<KF, NSL> &sm) {
    constexpr int kPfxWaves = W;
    constexpr int kPfxRows = kPfxWaves * kPfxRowsPerWave;
    constexpr int kPfxThreads = 64 * kPfxWaves;
    constexpr int kPfxDmaRows = kPfxKeys / kPfxWaves;  // rows of each tile one wave loads
    constexpr int kPfxNS = NSL;
    constexpr int D = 128;
    constexpr int ES = KF ? 1 : 2;                 // bytes per element
    constexpr int RB = D * ES;                     // bytes per K / V row in LDS
    constexpr int kDma = 2 * kPfxDmaRows * RB / 1024;  // DMA instructions per wave and tile
    static_assert(!KF || DT == 1, "float8 pools take bf16 queries");
    static_assert(kPfxNS >= 2 && kPfxDmaRows * kPfxWaves == kPfxKeys, "ring and row split");
    auto &kring = sm.kring;
    auto &vring = sm.vring;
    auto &spages = sm.spages;

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kq = lane >> 4, li = lane & 15;
    const int G = p.Hq / p.Hkv;
    const int R = p.B * G;

    const int t_begin = split * p.chunk;
    const int t_end = min(t_begin + p.chunk, p.prefix_len);
    const int ntiles = t_end > t_begin ? (t_end - t_begin + kPfxKeys - 1) / kPfxKeys : 0;

    const int pg0 = t_begin / p.page_size;  // first page of this split's keys
    const int npg = ntiles > 0 ? (t_end - 1) / p.page_size - pg0 + 1 : 0;

    // query rows of this wave: row = rc*256 + 32w + 16rb + li; B operand per (rb, ks)
    uint4 qb[kRB][4];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int row = rc * kPfxRows + w * kPfxRowsPerWave + rb * 16 + li;
        const bool ok = row < R;
        const int b = ok ? row / G : 0, hh = ok ? row - (row / G) * G : 0;
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hq + g * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[rb][ks] = ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * ks + 8 * kq) : make_uint4(0, 0, 0, 0);
    }

    // per-lane factors of the query rows 16rb + li: float8 descales of the row's request
    float ksc[kRB], vsc[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int row = rc * kPfxRows + w * kPfxRowsPerWave + rb * 16 + li;
        const int64_t i = (int64_t)(row < R ? row / G : 0) * p.Hkv + g;
        ksc[rb] = p.scale_log2 * (KF && p.k_descale ? p.k_descale[i] : 1.0f);
        vsc[rb] = KF && p.v_descale ? p.v_descale[i] : 1.0f;
    }

    // Lane-constant parts of the LDS read addresses: the piece swizzles depend only
    // on the lane, the ring slot and the key block enter as uniform offsets.
    //  K (A of S^T): row 16kb + li, the 8 (16-bit: 16 bytes) or 8 float8 (8 bytes)
    //  elements at d = 32ks + 8kq. 16-bit: piece 4ks + kq in slot (4ks + kq) ^ li;
    //  float8: half kq & 1 of piece 2ks + kq / 2 in slot piece ^ fp8_row_swz(16kb + li)
    //  = piece ^ (li / 2) ^ 4 (kb & 1), i.e. koff[ks] ^ 64 for odd kb.
    //  V (B of P V): 16-bit, row 32kk + ra0 (+16), ra0 = 4kq + li / 4 < 16, piece
    //  2db + p0 in slot (2db + p0) ^ ra0 = 2 (db ^ ra0 / 2) + (p0 ^ (ra0 & 1));
    //  float8, row 32kk + rv0, rv0 the (li / 2)-th of the lane group's 8 keys,
    //  piece db in slot db ^ fp8_row_swz(rv0) (32kk leaves the swizzle unchanged).
    uint32_t koff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        koff[ks] = KF ? (uint32_t)(li * 128 + 16 * ((2 * ks + (kq >> 1)) ^ (li >> 1)) + 8 * (kq & 1))
                      : (uint32_t)(li * 256 + 16 * ((4 * ks + kq) ^ li));
    uint32_t vlane, vsw;
    if constexpr (KF == 1) {
        const int k8 = li >> 1;
        const int rv0 = k8 < 4 ? 4 * kq + k8 : 16 + 4 * kq + (k8 - 4);
        vlane = (uint32_t)(rv0 * 128 + 8 * (li & 1));
        vsw = (uint32_t)fp8_row_swz(rv0);
    } else {
        const int ra0 = 4 * kq + (li >> 2);
        const int p0 = (li & 3) >> 1;
        vlane = (uint32_t)(ra0 * 256 + 16 * (p0 ^ (ra0 & 1)) + 8 * (li & 1));
        vsw = (uint32_t)(ra0 >> 1);
    }

    // DMA of tile `tile` into ring slot tile % kPfxNS: this wave's kPfxDmaRows rows
    // (8w .. 8w + 7 with eight waves) of K and of V, four rows (16-bit) or eight
    // (float8) per instruction
    // (one page: pages hold multiples of 16 keys); rows past the split's end
    // repeat its last key (masked below).
    // Default cache policy: unlike the split-KV kernels' streaming reads, the
    // non-temporal one measured slower here (the prefix block's loads are fewer and
    // its time goes to the matrix cores and the state writes, not to the stream)
    // Page ids come from the LDS copy of the split's page list, or (the first
    // tiles, issued before that copy exists) from registers loaded up front.
    const uint32_t stok = (uint32_t)(p.s_token * ES);
    constexpr int kPieces = RB / 16;           // 16-byte pieces per row
    constexpr int kRowsPerDma = 64 / kPieces;  // rows one instruction moves
    constexpr int kGroups = kPfxDmaRows / kRowsPerDma;  // instructions per wave for K (and for V)
    static_assert(2 * kGroups == kDma, "one K and one V instruction per row group");
    uint32_t voff_full[kGroups];               // lane offsets of a full tile
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
        const int r = kPfxDmaRows * w + kRowsPerDma * gi + lane / kPieces;
        const int sw = KF ? fp8_row_swz(r) : (r & 15);
        voff_full[gi] = (uint32_t)(lane / kPieces) * stok + 16u * (uint32_t)((lane % kPieces) ^ sw);
    }
    // the first source row of group gi of a tile (rows past the split's end
    // repeat its last key) and the page index holding it
    auto src_row = [&](int tile, int gi, int &t, int &pidx) {
        const int t0 = t_begin + tile * kPfxKeys;
        t = t0 + min(kPfxDmaRows * w + kRowsPerDma * gi, t_end - t0 - 1);
        pidx = p.page_shift >= 0 ? (t >> p.page_shift) : t / p.page_size;
    };
    // page ids of the first tiles, read before any tile load is issued (wave-
    // uniform scalar loads: nothing the kernel writes has happened yet)
    int ppage[kPfxNS - 1][kGroups] = {};
    if (ntiles > 0) {
#pragma unroll
        for (int tt = 0; tt < kPfxNS - 1; ++tt)
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                int t, pidx;
                src_row(min(tt, ntiles - 1), gi, t, pidx);
                ppage[tt][gi] = p.prefix_pages[__builtin_amdgcn_readfirstlane(pidx)];
            }
    }
    auto issue = [&](int tile, const int *pro) {
        const int t0 = t_begin + tile * kPfxKeys;
        const int nvalid = t_end - t0;
        const int slot = tile % kPfxNS;
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            const int r0 = kPfxDmaRows * w + kRowsPerDma * gi;
            const int rs = min(r0, nvalid - 1);  // the group's first source row
            int t, pidx;
            src_row(tile, gi, t, pidx);
            const int page = pro ? pro[gi] : spages[pidx - pg0];
            const int64_t eoff = (int64_t)page * p.s_outer + (int64_t)(t - pidx * p.page_size) * p.s_token +
                                 (int64_t)g * p.s_head;
            uint32_t voff = voff_full[gi];
            if (__builtin_expect(nvalid < kPfxKeys, 0)) {
                const int r = r0 + lane / kPieces;
                const int sw = KF ? fp8_row_swz(r) : (r & 15);
                voff = (uint32_t)(min(r, nvalid - 1) - rs) * stok + 16u * (uint32_t)((lane % kPieces) ^ sw);
            }
            dma16(reinterpret_cast<const char *>(p.k) + eoff * ES, voff, lds_addr(kring[slot]) + (uint32_t)RB * r0);
            dma16(reinterpret_cast<const char *>(p.v) + eoff * ES, voff, lds_addr(vring[slot]) + (uint32_t)RB * r0);
        }
    };

    constexpr float kTau = 8.0f;
    constexpr float kFloor = -1.0e30f;
    float m[kRB], tmax[kRB], l[kRB];
    f32x4_v o[kRB][8];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        m[rb] = kFloor;
        tmax[rb] = kNegInf;
        l[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rb][db] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // The first tile's loads go out at once, so that their latency overlaps the
    // query loads above and the page-list copy below. One wait (modelled by the
    // compiler, so no later wait of its own counts the tile loads) covers those;
    // the second tile then streams in while the first is computed, and the first
    // iteration's barrier publishes the page list.
    const int npro = min(kPfxNS - 1, ntiles);
    if (npro > 0) issue(0, ppage[0]);
    for (int i = tid; i < npg; i += kPfxThreads) spages[i] = p.prefix_pages[pg0 + i];
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int t = 1; t < kPfxNS - 1; ++t)
        if (t < npro) issue(t, ppage[t]);
    for (int tile = 0; tile < ntiles; ++tile) {
        // this wave's part of the tile has landed once only later tiles' loads
        // remain; the barrier then covers every wave's part, and every wave is
        // done with the slot the next DMA overwrites (read two tiles ago)
        wait_vm_n<kDma>(min(kPfxNS - 2, ntiles - 1 - tile));
        __syncthreads();
        if (tile + kPfxNS - 1 < ntiles) issue(tile + kPfxNS - 1, nullptr);
        const int t0 = t_begin + tile * kPfxKeys;
        // the slot's LDS bases as scalars (one value per wave), so each read adds
        // only its lane-constant offset
        const uint32_t slot_off = (uint32_t)(tile % kPfxNS) * (uint32_t)(kPfxKeys * RB);
        pfx_lds_u8 *K = pfx_lds(__builtin_amdgcn_readfirstlane(lds_addr(kring[0]) + slot_off));
        pfx_lds_u8 *V = pfx_lds(__builtin_amdgcn_readfirstlane(lds_addr(vring[0]) + slot_off));

        // ---- S^T = K Q^T: s[kb][rb] holds keys 16kb + 4kq + r of row 16rb + li
        f32x4_v s[4][kRB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) s[kb][rb] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint4 a;
                if constexpr (KF == 1) {
                    const pfx_u32x2_v k8 = *(const __attribute__((address_space(3))) pfx_u32x2_v *)(
                        K + 2048 * kb + (koff[ks] ^ (64u * (uint32_t)(kb & 1))));
                    const uint2 lo = fp8x4_to_bf16(k8.x), hi = fp8x4_to_bf16(k8.y);
                    a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    const pfx_u32x4_v k16 =
                        *(const __attribute__((address_space(3))) pfx_u32x4_v *)(K + 4096 * kb + koff[ks]);
                    a = make_uint4(k16.x, k16.y, k16.z, k16.w);
                }
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb) s[kb][rb] = Mfma<DT>::run(a, qb[rb][ks], s[kb][rb]);
            }
        }

        // ---- online softmax per query row (only a split's last tile can hold keys
        // past its end)
        const int nvalid = t_end - t0;
        bool move = false;
        float mx[kRB];
        if (__builtin_expect(nvalid < kPfxKeys, 0)) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * kb + 4 * kq + r >= nvalid) s[kb][rb][r] = kNegInf;
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float x = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) x = fmaxf(x, s[kb][rb][r]);
            x = across_rows(x, MaxOp{});  // lanes L, L ^ 16, L ^ 32, L ^ 48: the row's 64 keys
            x *= ksc[rb];  // the largest scaled score (rounding is monotone, the factor positive)
            mx[rb] = x;
            tmax[rb] = fmaxf(tmax[rb], x);
            move |= x > m[rb] + kTau;
        }
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
            // move the reference; a lane's O^T values belong to its own row
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const float mn = fmaxf(m[rb], mx[rb]);
                const float alpha = fexp2(m[rb] - mn);
                m[rb] = mn;
                l[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[rb][db][r] *= alpha;
            }
        }
        // P rounded to the input type, packed as the B operand of V^T P^T (the sum
        // of weights stays in fp32): K-slot 8kq + e is key
        // 32kk + 4kq + e (e < 4) or 32kk + 16 + 4kq + (e - 4) (e >= 4)
        uint4 pa[kRB][2];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float ps = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint32_t wv[4];
#pragma unroll
                for (int hbk = 0; hbk < 2; ++hbk) {
                    const int kb = 2 * kk + hbk;
                    float pv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pv[r] = fexp2(fmaf(s[kb][rb][r], ksc[rb], -m[rb]));
                        ps += pv[r];  // the denominator keeps fp32 weights
                    }
                    wv[2 * hbk] = pfx_pack2<DT>(pv[0], pv[1]);
                    wv[2 * hbk + 1] = pfx_pack2<DT>(pv[2], pv[3]);
                }
                pa[rb][kk] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            l[rb] += ps;
        }

        // ---- O^T += V^T P^T
        // A operand of K-slots 8kq .. 8kq + 7 at d = 16db + li: keys 32kk + 4kq + 0..3
        // and 32kk + 16 + 4kq + 0..3, each set from one transpose read whose lane m
        // (of 16) addresses key row 32kk (+16) + 4kq + m / 4, d 16db + 4 (m % 4) .. + 3.
        // Float8: one 8-bit transpose read (in each group of 16 lanes, lane j gets
        // byte j % 8 of the 8-byte chunks of lanes j / 8 + 2k, k = 0..7) whose lane m
        // addresses the k = m / 2-th of those 8 keys, bytes 16db + 8 (m & 1) .. + 7
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if constexpr (KF == 1) {
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const pfx_i32x2_v x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (pfx_lds_i32x2 *)(V + 4096 * kk + vlane + 16u * ((uint32_t)db ^ vsw)));
                    const uint2 v0 = fp8x4_to_bf16((uint32_t)x[0]), v1 = fp8x4_to_bf16((uint32_t)x[1]);
                    const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
                    for (int rb = 0; rb < kRB; ++rb) o[rb][db] = Mfma<DT>::run(bop, pa[rb][kk], o[rb][db]);
                }
            } else {
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    pfx_lds_u8 *va = V + 8192 * kk + vlane + 32u * ((uint32_t)db ^ vsw);
                    const pfx_s16x4_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pfx_lds_s16x4 *)va);
                    const pfx_s16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pfx_lds_s16x4 *)(va + 4096));
                    const uint2 v0 = __builtin_bit_cast(uint2, x0), v1 = __builtin_bit_cast(uint2, x1);
                    const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
                    for (int rb = 0; rb < kRB; ++rb) o[rb][db] = Mfma<DT>::run(bop, pa[rb][kk], o[rb][db]);
                }
            }
        }

    }

    // ---- states against the true maximum: O~ = O 2^(m - T), d = l 2^(m - T).
    // Lane (kq, li) holds d = 16db + 4kq .. + 3 of row 16rb + li: one 16-byte
    // store per (rb, db).
    const int64_t slot = p.s_offset + split;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const float lt = across_rows(l[rb], AddOp{});
        const float T = tmax[rb];
        const float f = (T == kNegInf) ? 0.0f : fexp2(m[rb] - T);
        const int row = rc * kPfxRows + w * kPfxRowsPerWave + 16 * rb + li;
        if (row >= R) continue;
        const int b = row / G, hh = row - b * G;
        const int64_t bh = (int64_t)b * p.Hq + g * G + hh;
        const float fo = f * vsc[rb];  // V's descale (1 for 16-bit pools)
        float4 *dst = reinterpret_cast<float4 *>(p.po + (bh * p.s_total + slot) * D + 4 * kq);
#pragma unroll
        for (int db = 0; db < 8; ++db)
            dst[4 * db] = make_float4(o[rb][db][0] * fo, o[rb][db][1] * fo, o[rb][db][2] * fo, o[rb][db][3] * fo);
        if (kq == 0) {
            p.pd[bh * p.s_total + slot] = lt * f;
            p.pm[bh * p.s_total + slot] = (T == kNegInf) ? kNegInf : T * kLn2;
        }
    }
}


}  // namespace fdec
