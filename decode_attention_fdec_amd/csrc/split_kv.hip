// Split-KV map kernel (the FlashDecoding map stage) for gfx950.
//
// Method: lpnh.cn FlashDecoding explainer §2 stage 1 and tbr8.org "FlashDecoding 与
// FlashInfer 深度解析" §2.1 steps 1-2: the KV sequence of each (request, KV head)
// is cut into equal chunks; each chunk yields the local max m_i, the local sum of
// exponentials d_i and the unnormalised output O~_i. With a single-kernel merge
// (lpnh §3, unified kernel with atomics) the last block to finish a
// (request, head group) merges its splits. Optional KV append with NeoX rotary
// follows the flash-attn "Inference Cookbook / 推理优化" page §3.3-3.4.
//
// Layout on the chip. Grid (split, request, head group); a block has one wave
// per KV head of its group (up to 8), so together its waves read whole token
// rows of the NHD cache -- the DRAM-friendly order -- while each wave serves
// the G = Hq/Hkv query heads of its KV head (GQA reuse, lpnh §3): every K/V byte
// is read from HBM once. A wave streams the split's 16-token tiles on its own;
// a tile is two groups of 8 rows, one row per 8 lanes. Lane (row a = lane / 8,
// chunk c = lane % 8) loads the 16-byte pieces [8c, 8c+8) and [64+8c, 64+8c+8)
// of its row (D = 128), so every load instruction covers eight full 128-byte
// lines. q.k uses v_dot2 on packed fp16/bf16 (products exact in fp32) and an
// 8-lane DPP sum; softmax runs in the log2 domain in fp32; the next tiles' loads
// are in flight while the current one is computed. Each lane row keeps its own
// (m, d, acc); the eight row states are merged with shuffles and the wave writes
// its heads' states itself.
//
// Float8 e4m3fn caches (plain decode, bf16 queries): a lane loads the same
// elements as for 16-bit caches, as 8-byte pieces (a row is D bytes), and
// widens them exactly to packed bf16 before q.k and P.V; K's descale scales
// the scores and V's the state's O~.
#include <type_traits>

#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

// Kernel-only modes over a float8 e4m3fn cache: plain decode, and the two
// append modes (the new row stored as codes of value / descale).
constexpr int kPlainF8 = 3, kAppendF8 = 4, kAppendRopeF8 = 5;
static_assert(kPlainF8 != kPlain && kPlainF8 != kAppend && kPlainF8 != kAppendRope && kAppendF8 > kAppendRope,
              "distinct modes");

// Register tiles in flight per wave and the waves per SIMD the kernel is
// compiled for, by GQA group size (D = 128): more tiles hide more latency,
// fewer registers allow more resident waves.
#ifndef FDEC_NBUF_G4
#define FDEC_NBUF_G4 2
#endif
#ifndef FDEC_OCC_G4
#define FDEC_OCC_G4 2
#endif
template <int G, int D> struct MapConfig {
    static constexpr bool big = (G >= 8 && D >= 128);  // needs more than 256 registers per lane
    static constexpr int nbuf = big ? 2 : (G == 4 && D >= 128) ? FDEC_NBUF_G4 : 3;
    static constexpr int occ = big ? 1 : (G == 4 && D >= 128) ? FDEC_OCC_G4 : 2;
    static constexpr int max_waves = big ? kMapMaxWavesBig : kMapMaxWaves;
};

template <int DT, int D, int G, bool PAGED, int MODE>
__global__ __launch_bounds__((64 * MapConfig<G, D>::max_waves), (MapConfig<G, D>::occ)) void map_kernel(
    const MapParams p) {
    constexpr int NCH = D / 64;           // 16-byte pieces per lane per row
    constexpr int NE = NCH * 8;           // elements per lane per row
    constexpr int NQ = NCH * 4;           // packed dwords per lane per row
    constexpr int NR = (G >= 8) ? 1 : 2;  // 8-row groups per tile
    constexpr int TT = 8 * NR;            // tokens per tile
    constexpr bool QF32 = (MODE == kAppendRope || MODE == kAppendRopeF8);  // rotary: q in fp32
    constexpr int NBUF = MapConfig<G, D>::nbuf;
    constexpr bool F8 = (MODE == kPlainF8 || MODE == kAppendF8 || MODE == kAppendRopeF8);
    constexpr bool APPEND = (MODE == kAppend || MODE == kAppendRope || MODE == kAppendF8 || MODE == kAppendRopeF8);
    constexpr int ES = F8 ? 1 : 2;  // bytes per cache element
    static_assert(!F8 || DT == 1, "float8 caches take bf16 queries");
    using E = Elem<DT>;
    using Piece = typename std::conditional<F8, uint2, uint4>::type;  // one lane's 8 elements of a row

    __shared__ float sm_vec[QF32 ? MapConfig<G, D>::max_waves * (G + 1) * D : 1];
    __shared__ int sm_flag;

    const int split = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.z * p.heads_per_block + wv;
    const int ra = lane >> 3, cb = lane & 7;
    const int hq0 = g * G;

    const int c_app = p.seq_lens[b];
    const int L = APPEND ? c_app + 1 : c_app;
    const int lp = p.leftpad ? p.leftpad[b] : 0;            // first valid row (left padding)
    const int64_t crow = p.batch_idx ? p.batch_idx[b] : b;  // contiguous caches: the request's cache row
    // split boundaries: multiples of 16 rows from the 16-row tile holding the
    // first valid row (tiles of a paged cache then stay on one page)
    const int t_begin = (lp & ~15) + split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);

    // Element offset of logical token t (KV head g), page table read for paged caches.
    auto row_offset = [&](int t) -> int64_t {
        if constexpr (PAGED) {
            int pidx = p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
            int slot = t - pidx * p.page_size;
            int64_t page = p.page_table[(int64_t)b * p.max_pages + pidx];
            return page * p.s_outer + (int64_t)slot * p.s_token + (int64_t)g * p.s_head;
        } else {
            return crow * p.s_outer + (int64_t)t * p.s_token + (int64_t)g * p.s_head;
        }
    };

    // Float8 append: the new row's codes, value / descale rounded to e4m3fn
    // (the k value from kf in fp32 when rotated, else from the bf16 ksrc).
    auto store_row_f8 = [&](int64_t off, const float *kf, const uint16_t *ksrc, const uint16_t *vsrc, int ln) {
        uint8_t *kd = reinterpret_cast<uint8_t *>(const_cast<char *>(p.k)) + off;
        uint8_t *vd = reinterpret_cast<uint8_t *>(const_cast<char *>(p.v)) + off;
        const float kds = kv_descale(p.k_descale, p, b, g), vds = kv_descale(p.v_descale, p, b, g);
        for (int i = ln; i < D; i += 64) {
            const float kx = kf ? kf[i] : Elem<1>::lo((uint32_t)ksrc[i]);
            kd[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(kx, kds));
            vd[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(Elem<1>::lo((uint32_t)vsrc[i]), vds));
        }
    };
    (void)store_row_f8;

    // ---------------------------------------------------------------- q (and append)
    uint32_t qp[QF32 ? 1 : G][NQ];
    float qf[QF32 ? G : 1][QF32 ? NE : 1];
    const bool owner = APPEND && (t_begin <= c_app) && (c_app < t_begin + p.chunk);
    if constexpr (QF32) {
        // rotate q (and, in the block owning the new row, k_new) in this wave's
        // part of LDS, fp32
        float *qs = sm_vec + wv * (G + 1) * D;
        float *ks = qs + G * D;
        const uint16_t *qsrc = reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hq + hq0) * D;
        const uint16_t *ksrc = reinterpret_cast<const uint16_t *>(p.k_new) + ((int64_t)b * p.Hkv + g) * D;
        for (int i = lane; i < G * D; i += 64) qs[i] = E::lo((uint32_t)qsrc[i]);
        if (owner)
            for (int i = lane; i < D; i += 64) ks[i] = E::lo((uint32_t)ksrc[i]);
        __builtin_amdgcn_wave_barrier();
        const int half = p.rotary_dim >> 1;
        // the new row's position among the valid rows
        const float *cs = p.rope_cos + (int64_t)(c_app - lp) * half;
        const float *sn = p.rope_sin + (int64_t)(c_app - lp) * half;
        const int nvec = owner ? G + 1 : G;
        for (int i = lane; i < nvec * half; i += 64) {
            int h = i / half, j = i - h * half;
            float *x = qs + h * D;
            float c = cs[j], s = sn[j];
            float x0 = x[j], x1 = x[j + half];
            x[j] = x0 * c - x1 * s;
            x[j + half] = x0 * s + x1 * c;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[h][c * 8 + e] = qs[h * D + 64 * c + 8 * cb + e];
        if (owner) {
            const int64_t off = row_offset(c_app);
            const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(p.v_new) + ((int64_t)b * p.Hkv + g) * D;
            if constexpr (F8) {
                store_row_f8(off, ks, nullptr, vsrc, lane);
            } else {
                uint16_t *kd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.k)) + off;
                uint16_t *vd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.v)) + off;
                for (int i = lane; i < D; i += 64) {
                    kd[i] = E::from_float(ks[i]);
                    vd[i] = vsrc[i];
                }
            }
            // this wave reads the row back below, through the same L2; no
            // earlier load of this kernel cached it in L1: completing the
            // stores is enough (an agent-scope fence would also write the
            // XCD's L2 back to memory)
            __builtin_amdgcn_s_waitcnt(0);
        }
    } else {
        const uint16_t *qsrc = reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hq + hq0) * D;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                uint4 u = *reinterpret_cast<const uint4 *>(qsrc + h * D + 64 * c + 8 * cb);
                qp[h][4 * c + 0] = u.x;
                qp[h][4 * c + 1] = u.y;
                qp[h][4 * c + 2] = u.z;
                qp[h][4 * c + 3] = u.w;
            }
        if constexpr (APPEND) {
            if (owner) {
                const int64_t off = row_offset(c_app);
                const uint16_t *ksrc = reinterpret_cast<const uint16_t *>(p.k_new) + ((int64_t)b * p.Hkv + g) * D;
                const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(p.v_new) + ((int64_t)b * p.Hkv + g) * D;
                if constexpr (F8) {
                    store_row_f8(off, nullptr, ksrc, vsrc, lane);
                } else {
                    uint16_t *kd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.k)) + off;
                    uint16_t *vd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.v)) + off;
                    for (int i = lane; i < D; i += 64) {
                        kd[i] = ksrc[i];
                        vd[i] = vsrc[i];
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);  // as above: the stores complete before the read-back
            }
        }
    }

    // ---------------------------------------------------------------- stream the split
    // Online softmax with a lazily moved reference: scores are in the log2
    // domain; m is the reference every exponential is taken against and only
    // moves (rescaling l and acc) when a score exceeds it by more than kTau, so
    // p <= 2^kTau. tmax tracks the true maximum for the state written out.
    // Rows of a lane group that have seen no token keep m = kFloor (finite), so
    // masked scores (-inf) give p = 0 without a NaN.
    constexpr float kTau = 8.0f;
    constexpr float kFloor = -1.0e30f;
    float m[G], tmax[G], l[G], acc[G][NE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kFloor;
        tmax[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[h][e] = 0.0f;
    }

    // tokens [t_lo, t_end) in tiles of TT rows from t_first; the first tile's
    // rows below t_lo are left padding (read as row t_lo, masked)
    const int t_lo = max(t_begin, lp);
    const int t_first = t_lo & ~(TT - 1);
    const int nskip0 = t_lo - t_first;
    const int ntiles = t_end > t_lo ? (t_end - t_first + TT - 1) / TT : 0;
    const char *kbase = p.k;
    const char *vbase = p.v;
    const uint32_t tok_bytes = (uint32_t)(p.s_token * ES);
    // float8: scores in log2 units with K's descale, O~ with V's
    const float score_scale = F8 ? p.scale_log2 * kv_descale(p.k_descale, p, b, g) : p.scale_log2;
    const float o_scale = F8 ? kv_descale(p.v_descale, p, b, g) : 1.0f;

    struct Tile {
        Piece k[NR][NCH];
        Piece v[NR][NCH];
    };
    // the NQ packed 16-bit dwords of one row of a tile (float8: widened to bf16)
    auto row_words = [](const Piece (&r)[NCH], uint32_t (&w)[NQ]) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if constexpr (F8) {
                const uint2 a = fp8x4_to_bf16(r[c].x), bb = fp8x4_to_bf16(r[c].y);
                w[4 * c + 0] = a.x;
                w[4 * c + 1] = a.y;
                w[4 * c + 2] = bb.x;
                w[4 * c + 3] = bb.y;
            } else {
                w[4 * c + 0] = r[c].x;
                w[4 * c + 1] = r[c].y;
                w[4 * c + 2] = r[c].z;
                w[4 * c + 3] = r[c].w;
            }
        }
    };
    auto tile_t0 = [&](int i) { return t_first + i * TT; };

    // Per-lane byte offsets of this lane's rows within a tile: loop-invariant,
    // except in the split's last tile, whose rows past t_end clamp to its last
    // valid row, and a first tile with left padding, whose rows below t_lo
    // clamp to its first valid row (their scores are masked later).
    const int last_t0 = t_first + (ntiles - 1) * TT;
    const int nvalid_last = t_end - last_t0;
    const int nhi_first = (ntiles == 1 ? nvalid_last : TT) - 1;
    uint32_t off_full[NR], off_last[NR], off_first[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        off_full[j] = (uint32_t)(8 * j + ra) * tok_bytes + (uint32_t)cb * 8u * ES;
        off_last[j] = (uint32_t)min(8 * j + ra, nvalid_last - 1) * tok_bytes + (uint32_t)cb * 8u * ES;
        off_first[j] = (uint32_t)min(max(8 * j + ra, nskip0), nhi_first) * tok_bytes + (uint32_t)cb * 8u * ES;
    }

    // Issue the loads of the tile starting at token t0.
    auto issue = [&](Tile &T, int t0) {
        const int64_t base = row_offset(t0);
        const char *kb = kbase + base * ES;
        const char *vb = vbase + base * ES;
        const bool last = (t0 == last_t0);
        const bool first = (t0 == t_first) && nskip0 > 0;
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const uint32_t off = first ? off_first[j] : last ? off_last[j] : off_full[j];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                T.k[j][c] = load_nt<Piece>(kb + off + c * 64 * ES);
                T.v[j][c] = load_nt<Piece>(vb + off + c * 64 * ES);
            }
        }
    };

    auto compute = [&](const Tile &T, int t0) {
        const int nvalid = t_end - t0;
        const int nskip = (t0 == t_first) ? nskip0 : 0;
        float sc[NR][G];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            uint32_t kw[NQ];
            row_words(T.k[j], kw);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = 0.0f;
                if constexpr (QF32) {
#pragma unroll
                    for (int i = 0; i < NQ; ++i) {
                        s = fmaf(qf[h][2 * i], E::lo(kw[i]), s);
                        s = fmaf(qf[h][2 * i + 1], E::hi(kw[i]), s);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < NQ; ++i) s = E::dot2(qp[h][i], kw[i], s);
                }
                sc[j][h] = sum8(s) * score_scale;
            }
        }
        if (nvalid < TT || nskip > 0) {  // a split's last tile, a padded first tile (wave-uniform branch)
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (8 * j + ra >= nvalid || 8 * j + ra < nskip) sc[j][h] = kNegInf;
        }
        float mx[G];
        bool move = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mx[h] = sc[0][h];
#pragma unroll
            for (int j = 1; j < NR; ++j) mx[h] = fmax_nc(mx[h], sc[j][h]);
            tmax[h] = fmax_nc(tmax[h], mx[h]);
            move |= mx[h] > m[h] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(move) != 0) {  // rare after the first tiles
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mn = fmax_nc(m[h], mx[h]);
                const float alpha = fexp2(m[h] - mn);
                m[h] = mn;
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[h][e] *= alpha;
            }
        }
        float vf[NR][NE];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            uint32_t vw[NQ];
            row_words(T.v[j], vw);
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                vf[j][2 * i] = E::lo(vw[i]);
                vf[j][2 * i + 1] = E::hi(vw[i]);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float pj[NR];
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                pj[j] = fexp2(sc[j][h] - m[h]);
                l[h] += pj[j];
            }
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                float a = acc[h][e];
#pragma unroll
                for (int j = 0; j < NR; ++j) a = fmaf(pj[j], vf[j][e], a);
                acc[h][e] = a;
            }
        }
    };

    if (ntiles > 0) {
        // NBUF register tiles rotate: while one is computed, the next NBUF - 1
        // are in flight. Loads are unconditional -- indices past the end
        // re-issue the last tile -- so every wait count in the loop is static.
        Tile T[NBUF];
        const int last = ntiles - 1;
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) issue(T[u], tile_t0(min(u, last)));
        int i = 0;
        for (; i + NBUF <= ntiles; i += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                issue(T[(u + NBUF - 1) % NBUF], tile_t0(min(i + u + NBUF - 1, last)));
                compute(T[u], tile_t0(i + u));
            }
        }
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u)
            if (i + u < ntiles) compute(T[u], tile_t0(i + u));
    }

    // ---------------------------------------------------------------- merge the lane rows
#pragma unroll
    for (int step = 8; step <= 32; step <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = shfl_xor(m[h], step);
            const float lo = shfl_xor(l[h], step);
            tmax[h] = fmax_nc(tmax[h], shfl_xor(tmax[h], step));
            const float mn = fmax_nc(m[h], mo);
            const float as = fexp2(m[h] - mn), ao = fexp2(mo - mn);
            l[h] = l[h] * as + lo * ao;
            m[h] = mn;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const float x = shfl_xor(acc[h][e], step);
                acc[h][e] = acc[h][e] * as + x * ao;
            }
        }
    }

    // The wave's state per head, re-expressed against the true maximum T of the
    // split: O~ = 2^(m - T) acc, d = 2^(m - T) l (m <= T, so the factor is <= 1).
    const int64_t slot = p.s_offset + split;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float T = tmax[h];
        const float f = (T == kNegInf) ? 0.0f : fexp2(m[h] - T);
        const float fo = F8 ? f * o_scale : f;  // O~ carries V's descale
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        if (ra == 0) {
            float *dst = p.po + (bh * p.s_total + slot) * D;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float4 lo4 = make_float4(acc[h][8 * c] * fo, acc[h][8 * c + 1] * fo, acc[h][8 * c + 2] * fo,
                                         acc[h][8 * c + 3] * fo);
                float4 hi4 = make_float4(acc[h][8 * c + 4] * fo, acc[h][8 * c + 5] * fo, acc[h][8 * c + 6] * fo,
                                         acc[h][8 * c + 7] * fo);
                *reinterpret_cast<float4 *>(dst + 64 * c + 8 * cb) = lo4;
                *reinterpret_cast<float4 *>(dst + 64 * c + 8 * cb + 4) = hi4;
            }
        }
        if (lane == 0) {
            p.pm[bh * p.s_total + slot] = (T == kNegInf) ? kNegInf : T * kLn2;
            p.pd[bh * p.s_total + slot] = l[h] * f;
        }
    }

    if (p.counters == nullptr) return;

    // ---------------------------------------------------------------- single-kernel merge
    // Publish this block's states device-wide and count arrivals per
    // (request, head group); the last block to arrive merges all splits (in split
    // order, with the merge kernel's code) and resets the counter.
    __syncthreads();  // every wave's state stores are complete
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

template <int DT, int D, int G, bool PAGED, int MODE>
static hipError_t launch_t(const MapParams &p, int S, hipStream_t st) {
    dim3 grid(S, p.B, p.Hkv / p.heads_per_block);
    hipLaunchKernelGGL((map_kernel<DT, D, G, PAGED, MODE>), grid, dim3(64 * p.heads_per_block), 0, st, p);
    return hipGetLastError();
}

template <int DT, int D, int G, bool PAGED>
static hipError_t launch_mode(const MapParams &p, int S, hipStream_t st) {
    if (p.kv_fp8) {  // bf16 queries only
        if constexpr (DT == 1) {
            switch (p.mode) {
                case kPlain: return launch_t<DT, D, G, PAGED, kPlainF8>(p, S, st);
                case kAppend: return launch_t<DT, D, G, PAGED, kAppendF8>(p, S, st);
                default: return launch_t<DT, D, G, PAGED, kAppendRopeF8>(p, S, st);
            }
        }
        return hipErrorInvalidValue;
    }
    switch (p.mode) {
        case kPlain: return launch_t<DT, D, G, PAGED, kPlain>(p, S, st);
        case kAppend: return launch_t<DT, D, G, PAGED, kAppend>(p, S, st);
        default: return launch_t<DT, D, G, PAGED, kAppendRope>(p, S, st);
    }
}

template <int DT, int D, int G>
static hipError_t launch_paged(const MapParams &p, int S, hipStream_t st) {
    return p.page_table ? launch_mode<DT, D, G, true>(p, S, st) : launch_mode<DT, D, G, false>(p, S, st);
}

template <int DT, int D>
static hipError_t launch_g(const MapParams &p, int S, hipStream_t st) {
    switch (p.Hq / p.Hkv) {
        case 1: return launch_paged<DT, D, 1>(p, S, st);
        case 2: return launch_paged<DT, D, 2>(p, S, st);
        case 4: return launch_paged<DT, D, 4>(p, S, st);
        case 8: return launch_paged<DT, D, 8>(p, S, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_map(const MapParams &p, int num_splits, hipStream_t st) {
    if (p.mfma) {
        if (!map_mfma_eligible(p) || p.heads_per_block > kMapMfmaWaves) return hipErrorInvalidValue;
        return launch_map_mfma_g4(p, num_splits, st);
    }
    if (p.head_dim == 128)
        return p.dtype == 0 ? launch_g<0, 128>(p, num_splits, st) : launch_g<1, 128>(p, num_splits, st);
    if (p.head_dim == 64)
        return p.dtype == 0 ? launch_g<0, 64>(p, num_splits, st) : launch_g<1, 64>(p, num_splits, st);
    return hipErrorInvalidValue;
}

}  // namespace fdec
