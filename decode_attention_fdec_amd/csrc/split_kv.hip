// Split-KV map kernel (the FlashDecoding map stage) for gfx950.
//
// Method: lpnh.cn FlashDecoding explainer §2 stage 1 and tbr8.org "FlashDecoding 与
// FlashInfer 深度解析" §2.1 steps 1-2: the KV sequence of each (request, KV head)
// is cut into equal chunks; each chunk yields the local max m_i, the local sum of
// exponentials d_i and the unnormalised output O~_i. With a single-kernel merge
// (lpnh §3, unified kernel with atomics) the last block to finish a
// (request, KV head) merges its splits. Optional KV append with NeoX rotary
// follows the flash-attn "Inference Cookbook / 推理优化" page §3.3-3.4.
//
// Layout on the chip. Grid (split, kv_head, request), 4 waves per block. One
// block serves all G = Hq/Hkv query heads of its KV head (GQA reuse, lpnh §3), so
// every K/V byte is read from HBM once. A wave streams 16-token tiles (tiles of a
// block are dealt round-robin to its waves, so the four waves read neighbouring
// rows): each tile is two groups of 8 rows, one row per 8 lanes. Lane
// (row a = lane / 8, chunk c = lane % 8) loads the 16-byte pieces [8c, 8c+8) and
// [64+8c, 64+8c+8) of its row (D = 128), so every load instruction covers eight
// full 128-byte lines. q.k uses v_dot2 on packed fp16/bf16 (products exact in
// fp32) and an 8-lane DPP sum; softmax runs in the log2 domain in fp32; the
// next tile's loads are in flight while the current one is computed. Each lane
// row keeps its own (m, d, acc); the eight row states of a wave and then the
// four waves are merged once at the end.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {

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
    static constexpr int nbuf = (G >= 8 && D >= 128) ? 2 : (G == 4 && D >= 128) ? FDEC_NBUF_G4 : 3;
    static constexpr int occ = (G >= 8 && D >= 128) ? 1 : (G == 4 && D >= 128) ? FDEC_OCC_G4 : 2;
};

template <int DT, int D, int G, bool PAGED, int MODE>
__global__ __launch_bounds__(kMapThreads, (MapConfig<G, D>::occ)) void map_kernel(const MapParams p) {
    constexpr int NCH = D / 64;           // 16-byte pieces per lane per row
    constexpr int NE = NCH * 8;           // elements per lane per row
    constexpr int NQ = NCH * 4;           // packed dwords per lane per row
    constexpr int NR = (G >= 8) ? 1 : 2;  // 8-row groups per tile
    constexpr int TT = 8 * NR;            // tokens per tile
    constexpr bool QF32 = (MODE == kAppendRope);
    constexpr int NBUF = MapConfig<G, D>::nbuf;
    using E = Elem<DT>;

    __shared__ float sm_acc[kMapWaves][G][D];
    __shared__ float sm_m[kMapWaves][G];
    __shared__ float sm_l[kMapWaves][G];
    __shared__ float sm_t[kMapWaves][G];
    __shared__ float sm_vec[(MODE == kAppendRope) ? (G + 1) * D : 1];
    __shared__ int sm_flag;

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ra = lane >> 3, cb = lane & 7;
    const int hq0 = g * G;

    const int c_app = p.seq_lens[b];
    const int L = (MODE == kPlain) ? c_app : c_app + 1;
    const int t_begin = split * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);

    // Element offset of logical token t (KV head g), page table read for paged caches.
    auto row_offset = [&](int t) -> int64_t {
        if constexpr (PAGED) {
            int pidx = p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
            int slot = t - pidx * p.page_size;
            int64_t page = p.page_table[(int64_t)b * p.max_pages + pidx];
            return page * p.s_outer + (int64_t)slot * p.s_token + (int64_t)g * p.s_head;
        } else {
            return (int64_t)b * p.s_outer + (int64_t)t * p.s_token + (int64_t)g * p.s_head;
        }
    };

    // ---------------------------------------------------------------- q (and append)
    uint32_t qp[QF32 ? 1 : G][NQ];
    float qf[QF32 ? G : 1][QF32 ? NE : 1];
    if constexpr (MODE == kAppendRope) {
        // rotate q (and, in the block owning the new row, k_new) in LDS, fp32
        float *qs = sm_vec;
        float *ks = sm_vec + G * D;
        const bool owner = (t_begin <= c_app) && (c_app < t_begin + p.chunk);
        const uint16_t *qsrc = reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)b * p.Hq + hq0) * D;
        const uint16_t *ksrc = reinterpret_cast<const uint16_t *>(p.k_new) + ((int64_t)b * p.Hkv + g) * D;
        for (int i = tid; i < G * D; i += kMapThreads) {
            uint32_t u = qsrc[i];
            qs[i] = E::lo(u);
        }
        if (owner)
            for (int i = tid; i < D; i += kMapThreads) ks[i] = E::lo((uint32_t)ksrc[i]);
        __syncthreads();
        const int half = p.rotary_dim >> 1;
        const float *cs = p.rope_cos + (int64_t)c_app * half;
        const float *sn = p.rope_sin + (int64_t)c_app * half;
        const int nvec = owner ? G + 1 : G;
        for (int i = tid; i < nvec * half; i += kMapThreads) {
            int h = i / half, j = i - h * half;
            float *x = sm_vec + h * D;
            float c = cs[j], s = sn[j];
            float x0 = x[j], x1 = x[j + half];
            x[j] = x0 * c - x1 * s;
            x[j + half] = x0 * s + x1 * c;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[h][c * 8 + e] = qs[h * D + 64 * c + 8 * cb + e];
        if (owner) {
            const int64_t off = row_offset(c_app);
            uint16_t *kd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.k)) + off;
            uint16_t *vd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.v)) + off;
            const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(p.v_new) + ((int64_t)b * p.Hkv + g) * D;
            for (int i = tid; i < D; i += kMapThreads) {
                kd[i] = E::from_float(ks[i]);
                vd[i] = vsrc[i];
            }
            __threadfence();
        }
        __syncthreads();
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
        if constexpr (MODE == kAppend) {
            const bool owner = (t_begin <= c_app) && (c_app < t_begin + p.chunk);
            if (owner) {
                const int64_t off = row_offset(c_app);
                uint16_t *kd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.k)) + off;
                uint16_t *vd = reinterpret_cast<uint16_t *>(const_cast<char *>(p.v)) + off;
                const uint16_t *ksrc = reinterpret_cast<const uint16_t *>(p.k_new) + ((int64_t)b * p.Hkv + g) * D;
                const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(p.v_new) + ((int64_t)b * p.Hkv + g) * D;
                for (int i = tid; i < D; i += kMapThreads) {
                    kd[i] = ksrc[i];
                    vd[i] = vsrc[i];
                }
                __threadfence();
            }
            __syncthreads();
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

    const int ntok = t_end - t_begin;
    const int ntiles = ntok > 0 ? (ntok + TT - 1) / TT : 0;
    // tiles wv, wv + 4, wv + 8, ... of this split belong to wave wv (wave-uniform values)
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int n_my = ntiles > wvu ? (ntiles - wvu + kMapWaves - 1) / kMapWaves : 0;
    const char *kbase = p.k;
    const char *vbase = p.v;
    const uint32_t tok_bytes = (uint32_t)(p.s_token * 2);

    struct Tile {
        uint4 k[NR][NCH];
        uint4 v[NR][NCH];
    };
    auto tile_t0 = [&](int i) { return t_begin + (wvu + i * kMapWaves) * TT; };

    // Per-lane byte offsets of this lane's rows within a tile: loop-invariant,
    // except in the split's last tile, whose rows past t_end clamp to its last
    // valid row (their scores are masked later).
    const int last_t0 = t_begin + (ntiles - 1) * TT;
    const int nvalid_last = t_end - last_t0;
    uint32_t off_full[NR], off_last[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        off_full[j] = (uint32_t)(8 * j + ra) * tok_bytes + (uint32_t)cb * 16u;
        off_last[j] = (uint32_t)min(8 * j + ra, nvalid_last - 1) * tok_bytes + (uint32_t)cb * 16u;
    }

    // Issue the loads of the tile starting at token t0.
    auto issue = [&](Tile &T, int t0) {
        const int64_t base = row_offset(t0);
        const char *kb = kbase + base * 2;
        const char *vb = vbase + base * 2;
        const bool last = (t0 == last_t0);
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const uint32_t off = last ? off_last[j] : off_full[j];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                T.k[j][c] = *reinterpret_cast<const uint4 *>(kb + off + c * 128);
                T.v[j][c] = *reinterpret_cast<const uint4 *>(vb + off + c * 128);
            }
        }
    };

    auto compute = [&](const Tile &T, int t0) {
        const int nvalid = t_end - t0;
        float sc[NR][G];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const uint32_t *kw = reinterpret_cast<const uint32_t *>(&T.k[j][0]);
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
                sc[j][h] = sum8(s) * p.scale_log2;
            }
        }
        if (nvalid < TT) {  // only a split's last tile is partial (wave-uniform branch)
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (8 * j + ra >= nvalid) sc[j][h] = kNegInf;
        }
        float mx[G];
        bool move = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mx[h] = sc[0][h];
#pragma unroll
            for (int j = 1; j < NR; ++j) mx[h] = fmaxf(mx[h], sc[j][h]);
            tmax[h] = fmaxf(tmax[h], mx[h]);
            move |= mx[h] > m[h] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(move) != 0) {  // rare after the first tiles
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mn = fmaxf(m[h], mx[h]);
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
            const uint32_t *vw = reinterpret_cast<const uint32_t *>(&T.v[j][0]);
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

    if (n_my > 0) {
        // NBUF register tiles rotate: while one is computed, the next NBUF - 1
        // are in flight (under load the memory latency is about two tiles'
        // compute time). Loads are unconditional -- indices past the end
        // re-issue the last tile -- so every wait count in the loop is static.
        Tile T[NBUF];
        const int last = n_my - 1;
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) issue(T[u], tile_t0(min(u, last)));
        int i = 0;
        for (; i + NBUF <= n_my; i += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                issue(T[(u + NBUF - 1) % NBUF], tile_t0(min(i + u + NBUF - 1, last)));
                compute(T[u], tile_t0(i + u));
            }
        }
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u)
            if (i + u < n_my) compute(T[u], tile_t0(i + u));
    }

    // ---------------------------------------------------------------- merge lane rows, then waves
#pragma unroll
    for (int step = 8; step <= 32; step <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = shfl_xor(m[h], step);
            const float lo = shfl_xor(l[h], step);
            tmax[h] = fmaxf(tmax[h], shfl_xor(tmax[h], step));
            const float mn = fmaxf(m[h], mo);
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
    if (ra == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm_acc[wv][h][64 * c + 8 * cb + e] = acc[h][8 * c + e];
            if (cb == 0) {
                sm_m[wv][h] = m[h];
                sm_l[wv][h] = l[h];
                sm_t[wv][h] = tmax[h];
            }
        }
    }
    __syncthreads();

    // Block state per head, re-expressed against the true maximum T of the split:
    // O~ = sum_w 2^(m_w - T) acc_w, d = sum_w 2^(m_w - T) l_w (each factor <= 2^kTau).
    const int64_t slot = p.s_offset + split;
    for (int i = tid; i < G * D; i += kMapThreads) {
        const int h = i / D, d = i - h * D;
        float T = sm_t[0][h];
#pragma unroll
        for (int w = 1; w < kMapWaves; ++w) T = fmaxf(T, sm_t[w][h]);
        float o = 0.0f, lsum = 0.0f;
        if (T != kNegInf) {
#pragma unroll
            for (int w = 0; w < kMapWaves; ++w) {
                const float a = fexp2(sm_m[w][h] - T);
                o += a * sm_acc[w][h][d];
                lsum += a * sm_l[w][h];
            }
        }
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        p.po[(bh * p.s_total + slot) * D + d] = o;
        if (d == 0) {
            p.pm[bh * p.s_total + slot] = (T == kNegInf) ? kNegInf : T * kLn2;
            p.pd[bh * p.s_total + slot] = lsum;
        }
    }

    if (p.counters == nullptr) return;

    // ---------------------------------------------------------------- single-kernel merge
    // Publish this block's states device-wide and count arrivals per
    // (request, KV head); the last block to arrive merges all splits (in split
    // order, with the merge kernel's code) and resets the counter.
    __syncthreads();  // every wave's state stores are complete
    if (tid == 0) {
        int *cnt = p.counters + (int64_t)b * p.Hkv + g;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (int)gridDim.x - 1);
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_flag = last;
    }
    __syncthreads();
    if (!sm_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int h = wv; h < G; h += kMapWaves) {
        const int64_t bh = (int64_t)b * p.Hq + hq0 + h;
        merge_states_wave<D>(p.po + bh * p.s_total * D, p.pm + bh * p.s_total, p.pd + bh * p.s_total,
                             p.s_total, p.out + bh * D, p.lse ? p.lse + bh : nullptr, lane);
    }
}

template <int DT, int D, int G, bool PAGED, int MODE>
static hipError_t launch_t(const MapParams &p, int S, hipStream_t st) {
    dim3 grid(S, p.Hkv, p.B);
    hipLaunchKernelGGL((map_kernel<DT, D, G, PAGED, MODE>), grid, dim3(kMapThreads), 0, st, p);
    return hipGetLastError();
}

template <int DT, int D, int G, bool PAGED>
static hipError_t launch_mode(const MapParams &p, int S, hipStream_t st) {
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
    if (p.head_dim == 128)
        return p.dtype == 0 ? launch_g<0, 128>(p, num_splits, st) : launch_g<1, 128>(p, num_splits, st);
    if (p.head_dim == 64)
        return p.dtype == 0 ? launch_g<0, 64>(p, num_splits, st) : launch_g<1, 64>(p, num_splits, st);
    return hipErrorInvalidValue;
}

}  // namespace fdec
