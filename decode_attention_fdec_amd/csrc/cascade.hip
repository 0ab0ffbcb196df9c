// Cascade shared-prefix kernel (matrix cores) for gfx950.
//
// Cascade attention (vLLM notes "FlashAttention 與 FlashInfer", design motivation:
// a prefix shared by the requests of a batch is computed once) splits each
// request's keys into the shared prefix and its own suffix. The suffix goes
// through the split-KV map kernel; this kernel produces the prefix's partial
// states (O~, m, d) for every query row at once -- the FlashDecoding map stage
// (lpnh.cn explainer §2 stage 1) over the prefix -- and the merge kernel then
// combines prefix and suffix states exactly (lpnh §2 stage 2). The block's code
// is cascade_prefix_body (cascade_prefix.h); with G = 4 its 4-wave form also runs
// as the prefix role of the single-launch cascade kernel (split_kv_mfma.hip),
// beside the balanced suffix blocks.
//
// With B requests and G query heads per KV head, the prefix sees R = B*G query
// rows per KV head (256 in the 64-request, 4:1 GQA workload): a real dense
// contraction, so it runs on MFMA (v_mfma_f32_16x16x32_{bf16,f16}). Grid
// (prefix split, KV head, 256-row chunk); 8 waves, each owning 32 query rows
// (two 16-row blocks), two waves per SIMD so one's matrix work hides the
// other's softmax. Per 64-key tile:
//   - K and V go global -> LDS row-major by LDS-DMA (global_load_lds_dwordx4,
//     no registers), each wave its 8 rows, into a ring of kPfxNS tiles (two in
//     flight; the first goes out beside the query loads, so the block's start
//     waits for one memory round trip, not two); 16-byte pieces of row r sit in slot piece ^ (r mod 16), so the
//     K reads below and the transpose reads of V touch distinct banks;
//   - S^T = K Q^T: A = K (16 keys x 32 d from LDS), B = Q^T (query rows held in
//     registers), so each lane's result column is one query row and its four
//     values are four keys of that row;
//   - online softmax per row in the log2 domain (lazily moved reference as in the
//     map kernel; the scale enters with the reference in one FMA per score, and
//     the row maximum is taken over raw scores, then scaled: rounding is
//     monotone); P enters the matrix core rounded to the input type (hardware
//     nearest-even conversion), while the denominator sums the fp32 weights;
//   - O^T += V^T P^T: A = V^T from two ds_read_b64_tr_b16 of the row-major V
//     tile (4 keys at one d per lane each), B = P^T straight from the S^T
//     registers (the key order inside the K dimension is permuted identically
//     for A and B). Each lane's result column is then its own query row, so a
//     moved reference rescales O in the lane, and the states leave as 16-byte
//     stores of four consecutive d.
// Float8 pools (the pages' FP8 KV cache, e4m3fn with per-(request, KV head)
// descales): rows of 128 bytes, one DMA instruction per wave for its 8 rows of
// K and one for V; K pieces and V (by the 8-bit transpose read) widen to bf16
// in registers (exact), the K descale of each query row's request scales its
// scores and the V descale its state.
// Layout of v_mfma_f32_16x16x32 (lane l, kq = l / 16): A holds row l % 16,
// k = 8 kq .. 8 kq + 7; B holds column l % 16, k = 8 kq .. 8 kq + 7; D holds rows
// 4 kq .. 4 kq + 3 of column l % 16.
#include "cascade_prefix.h"

namespace fdec {

// The standalone prefix kernel: 8 waves (256 query rows), a 3-slot ring (two
// tiles in flight; four measured no faster).
constexpr int kPfxKernelWaves = 8;
constexpr int kPfxKernelSlots = 3;

template <int DT, int KF>
__global__ __launch_bounds__(64 * kPfxKernelWaves, 1) void cascade_prefix_kernel(const CascadeParams p) {
    __shared__ PfxLds<KF, kPfxKernelSlots> sm;
    cascade_prefix_body<DT, KF, kPfxKernelWaves, kPfxKernelSlots>(p, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

hipError_t launch_cascade_prefix(const CascadeParams &p, int splits, hipStream_t st) {
    const int R = p.B * (p.Hq / p.Hkv);
    constexpr int kRows = kPfxKernelWaves * kPfxRowsPerWave;
    dim3 grid(splits, p.Hkv, (R + kRows - 1) / kRows);
    if (p.kv_fp8) {
        if (p.dtype != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((cascade_prefix_kernel<1, 1>), grid, dim3(64 * kPfxKernelWaves), 0, st, p);
    } else if (p.dtype == 0) {
        hipLaunchKernelGGL((cascade_prefix_kernel<0, 0>), grid, dim3(64 * kPfxKernelWaves), 0, st, p);
    } else {
        hipLaunchKernelGGL((cascade_prefix_kernel<1, 0>), grid, dim3(64 * kPfxKernelWaves), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace fdec
