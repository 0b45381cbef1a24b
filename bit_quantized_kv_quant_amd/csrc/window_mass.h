// Per-key probability mass from a block of observation-window rows: the
// arithmetic of selective flash attention's second pass (gptget.net summary of
// arXiv 2411.18077, 方法详解: a second kernel turns the logits into importance
// without storing a T x T matrix).  Shared by the stand-alone pass
// (window_scores.hip) and the single-pass variant that runs inside pass 1
// (prefill.hip), so both give the same bits for the same inputs.
#pragma once

#include "common.h"

namespace minikv {
namespace wmass {

constexpr float kLog2e = 1.4426950408889634f;

// K^T operand of key block kt0: lane holds k[kt0 + lane % 32][16 kk + 8 half + 0..7]
// (rows past the buffer's end read as zeros through the buffer resource).
template <int D>
__device__ __forceinline__ void load_kblock(__amdgpu_buffer_rsrc_t rk, int kt0, int lane, bf16x8 (&kreg)[D / 16]) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        kreg[kk] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ((kt0 + (lane & 31)) * D + 16 * kk + 8 * (lane >> 5)) * 2, 0, 0));
}

// Mass of the keys of block kt0 from 32 window rows starting at row0, given
// their Q operand (qa: lane holds q[row0 + lane % 32][16 kk + 8 half + 0..7])
// and the lane's 16 row log-sum-exps in the log2 domain (l2[e] for row
// row0 + 8 (e / 4) + 4 half + e % 4; +inf for rows past the window).  S = Q K^T
// puts one key per accumulator column, so the lane's sum covers 16 rows; the
// caller adds the other lane half.
template <int D>
__device__ __forceinline__ float block_mass(const bf16x8 (&qa)[D / 16], const bf16x8 (&kreg)[D / 16], const float (&l2)[16],
                                            float scale_log2, int row0, int kt0, int lane) {
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kreg[kk], sacc, 0, 0, 0);
    const int half = lane >> 5;
    const int j = kt0 + (lane & 31);
    float acc = 0.0f;
    if (kt0 + 31 <= row0) {  // every window row of the block sees every key of the block
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += exp2f(fmaf(sacc[e], scale_log2, -l2[e]));
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = row0 + 8 * (e >> 2) + 4 * half + (e & 3);
            if (j <= i) acc += exp2f(fmaf(sacc[e], scale_log2, -l2[e]));
        }
    }
    return acc;
}

// Q operand of window rows w0 + 32 rb + (lane % 32), zero past the window.
template <int D>
__device__ __forceinline__ void load_qrows(const uint16_t* __restrict__ q, size_t qbase, int w0, int W, int rb, int lane,
                                           bf16x8 (&qa)[D / 16]) {
    const int half = lane >> 5;
    const int r = 32 * rb + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qa[kk] = r < W ? *reinterpret_cast<const bf16x8*>(q + (qbase + w0 + r) * D + 16 * kk + 8 * half) : bf16x8{};
}

// Window row of accumulator element e of this lane, relative to the row block.
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

}  // namespace wmass
}  // namespace minikv
