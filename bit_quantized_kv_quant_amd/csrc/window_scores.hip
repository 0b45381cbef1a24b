// Selective flash attention, pass 2 (the "second kernel"): per-key importance.
//
// Method: gptget.net summary of arXiv 2411.18077, 方法详解 (selective flash
// attention realised with a second kernel, keeping memory low) and 术语表
// "adaptive KV" (importance-based retention).  For KV head g:
//   score[j] = sum_{h in group(g)} sum_{i = T-W}^{T-1} [j <= i] exp(q_i . k_j * scale - lse_h[i])
// i.e. the softmax probability mass key j receives from the W observation rows,
// recomputed from the logits and pass 1's per-row lse, never stored as a matrix.
//
// gfx950 design: a wave owns 32 keys and holds them as the B operand of
// S = Q_window K^T (bf16 MFMA 32x32x16), so an accumulator column is one key:
// the sum over window rows is a per-lane sum plus one permlane32 swap.  K is
// read from HBM once; the window queries (W x D per head) and their lse come
// from L2.  Summation order is fixed, so the scores are deterministic.
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(256) void window_scores_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const float* __restrict__ lse, int T_ctx, int Hq,
                                                            int Hkv, int W, float scale_log2,
                                                            float* __restrict__ scores) {
    constexpr int KS = D / 16;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int R = Hq / Hkv;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int kt0 = (blockIdx.x * 4 + wave) * 32;
    if (kt0 >= T_ctx) return;
    const int j = kt0 + (lane & 31);
    const size_t kvbase = ((size_t)b * Hkv + g) * T_ctx;
    const int w0 = T_ctx - W;  // first window row

    // K^T operand: lane holds k[j][16 kk + 8 half + 0..7]
    bf16x8 kreg[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
        kreg[kk] = (j < T_ctx) ? *reinterpret_cast<const bf16x8*>(k + (kvbase + j) * D + 16 * kk + 8 * half)
                               : bf16x8{};

    float acc = 0.0f;
    const int nrb = (W + 31) / 32;
    for (int r = 0; r < R; ++r) {
        const int h = g * R + r;
        const size_t qbase = ((size_t)b * Hq + h) * T_ctx;
        for (int rb = 0; rb < nrb; ++rb) {
            // rows of this block whose last key is below kt0 contribute nothing
            const int row0 = w0 + 32 * rb;
            if (row0 + 31 < kt0) continue;
            const int qrow = row0 + (lane & 31);
            const bool qvalid = 32 * rb + (lane & 31) < W;
            f32x16 sacc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const bf16x8 a = qvalid ? *reinterpret_cast<const bf16x8*>(q + (qbase + qrow) * D + 16 * kk + 8 * half)
                                        : bf16x8{};
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kreg[kk], sacc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = 8 * (e >> 2) + 4 * half + (e & 3);  // accumulator row = window row in block
                const int i = row0 + m;
                if (32 * rb + m < W && j <= i) {
                    const float l2 = lse[qbase + i] * kLog2e;
                    acc += exp2f(fmaf(sacc[e], scale_log2, -l2));
                }
            }
        }
    }
    acc += swap_halves(acc);
    if (half == 0 && j < T_ctx) scores[kvbase + j] = acc;
}

template <int D>
hipError_t launch_ws(const void* q, const void* k, const float* lse, int B, int T_ctx, int Hq, int Hkv, int W,
                     float sm_scale, float* scores, hipStream_t stream) {
    const int nkb = (T_ctx + 127) / 128;
    hipLaunchKernelGGL((window_scores_kernel<D>), dim3(nkb, Hkv, B), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), lse, T_ctx, Hq, Hkv, W,
                       sm_scale * kLog2e, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_window_scores(const void* q, const void* k, const float* lse, int B, int T_ctx, int Hq,
                                int Hkv, int D, int window, float sm_scale, float* scores,
                                hipStream_t stream) {
    if (D == 128) return launch_ws<128>(q, k, lse, B, T_ctx, Hq, Hkv, window, sm_scale, scores, stream);
    return launch_ws<64>(q, k, lse, B, T_ctx, Hq, Hkv, window, sm_scale, scores, stream);
}

}  // namespace minikv
