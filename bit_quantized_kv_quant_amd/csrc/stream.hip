// Streaming decode: tokens into the exact residual window.
//
// Method: gptget.net summary of arXiv 2411.18077, 方法论 / 方法详解 (keys are
// quantised per channel over groups of tokens, so a key group needs whole
// groups of tokens; the cache layout is compact).  The packed region holds whole
// 32-token groups; the kept tokens that do not fill a group, and the tokens
// generated after them, wait unquantised in a residual window of 32 slots per
// (sequence, KV head) until 32 are there, when the window is packed as the next
// group (stream pack = quantise-and-pack at a group offset of a fixed-capacity
// layout).  This file copies tokens into the window and writes the device-side
// counts of a generation step (the step's append itself, which packs the window
// when it fills, is in quant_pack.hip).
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

// One wave per (sequence, KV head): rows idx[j] (or j) of the head's T rows of
// k and v go to residual slots slot + j, j < n.  Lane l moves dword l of each
// row (D / 2 dwords of bf16 pairs: all 64 lanes for D = 128, 32 for D = 64).
template <int D>
__global__ __launch_bounds__(64) void stream_append_kernel(const uint32_t* __restrict__ k,
                                                           const uint32_t* __restrict__ v,
                                                           const int32_t* __restrict__ idx, int idx_stride,
                                                           int T_ctx, int n, int slot, uint32_t* __restrict__ k_res,
                                                           uint32_t* __restrict__ v_res) {
    constexpr int W = D / 2;  // dwords per row
    const int unit = blockIdx.x;
    const int lane = threadIdx.x;
    if (lane >= W) return;
    const uint32_t* kr = k + (size_t)unit * T_ctx * W;
    const uint32_t* vr = v + (size_t)unit * T_ctx * W;
    uint32_t* kd = k_res + ((size_t)unit * kGroup + slot) * W;
    uint32_t* vd = v_res + ((size_t)unit * kGroup + slot) * W;
    for (int j = 0; j < n; ++j) {
        const int pos = idx ? idx[(size_t)unit * idx_stride + j] : j;
        kd[(size_t)j * W + lane] = kr[(size_t)pos * W + lane];
        vd[(size_t)j * W + lane] = vr[(size_t)pos * W + lane];
    }
}

__global__ __launch_bounds__(64) void stream_set_counts_kernel(int32_t* __restrict__ counts, int n_packed, int n_res) {
    if (threadIdx.x == 0) {
        counts[0] = n_packed;
        counts[1] = n_res;
        counts[2] = 0;
        counts[3] = 0;
    }
}

template <int D>
hipError_t launch_append(const void* k, const void* v, const int32_t* idx, int idx_stride, int B, int Hkv, int T_ctx,
                         int n, int slot, void* k_res, void* v_res, hipStream_t stream) {
    hipLaunchKernelGGL((stream_append_kernel<D>), dim3(B * Hkv), dim3(64), 0, stream, static_cast<const uint32_t*>(k),
                       static_cast<const uint32_t*>(v), idx, idx_stride, T_ctx, n, slot,
                       static_cast<uint32_t*>(k_res), static_cast<uint32_t*>(v_res));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_append(const void* k, const void* v, const int32_t* idx, int idx_stride, int B, int Hkv,
                                int T_ctx, int D, int n, int slot, void* k_res, void* v_res, hipStream_t stream) {
    if (D == 128) return launch_append<128>(k, v, idx, idx_stride, B, Hkv, T_ctx, n, slot, k_res, v_res, stream);
    return launch_append<64>(k, v, idx, idx_stride, B, Hkv, T_ctx, n, slot, k_res, v_res, stream);
}

hipError_t launch_stream_set_counts(int32_t* counts, int n_packed, int n_res, hipStream_t stream) {
    hipLaunchKernelGGL(stream_set_counts_kernel, dim3(1), dim3(64), 0, stream, counts, n_packed, n_res);
    return hipGetLastError();
}


}  // namespace minikv
