// Streaming decode: tokens into the exact residual window.
//
// Method: gptget.net summary of arXiv 2411.18077, 方法论 / 方法详解 (keys are
// quantised per channel over groups of tokens, so a key group needs whole
// groups of tokens; the cache layout is compact).  The packed region holds whole
// 32-token groups; the kept tokens that do not fill a group, and the tokens
// generated after them, wait unquantised in a residual window of 32 slots per
// (sequence, KV head) until 32 are there, when the window is packed as the next
// group (stream pack = quantise-and-pack at a group offset of a fixed-capacity
// layout).  This file copies tokens into the window and, for a generation
// step whose counts live in device memory (so that a fixed launch sequence can
// be captured in a HIP graph and replayed), writes and advances those counts.
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

// One wave per (sequence, KV head): rows idx[j] (or j) of the head's T rows of
// k and v go to residual slots slot + j, j < n.  Lane l moves dword l of each
// row (D / 2 dwords of bf16 pairs: all 64 lanes for D = 128, 32 for D = 64).
// With counts (device int32 {n_packed, n_res, overflow}) the slot is n_res,
// read on the device, and nothing is written once the cache has overflowed.
template <int D>
__global__ __launch_bounds__(64) void stream_append_kernel(const uint32_t* __restrict__ k,
                                                           const uint32_t* __restrict__ v,
                                                           const int32_t* __restrict__ idx, int idx_stride,
                                                           int T_ctx, int n, int slot, uint32_t* __restrict__ k_res,
                                                           uint32_t* __restrict__ v_res,
                                                           const int32_t* __restrict__ counts) {
    constexpr int W = D / 2;  // dwords per row
    const int unit = blockIdx.x;
    const int lane = threadIdx.x;
    if (counts) {
        if (counts[2] != 0) return;
        slot = counts[1];
    }
    if (lane >= W || slot < 0 || slot + n > kGroup) return;
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

// Counts after one appended token: the window grows, and a full window has
// been packed as the next group (by the pack launched before this) unless the
// capacity is exhausted, which sets the overflow flag and keeps the window.
__global__ __launch_bounds__(64) void stream_advance_kernel(int32_t* __restrict__ counts, int cap) {
    if (threadIdx.x != 0 || counts[2] != 0) return;
    const int r = counts[1] + 1;
    if (r < kGroup) {
        counts[1] = r;
    } else if (counts[0] + kGroup <= cap) {
        counts[0] += kGroup;
        counts[1] = 0;
    } else {
        counts[2] = 1;
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
                         int n, int slot, void* k_res, void* v_res, const int32_t* counts, hipStream_t stream) {
    hipLaunchKernelGGL((stream_append_kernel<D>), dim3(B * Hkv), dim3(64), 0, stream, static_cast<const uint32_t*>(k),
                       static_cast<const uint32_t*>(v), idx, idx_stride, T_ctx, n, slot,
                       static_cast<uint32_t*>(k_res), static_cast<uint32_t*>(v_res), counts);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_append(const void* k, const void* v, const int32_t* idx, int idx_stride, int B, int Hkv,
                                int T_ctx, int D, int n, int slot, void* k_res, void* v_res, hipStream_t stream) {
    if (D == 128) return launch_append<128>(k, v, idx, idx_stride, B, Hkv, T_ctx, n, slot, k_res, v_res, nullptr, stream);
    return launch_append<64>(k, v, idx, idx_stride, B, Hkv, T_ctx, n, slot, k_res, v_res, nullptr, stream);
}

hipError_t launch_stream_set_counts(int32_t* counts, int n_packed, int n_res, hipStream_t stream) {
    hipLaunchKernelGGL(stream_set_counts_kernel, dim3(1), dim3(64), 0, stream, counts, n_packed, n_res);
    return hipGetLastError();
}

hipError_t launch_stream_step_append(const void* k_new, const void* v_new, int B, int Hkv, int D, int cap,
                                     int32_t* counts, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes,
                                     uint32_t* v_sz, void* k_res, void* v_res, hipStream_t stream) {
    // 1. the token into window slot n_res
    hipError_t e = D == 128 ? launch_append<128>(k_new, v_new, nullptr, 1, B, Hkv, 1, 1, 0, k_res, v_res, counts, stream)
                            : launch_append<64>(k_new, v_new, nullptr, 1, B, Hkv, 1, 1, 0, k_res, v_res, counts, stream);
    if (e != hipSuccess) return e;
    // 2. the window as group n_packed / 32 when this token filled it (decided on the device)
    e = launch_stream_pack_counted(k_res, v_res, B, Hkv, D, cap, counts, k_codes, k_sz, v_codes, v_sz, stream);
    if (e != hipSuccess) return e;
    // 3. the counts
    hipLaunchKernelGGL(stream_advance_kernel, dim3(1), dim3(64), 0, stream, counts, cap);
    return hipGetLastError();
}

}  // namespace minikv
