// Heavy-hitter + recent-window token selection (adaptive KV policy): one
// 1024-thread workgroup per (sequence, KV head) row running the shared row
// selection (select_row.h, where the method and the rule are described).
#include "common.h"
#include "kernels.h"
#include "select_row.h"

namespace minikv {
namespace {

constexpr int kThreads = 1024;

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void select_topk_kernel(const float* __restrict__ scores, int T_ctx,
                                                              int n_heavy, int n_recent,
                                                              int32_t* __restrict__ idx) {
    __shared__ sel::Shared<kThreads> sh;
    const int row = blockIdx.x;
    sel::select_row<ITEMS, kThreads>(scores + (size_t)row * T_ctx, T_ctx, n_heavy, n_recent,
                                     idx + (size_t)row * (n_heavy + n_recent), sh);
}

template <int ITEMS>
hipError_t launch_items(const float* scores, int rows, int T_ctx, int n_heavy, int n_recent, int32_t* idx,
                        hipStream_t stream) {
    hipLaunchKernelGGL((select_topk_kernel<ITEMS>), dim3(rows), dim3(kThreads), 0, stream, scores, T_ctx,
                       n_heavy, n_recent, idx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select_topk(const float* scores, int B, int Hkv, int T_ctx, int n_heavy, int n_recent,
                              int32_t* idx, hipStream_t stream) {
    const int rows = B * Hkv;
    const int per = (T_ctx - n_recent + kThreads - 1) / kThreads;
    if (per <= 4) return launch_items<4>(scores, rows, T_ctx, n_heavy, n_recent, idx, stream);
    if (per <= 8) return launch_items<8>(scores, rows, T_ctx, n_heavy, n_recent, idx, stream);
    if (per <= 16) return launch_items<16>(scores, rows, T_ctx, n_heavy, n_recent, idx, stream);
    if (per <= 32) return launch_items<32>(scores, rows, T_ctx, n_heavy, n_recent, idx, stream);
    return launch_items<64>(scores, rows, T_ctx, n_heavy, n_recent, idx, stream);
}

}  // namespace minikv
