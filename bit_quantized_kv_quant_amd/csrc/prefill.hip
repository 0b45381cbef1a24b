// Selective flash attention, pass 1: causal attention with per-row log-sum-exp.
//
// Method: paper-listing abstract (kernels that keep the 2-bit cache compatible
// with FlashAttention) and gptget.net summary, 方法详解 (selective flash
// attention built from a second kernel, memory kept low).  This pass computes
//   o[i]   = sum_{j<=i} softmax_j(q_i . k_j * scale) v_j
//   lse[i] = log sum_{j<=i} exp(q_i . k_j * scale)
// in one sweep over the keys with an online softmax; the second kernel
// (window_scores.hip) reuses lse to turn the last rows' logits into
// probabilities without storing any T x T matrix.
//
// gfx950 design: a workgroup of 4 waves owns 128 query rows (32 per wave) and
// streams 64-key tiles of K and V through LDS (XOR-swizzled 16-byte chunks,
// register-prefetched one tile ahead).  Each wave computes S^T = K Q^T with
// bf16 MFMA 32x32x16, so an accumulator column is one query: a lane owns the
// softmax state (running max, partial sum) of its query, and the row max needs
// one permlane32 swap.  P^T is already in the B-operand layout of the second
// product O^T = V^T P^T; the V^T operand comes straight from the row-major V
// tile with ds_read_b64_tr_b16 (LDS transpose read).  The key order inside a
// 32-key block is permuted (phys) so that accumulator register v of a lane is
// key 16*half + v, which makes both operand layouts line up without shuffles.
// Causal: tiles above the diagonal are never loaded; only tiles that cross it
// apply the mask.  Query blocks are issued longest-first.
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// logical accumulator row r of a 32-key block -> physical key within the block
__device__ __forceinline__ int phys_key(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// XOR swizzles of the 16-byte chunk index inside a 256-byte (D = 128) row:
// K rows are read 32 rows x one chunk at a time, V rows 4 rows x 4 chunks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return ((r & 7) | (((r >> 4) & 1) << 3)) & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    return (4 * (r & 3)) & (D / 8 - 1);
}

template <int D, bool kWithO>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int T_ctx, int Hq,
                                                         int Hkv, float scale_log2, __bf16* __restrict__ o,
                                                         float* __restrict__ lse) {
    constexpr int CH = D / 8;           // 16-byte chunks per row
    constexpr int KS = D / 16;          // MFMA k-steps over the head dim
    constexpr int DB = D / 32;          // 32-wide output blocks over the head dim
    constexpr int LOADS = kBN * CH / 256;  // 16-byte chunks per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kWithO ? kBN * D : 8];

    const int nqb = gridDim.x;
    const int qb = nqb - 1 - blockIdx.x;  // longest rows first
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int q0 = qb * kBM;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int qw0 = q0 + 32 * wave;
    const int qi = qw0 + (lane & 31);

    const size_t qbase = ((size_t)b * Hq + h) * T_ctx;
    const size_t kvbase = ((size_t)b * Hkv + g) * T_ctx;

    // Q^T operand: lane holds q[qi][16 kk + 8 half + 0..7]
    bf16x8 qreg[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (qi < T_ctx)
            qreg[kk] = *reinterpret_cast<const bf16x8*>(q + (qbase + qi) * D + 16 * kk + 8 * half);
        else
            qreg[kk] = bf16x8{};
    }

    const int kv_end = min(T_ctx, q0 + kBM);  // keys this workgroup needs
    const int ntiles = (kv_end + kBN - 1) / kBN;

    // tile loader: thread -> (row, chunk) pairs
    u32x4 pk[LOADS], pv[kWithO ? LOADS : 1];
    auto load_tile = [&](int n0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = threadIdx.x + 256 * i;
            const int r = e / CH, c = e % CH;
            const int j = n0 + r;
            if (j < T_ctx) {
                pk[i] = *reinterpret_cast<const u32x4*>(k + (kvbase + j) * D + 8 * c);
                if constexpr (kWithO) pv[i] = *reinterpret_cast<const u32x4*>(v + (kvbase + j) * D + 8 * c);
            } else {
                pk[i] = u32x4{0, 0, 0, 0};
                if constexpr (kWithO) pv[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = threadIdx.x + 256 * i;
            const int r = e / CH, c = e % CH;
            *reinterpret_cast<u32x4*>(sK + r * D + 8 * (c ^ swz_k<D>(r))) = pk[i];
            if constexpr (kWithO) {
                f16x8 h;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    h[2 * w] = (_Float16)__uint_as_float(pv[i][w] << 16);
                    h[2 * w + 1] = (_Float16)__uint_as_float(pv[i][w] & 0xFFFF0000u);
                }
                *reinterpret_cast<f16x8*>(sV + r * D + 8 * (c ^ swz_v<D>(r))) = h;
            }
        }
    };

    float m = -INFINITY;  // running max of the log2-domain logits of this lane's query
    float lsum = 0.0f;    // partial sum over this lane's half of the keys
    f32x16 oacc[kWithO ? DB : 1];
#pragma unroll
    for (int d = 0; d < (kWithO ? DB : 1); ++d) oacc[d] = f32x16{};

    // per-lane constant parts of the LDS addresses
    const int krow_l = phys_key(lane & 31);
    const int grp = lane >> 4;         // 16-lane group of the transpose read
    const int tj = (lane & 15) >> 2;   // row inside the 4-row transpose block
    const int tc = lane & 3;           // 4-element column chunk

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int n0 = t * kBN;
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(n0 + kBN);

        if (n0 <= qw0 + 31) {  // this wave has unmasked keys in the tile (n0 <= qw0 then)
            f32x16 sacc[2];
#pragma unroll
            for (int bk = 0; bk < 2; ++bk) {
                sacc[bk] = f32x16{};
                const int r = 32 * bk + krow_l;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const int c = 2 * kk + half;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + r * D + 8 * (c ^ swz_k<D>(r)));
                    sacc[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[bk], 0, 0, 0);
                }
            }
            const bool diag = n0 + kBN - 1 > qw0;  // some key in the tile lies above the diagonal
            float tmax = -INFINITY;
#pragma unroll
            for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float s = sacc[bk][e] * scale_log2;
                    if (diag && n0 + 32 * bk + 16 * half + e > qi) s = -INFINITY;
                    sacc[bk][e] = s;
                    tmax = fmaxf(tmax, s);
                }
            }
            tmax = fmaxf(tmax, swap_halves(tmax));
            const float m_new = fmaxf(m, tmax);
            const float alpha = exp2f(m - m_new);
            m = m_new;
            float psum = 0.0f;
            f16x8 pb[2][2];
#pragma unroll
            for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = exp2f(sacc[bk][e] - m_new);
                    psum += p;
                    pb[bk][e >> 3][e & 7] = (_Float16)p;
                }
            }
            lsum = fmaf(lsum, alpha, psum);
            if constexpr (kWithO) {
#pragma unroll
                for (int d = 0; d < DB; ++d)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
#pragma unroll
                for (int d = 0; d < DB; ++d) {
                    const int col = 32 * d + 16 * (grp & 1) + 4 * tc;  // element column this lane supplies
#pragma unroll
                    for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            const int kb = 32 * bk + 16 * (grp >> 1) + 8 * s;
                            const int r0 = kb + tj, r1 = kb + 4 + tj;
                            const uint16_t* p0 = sV + r0 * D + 8 * ((col >> 3) ^ swz_v<D>(r0)) + (col & 7);
                            const uint16_t* p1 = sV + r1 * D + 8 * ((col >> 3) ^ swz_v<D>(r1)) + (col & 7);
                            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(p0));
                            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(p1));
                            const i16x4 both[2] = {lo, hi};
                            f16x8 a;
                            __builtin_memcpy(&a, both, 16);
                            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[bk][s], oacc[d], 0, 0, 0);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    const float ltot = lsum + swap_halves(lsum);
    if (qi < T_ctx) {
        if (half == 0) lse[qbase + qi] = (m + __log2f(ltot)) * kLn2;
        if constexpr (kWithO) {
            const float inv = 1.0f / ltot;
#pragma unroll
            for (int d = 0; d < DB; ++d) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[d][4 * a4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(o + (qbase + qi) * D + 32 * d + 8 * a4 + 4 * half) = w;
                }
            }
        }
    }
}

template <int D, bool kWithO>
hipError_t launch_fa(const void* q, const void* k, const void* v, int B, int T_ctx, int Hq, int Hkv,
                     float sm_scale, void* o, float* lse, hipStream_t stream) {
    const int nqb = (T_ctx + kBM - 1) / kBM;
    hipLaunchKernelGGL((fa_fwd_kernel<D, kWithO>), dim3(nqb, Hq, B), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), T_ctx, Hq, Hkv, sm_scale * kLog2e,
                       static_cast<__bf16*>(o), lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const void* q, const void* k, const void* v, int B, int T_ctx, int Hq, int Hkv,
                          int D, float sm_scale, void* o, float* lse, hipStream_t stream) {
    if (D == 128) {
        if (o) return launch_fa<128, true>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, stream);
        return launch_fa<128, false>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, stream);
    }
    if (o) return launch_fa<64, true>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, stream);
    return launch_fa<64, false>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, stream);
}

}  // namespace minikv
