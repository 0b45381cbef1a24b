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
// streams 64-key tiles of K and V through two LDS stages (XOR-swizzled 16-byte
// chunks, register-prefetched; one barrier per tile).  Each wave computes S^T = K Q^T with
// bf16 MFMA 32x32x16, so an accumulator column is one query: a lane owns the
// softmax state (running max, partial sum) of its query, and the row max needs
// one permlane32 swap.  P^T is already in the B-operand layout of the second
// product O^T = V^T P^T; the V^T operand comes straight from the row-major V
// tile with ds_read_b64_tr_b16 (LDS transpose read).  The key order inside a
// 32-key block is permuted (phys) so that accumulator register v of a lane is
// key 16*half + v, which makes both operand layouts line up without shuffles.
// Causal: tiles above the diagonal are never loaded; only tiles that cross it
// apply the mask.  Query blocks are issued longest-first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

#ifndef MINIKV_FA_WAVES
#define MINIKV_FA_WAVES 8
#endif
constexpr int kFaWaves = MINIKV_FA_WAVES;  // waves per workgroup, 32 query rows each
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

template <int D, bool kWithO, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int T_ctx,
    int Hq, int Hkv, float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse) {
    constexpr int NT = 64 * WAVES;          // threads
    constexpr int BM = 32 * WAVES;          // query rows per workgroup
    constexpr int CH = D / 8;               // 16-byte chunks per row
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int DB = D / 32;              // 32-wide output blocks over the head dim
    constexpr int LOADS = kBN * CH / NT;    // V chunks per thread per tile
    constexpr int TILE = kBN * D;           // elements of one staged tile
    // two LDS stages: tile t is read from one while tile t+1 is written to the other
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kWithO ? 2 * TILE : 8];

    const int nqb = gridDim.x;
    const int qb = nqb - 1 - blockIdx.x;  // longest rows first
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int q0 = qb * BM;
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

    const int kv_end = min(T_ctx, q0 + BM);  // keys this workgroup needs
    const int ntiles = (kv_end + kBN - 1) / kBN;

    // K tiles go global -> LDS directly (global_load_lds_dwordx4: lane l of an
    // instruction fills the l-th 16-byte slot of a 1 KB run); the lane fetches the
    // chunk that belongs in its slot under the XOR swizzle.  Rows past the end
    // are clamped to the last row: those keys are always masked.
    auto dma_k = [&](int n0, int buf) {
        constexpr int kInstr = kBN * CH / kWave / WAVES;  // per wave
#pragma unroll
        for (int i = 0; i < kInstr; ++i) {
            const int run = WAVES * i + wave;
            const int sidx = run * kWave + lane;
            const int r = sidx / CH, pc = sidx % CH;
            const int j = min(n0 + r, T_ctx - 1);
            const uint16_t* src = k + (kvbase + j) * D + 8 * (pc ^ swz_k<D>(r));
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(sK + buf * TILE + run * kWave * 8),
                                             16, 0, 0);
        }
    };
    // V tiles are register-staged so they can be converted to fp16 on the way in.
    u32x4 pv[kWithO ? LOADS : 1];
    auto load_v = [&](int n0) {
        if constexpr (kWithO) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int e = threadIdx.x + NT * i;
                const int r = e / CH, c = e % CH;
                const int j = min(n0 + r, T_ctx - 1);
                pv[i] = *reinterpret_cast<const u32x4*>(v + (kvbase + j) * D + 8 * c);
            }
        }
    };
    auto store_v = [&](int buf) {
        if constexpr (kWithO) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int e = threadIdx.x + NT * i;
                const int r = e / CH, c = e % CH;
                f16x8 hv;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    hv[2 * w] = (_Float16)__uint_as_float(pv[i][w] << 16);
                    hv[2 * w + 1] = (_Float16)__uint_as_float(pv[i][w] & 0xFFFF0000u);
                }
                *reinterpret_cast<f16x8*>(sV + buf * TILE + r * D + 8 * (c ^ swz_v<D>(r))) = hv;
            }
        }
    };

    // Softmax state of this lane's query, log2 domain.  m_ref is the reference
    // max the probabilities are taken against; it moves only when a tile's max
    // exceeds it by more than 8, so p <= 2^8 and the accumulators are rescaled
    // rarely (the result does not depend on m_ref).
    float m_ref = -INFINITY;
    float lsum = 0.0f;  // partial sum over this lane's half of the keys
    f32x16 oacc[kWithO ? DB : 1];
#pragma unroll
    for (int d = 0; d < (kWithO ? DB : 1); ++d) oacc[d] = f32x16{};

    // Per-lane LDS offsets (elements).  K operand of k-step kk, key block bk:
    // koff[kk] + 32 bk D.  V^T operand of head-dim block d, key block bk, half
    // s, rows +0 / +4: voff[d] + (32 bk + 8 s + 4 hi) D.  The swizzle terms are
    // lane constants, so only these few offsets live in registers.
    const int krow = phys_key(lane & 31);
    int koff[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) koff[kk] = krow * D + 8 * ((2 * kk + half) ^ swz_k<D>(krow));
    const int grp = lane >> 4;        // 16-lane group of the transpose read
    const int tj = (lane & 15) >> 2;  // row inside the 4-row transpose block
    const int tc = lane & 3;          // 4-element column chunk
    int voff[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d)
        voff[d] = (16 * (grp >> 1) + tj) * D + 8 * (4 * (d ^ (tj & (DB - 1))) + 2 * (grp & 1) + (tc >> 1)) +
                  4 * (tc & 1);

    auto process = [&](int buf, int n0, auto mask_tag) {
        constexpr bool kMask = decltype(mask_tag)::value;
        const uint16_t* tk = sK + buf * TILE;
        // S^T = K Q^T, one 32-key block at a time; the block's K operands are
        // all requested before its MFMA chain so LDS latency overlaps
        f32x16 sacc[2];
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
            bf16x8 a[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                a[kk] = *reinterpret_cast<const bf16x8*>(tk + koff[kk] + 32 * bk * D);
            sacc[bk] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                sacc[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], qreg[kk], sacc[bk], 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if constexpr (kMask) {
                    if (n0 + 32 * bk + 16 * half + e > qi) sacc[bk][e] = -INFINITY;
                }
                tmax = fmaxf(tmax, sacc[bk][e]);
            }
        }
        const float tm = fmaxf(tmax, swap_halves(tmax)) * scale_log2;
        const bool need = tm > m_ref + 8.0f;
        if (__ballot(need)) {  // wave-uniform
            const float m_new = need ? tm : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            lsum *= alpha;
            if constexpr (kWithO) {
#pragma unroll
                for (int d = 0; d < DB; ++d)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
            }
            m_ref = m_new;
        }
        // probabilities: fp32 for the row sum (it defines lse, which the second
        // kernel turns back into probabilities), fp16 for the PV operand
        f16x8 pb[2][2];
        float psum = 0.0f;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[bk][e], scale_log2, -m_ref));
                psum += p;
                pb[bk][e >> 3][e & 7] = (_Float16)p;
            }
        }
        lsum += psum;
        if constexpr (kWithO) {
            // O^T += V^T P^T, one 32-wide block of the head dim at a time; the
            // next block's V^T operands are requested before this block's MFMAs
            // (the scheduling barrier keeps the compiler from hoisting more).
            const _Float16* tv = reinterpret_cast<const _Float16*>(sV + buf * TILE);
            auto read_v = [&](int d, f16x8 (&av)[2][2]) {
#pragma unroll
                for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const _Float16* p0 = tv + voff[d] + (32 * bk + 8 * s) * D;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(p0));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(p0 + 4 * D));
                        const i16x4 both[2] = {lo, hi};
                        __builtin_memcpy(&av[bk][s], both, 16);
                    }
                }
            };
            f16x8 va[2][2][2];
            read_v(0, va[0]);
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                if (d + 1 < DB) read_v(d + 1, va[(d + 1) & 1]);
#pragma unroll
                for (int bk = 0; bk < 2; ++bk)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[d & 1][bk][s], pb[bk][s], oacc[d], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    dma_k(0, 0);
    load_v(0);
    store_v(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int n0 = t * kBN;
        const int buf = t & 1;
        const bool more = t + 1 < ntiles;
        if (more) {  // next tile into the other stage while this one is consumed
            dma_k(n0 + kBN, buf ^ 1);
            load_v(n0 + kBN);
        }
        if (n0 <= qw0 + 31) {  // the wave has unmasked keys in this tile (then n0 <= qw0)
            if (n0 + kBN - 1 > qw0)
                process(buf, n0, std::true_type{});
            else
                process(buf, n0, std::false_type{});
        }
        if (more) store_v(buf ^ 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    const float ltot = lsum + swap_halves(lsum);
    if (qi < T_ctx) {
        if (half == 0) lse[qbase + qi] = (m_ref + __log2f(ltot)) * kLn2;
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
    constexpr int WAVES = kFaWaves;
    const int nqb = (T_ctx + 32 * WAVES - 1) / (32 * WAVES);
    hipLaunchKernelGGL((fa_fwd_kernel<D, kWithO, WAVES>), dim3(nqb, Hq, B), dim3(64 * WAVES), 0, stream,
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
