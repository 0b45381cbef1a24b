// Selective flash attention, pass 2 (the "second kernel"): per-key importance.
//
// Method: gptget.net summary of arXiv 2411.18077, 方法详解 (selective flash
// attention realised with a second kernel, keeping memory low) and 术语表
// "adaptive KV" (importance-based retention).  For KV head g:
//   score[j] = sum_{h in group(g)} sum_{i = T-W}^{T-1} [j <= i] exp(q_i . k_j * scale - lse_h[i])
// i.e. the softmax probability mass key j receives from the W observation rows,
// recomputed from the logits and pass 1's per-row lse, never stored as a matrix.
//
// gfx950 design: a wave walks a run of blocks of 32 keys, each held as the B operand
// of S = Q_window K^T (bf16 MFMA 32x32x16), so an accumulator column is one key:
// the sum over window rows is a per-lane sum plus one permlane32 swap.  K is
// read from HBM once, the next block's K loaded while the current one is
// reduced; for one query head and a window of up to 32 rows the Q operand and
// the row lse stay in registers, for up to four (query head, row block) sets
// they are staged once per workgroup in LDS; with more sets the keys stay in
// registers and the sets stream through LDS (window_scores_rows_kernel).
// Summation order is fixed, so the scores are deterministic.
#include "common.h"
#include "kernels.h"
#include "window_mass.h"

namespace minikv {
namespace {

using wmass::block_mass;
using wmass::kLog2e;
using wmass::load_kblock;

template <int D>
__device__ __forceinline__ void load_qblock(const uint16_t* __restrict__ q, const float* __restrict__ lse, size_t qbase,
                                            int w0, int W, int rb, int lane, bf16x8 (&qa)[D / 16], float (&l2)[16]) {
    wmass::load_qrows<D>(q, qbase, w0, W, rb, lane, qa);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int m = 32 * rb + wmass::acc_row(e, lane);
        l2[e] = m < W ? lse[qbase + w0 + m] * kLog2e : INFINITY;
    }
}

constexpr int kMaxStaged = 4;  // (query head, row block) operand sets a workgroup can keep in LDS

// grid (ceil(T / (128 nbw)), Hkv, B), 4 waves; wave w owns the nbw key blocks
// from (blockIdx.x * 4 + w) * nbw (nbw even).  kMode 0: one query head per KV
// head and a window of at most 32 rows (Q operand and row lse in registers);
// 1: at most kMaxStaged (query head, row block) pairs, staged once per
// workgroup in LDS in the operand layout.  More sets: window_scores_rows_kernel.
template <int D, int kMode>
__global__ __launch_bounds__(256, 3) void window_scores_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const float* __restrict__ lse, int T_ctx, int Hq,
                                                               int Hkv, int W, int nbw, float scale_log2,
                                                               float* __restrict__ scores) {
    constexpr int KS = D / 16;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int R = Hq / Hkv;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int kb0 = (blockIdx.x * 4 + wave) * nbw;
    const size_t kvbase = ((size_t)b * Hkv + g) * T_ctx;
    const int w0 = T_ctx - W;  // first window row
    const int nrb = (W + 31) / 32;

    // [set][kk][lane] Q operands and [set][row] lse * log2(e) of the staged sets
    __shared__ bf16x8 s_q[kMode == 1 ? kMaxStaged * KS * kWave : 1];
    __shared__ float s_l2[kMode == 1 ? kMaxStaged * 32 : 1];
    if constexpr (kMode == 1) {
        const int nset = R * nrb;
        for (int c = threadIdx.x; c < nset * 32 * (D / 8); c += 256) {  // coalesced 16-byte chunks
            const int set = c / (32 * (D / 8)), m = (c / (D / 8)) % 32, ch = c % (D / 8);
            const int r = set / nrb, row = 32 * (set % nrb) + m;
            const size_t qbase = ((size_t)b * Hq + g * R + r) * T_ctx;
            s_q[(set * KS + (ch >> 1)) * kWave + ((ch & 1) << 5 | m)] =
                row < W ? *reinterpret_cast<const bf16x8*>(q + (qbase + w0 + row) * D + 8 * ch) : bf16x8{};
        }
        for (int c = threadIdx.x; c < nset * 32; c += 256) {
            const int set = c / 32, r = set / nrb, row = 32 * (set % nrb) + c % 32;
            s_l2[c] = row < W ? lse[((size_t)b * Hq + g * R + r) * T_ctx + w0 + row] * kLog2e : INFINITY;
        }
        __syncthreads();
    }
    if (kb0 * 32 >= T_ctx) return;
    const int nb = min(nbw, (T_ctx - kb0 * 32 + 31) / 32);  // key blocks of this wave
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + kvbase * D), 0, T_ctx * D * 2, 0x00020000);
    auto emit = [&](int i, float a) {  // the block's per-key sums over the two lane halves
        a += swap_halves(a);
        const int j = (kb0 + i) * 32 + (lane & 31);
        if (half == 0 && j < T_ctx) scores[kvbase + j] = a;
    };

    bf16x8 ka[KS], kb[KS];
    load_kblock<D>(rk, kb0 * 32, lane, ka);
    if constexpr (kMode == 0) {
        // One query head, one row block: the Q operand and the row lse stay in
        // registers; K blocks stream through two register sets.
        bf16x8 qa[KS];
        float l2[16];
        load_qblock<D>(q, lse, ((size_t)b * Hq + g) * T_ctx, w0, W, 0, lane, qa, l2);
        for (int i = 0; i < nb; i += 2) {
            if (i + 1 < nb) load_kblock<D>(rk, (kb0 + i + 1) * 32, lane, kb);
            emit(i, block_mass<D>(qa, ka, l2, scale_log2, w0, (kb0 + i) * 32, lane));
            if (i + 2 < nb) load_kblock<D>(rk, (kb0 + i + 2) * 32, lane, ka);
            if (i + 1 < nb) emit(i + 1, block_mass<D>(qa, kb, l2, scale_log2, w0, (kb0 + i + 1) * 32, lane));
        }
    } else {
        // Per key block, every staged (query head, row block) set, operands from LDS.
        auto mass = [&](int i, const bf16x8 (&kr)[KS]) {
            const int kt0 = (kb0 + i) * 32;
            float a = 0.0f;
            for (int r = 0; r < R; ++r) {
                for (int rb = 0; rb < nrb; ++rb) {
                    const int row0 = w0 + 32 * rb;
                    if (row0 + 31 < kt0) continue;  // rows entirely before this key block
                    bf16x8 qa[KS];
                    float l2[16];
                    const int set = r * nrb + rb;
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) qa[kk] = s_q[(set * KS + kk) * kWave + lane];
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 t = *reinterpret_cast<const f32x4*>(s_l2 + set * 32 + 8 * g4 + 4 * half);
#pragma unroll
                        for (int e = 0; e < 4; ++e) l2[4 * g4 + e] = t[e];
                    }
                    a += block_mass<D>(qa, kr, l2, scale_log2, row0, kt0, lane);
                }
            }
            return a;
        };
        for (int i = 0; i < nb; i += 2) {
            if (i + 1 < nb) load_kblock<D>(rk, (kb0 + i + 1) * 32, lane, kb);
            emit(i, mass(i, ka));
            if (i + 2 < nb) load_kblock<D>(rk, (kb0 + i + 2) * 32, lane, ka);
            if (i + 1 < nb) emit(i + 1, mass(i + 1, kb));
        }
    }
}

// Many window rows (more (query head, row block) sets than a workgroup can
// keep, e.g. every prompt row for cumulative scores): the keys stay and the
// rows stream.  A workgroup owns a range of 8 key blocks (wave w: blocks 2w,
// 2w + 1, their K operands in registers) and walks the sets (query head
// outer, row block inner), staging each set's Q operand and row lse in LDS
// once for all four waves; a wave adds a set's mass for each of its blocks
// that the set's rows can see.  The summation order per key is the same as
// mode 1's, and ranges are paired (x, last - x) so every workgroup does about
// the same causal work.  grid (ceil(ranges / 2), Hkv, B).
template <int D>
__global__ __launch_bounds__(256) void window_scores_rows_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const float* __restrict__ lse, int T_ctx, int Hq,
                                                                 int Hkv, int W, int n_ranges, float scale_log2,
                                                                 float* __restrict__ scores) {
    constexpr int KS = D / 16;
    constexpr int KBW = 2;            // key blocks per wave
    constexpr int KR = 4 * KBW;       // key blocks per range
    constexpr int CPR = D / 8;        // 16-byte chunks per Q row
    __shared__ bf16x8 s_q[KS * kWave];
    __shared__ float s_l[32];
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int R = Hq / Hkv;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const size_t kvbase = ((size_t)b * Hkv + g) * T_ctx;
    const int w0 = T_ctx - W;
    const int nrb = (W + 31) / 32;
    const int nkb = (T_ctx + 31) / 32;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + kvbase * D), 0, T_ctx * D * 2, 0x00020000);
    for (int pass = 0; pass < 2; ++pass) {
        const int range = pass == 0 ? (int)blockIdx.x : n_ranges - 1 - (int)blockIdx.x;
        if (pass == 1 && range <= (int)blockIdx.x) break;  // workgroup-uniform
        const int kb_first = range * KR;
        bf16x8 kr[KBW][KS];
        float acc[KBW];
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            wmass::load_kblock<D>(rk, (kb_first + wave * KBW + i) * 32, lane, kr[i]);
            acc[i] = 0.0f;
        }
        for (int r = 0; r < R; ++r) {
            const size_t qbase = ((size_t)b * Hq + g * R + r) * T_ctx;
            for (int rb = 0; rb < nrb; ++rb) {
                const int row0 = w0 + 32 * rb;
                if (row0 + 31 < kb_first * 32) continue;  // rows before every key of the range
                __syncthreads();                          // the previous set is consumed
                for (int c = threadIdx.x; c < 32 * CPR; c += 256) {
                    const int m = c / CPR, cr = c % CPR;
                    const int row = 32 * rb + m;
                    s_q[(cr >> 1) * kWave + ((cr & 1) << 5 | m)] =
                        row < W ? *reinterpret_cast<const bf16x8*>(q + (qbase + w0 + row) * D + 8 * cr) : bf16x8{};
                }
                if (threadIdx.x < 32) {
                    const int row = 32 * rb + threadIdx.x;
                    s_l[threadIdx.x] = row < W ? lse[qbase + w0 + row] * kLog2e : INFINITY;
                }
                __syncthreads();
                bf16x8 qa[KS];
                float l2[16];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) qa[kk] = s_q[kk * kWave + lane];
#pragma unroll
                for (int e = 0; e < 16; ++e) l2[e] = s_l[wmass::acc_row(e, lane)];
#pragma unroll
                for (int i = 0; i < KBW; ++i) {
                    const int kb = kb_first + wave * KBW + i;
                    if (kb < nkb && row0 + 31 >= kb * 32)  // wave-uniform
                        acc[i] += block_mass<D>(qa, kr[i], l2, scale_log2, row0, kb * 32, lane);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const float a = acc[i] + swap_halves(acc[i]);
            const int j = (kb_first + wave * KBW + i) * 32 + (lane & 31);
            if (half == 0 && j < T_ctx) scores[kvbase + j] = a;
        }
    }
}

template <int D>
hipError_t launch_ws(const void* q, const void* k, const float* lse, int B, int T_ctx, int Hq, int Hkv, int W,
                     float sm_scale, float* scores, hipStream_t stream) {
    // Key blocks per wave: about one round of resident waves (256 CUs x 12),
    // even for the two-set K pipeline.
    const long long blocks = (long long)B * Hkv * ((T_ctx + 31) / 32);
    int nbw = (int)((blocks + 3071) / 3072);
    nbw = max(2, nbw + (nbw & 1));
    const int nwg = (T_ctx + 128 * nbw - 1) / (128 * nbw);
    const dim3 grid(nwg, Hkv, B);
    const auto qq = static_cast<const uint16_t*>(q);
    const auto kk = static_cast<const uint16_t*>(k);
    const float sl = sm_scale * kLog2e;
    const int sets = (Hq / Hkv) * ((W + 31) / 32);
    if (Hq == Hkv && W <= 32)
        hipLaunchKernelGGL((window_scores_kernel<D, 0>), grid, dim3(256), 0, stream, qq, kk, lse, T_ctx, Hq, Hkv, W, nbw, sl, scores);
    else if (sets <= kMaxStaged)
        hipLaunchKernelGGL((window_scores_kernel<D, 1>), grid, dim3(256), 0, stream, qq, kk, lse, T_ctx, Hq, Hkv, W, nbw, sl, scores);
    else {
        const int n_ranges = ((T_ctx + 31) / 32 + 7) / 8;
        hipLaunchKernelGGL((window_scores_rows_kernel<D>), dim3((n_ranges + 1) / 2, Hkv, B), dim3(256), 0, stream, qq,
                           kk, lse, T_ctx, Hq, Hkv, W, n_ranges, sl, scores);
    }
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
