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
// gfx950 design: a workgroup of 8 waves owns 256 query rows (32 per wave) and
// streams 64-key tiles of K and V through two LDS stages (XOR-swizzled 16-byte
// chunks, register-prefetched one tile ahead for V and two for K; one barrier
// per tile).  Workgroups are ordered XCD-aware so the K/V prefix a head's query
// blocks share stays in one L2.  Each wave software-pipelines its tiles: the
// QK^T MFMAs of tile t+1 are issued while the softmax of tile t runs.  Each wave computes S^T = K Q^T with
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
constexpr int kXcds = 8;                    // MI355X: 8 XCDs of 32 CUs, each with its own L2
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
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int B_,
    int T_ctx, int Hq, int Hkv, int nqb, float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse) {
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

    // XCD-aware order: workgroup L is dispatched to XCD L % 8.  Work item W =
    // (L % 8) * per + L / 8 gives each XCD a contiguous run of (sequence, head)
    // pairs, all query blocks of a head back to back (longest first), so the
    // K/V prefix a head's blocks re-read stays in that XCD's L2.
    const int nwork = nqb * Hq * B_;
    const int per = (nwork + kXcds - 1) / kXcds;
    const int W = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (W >= nwork) return;
    const int hs = W / nqb;
    const int qb = nqb - 1 - W % nqb;
    const int b = hs / Hq;
    const int h = hs % Hq;
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

    // K tiles are register-staged (global -> VGPR -> LDS, XOR-swizzled 16-byte
    // chunks).  Loads go through a buffer resource based at the tile's first
    // row and sized to the rows that exist: rows past T read as zeros, and such
    // keys sit only in diagonal tiles, where they are masked.  (A
    // global_load_lds path would skip the VGPR hop, but the compiler then waits
    // for every outstanding load before any LDS read.)
    u32x4 pk[LOADS];
    // Row and chunk of the first 16-byte chunk this thread stages; its later
    // chunks are kRowStep rows further down.
    const int row0 = (int)(threadIdx.x / CH);
    const int col0 = 8 * (int)(threadIdx.x % CH);
    constexpr int kRowStep = NT / CH;
    const int goff0 = (row0 * D + col0) * 2;  // byte offset of chunk 0 inside a tile
    auto tile_rsrc = [&](const uint16_t* base, int n0) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (kvbase + (size_t)n0) * D), 0,
                                                 (T_ctx - n0) * D * 2, 0x00020000);
    };
    auto load_k = [&](int n0) {
        const auto rk = tile_rsrc(k, n0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            pk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, goff0 + i * kRowStep * D * 2, 0, 0));
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = row0 + kRowStep * i, c = col0 / 8;
            *reinterpret_cast<u32x4*>(sK + buf * TILE + r * D + 8 * (c ^ swz_k<D>(r))) = pk[i];
        }
    };
    // V tiles are register-staged so they can be converted to fp16 on the way in.
    u32x4 pv[kWithO ? LOADS : 1];
    auto load_v = [&](int n0) {
        if constexpr (kWithO) {
            const auto rv = tile_rsrc(v, n0);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                pv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, goff0 + i * kRowStep * D * 2, 0, 0));
        }
    };

    auto store_v = [&](int buf) {
        if constexpr (kWithO) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int r = row0 + kRowStep * i, c = col0 / 8;
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

    // S^T = K Q^T of the tile in stage `buf`, one 32-key block at a time; a
    // block's K operands are all requested before its MFMA chain.
    auto qk = [&](int buf, f32x16 (&sacc)[2]) {
        const uint16_t* tk = sK + buf * TILE;
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
    };
    // Online softmax of one tile: returns the fp16 probabilities (PV operand)
    // and folds the fp32 row sum into lsum; rescales O when the reference max
    // moves.  Branch-free except the (rare, wave-uniform) rescale.
    auto softmax = [&](f32x16 (&sacc)[2], int n0, auto mask_tag, f16x8 (&pb)[2][2]) {
        constexpr bool kMask = decltype(mask_tag)::value;
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
        const float m_new = tm > m_ref + 8.0f ? tm : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 1 unless the max moved
        const bool moved = m_new != m_ref;
        m_ref = m_new;
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
        lsum = fmaf(lsum, alpha, psum);
        return moved;
    };
    // O^T += V^T P^T, one 32-wide block of the head dim at a time; the next
    // block's V^T operands are requested before this block's MFMAs.
    auto pv_mma = [&](int buf, const f16x8 (&pb)[2][2]) {
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
    };

    // Software pipeline over the key tiles of this wave: while the softmax of
    // tile t runs on the VALU, the QK^T MFMAs of tile t+1 are already issued
    // (they read the other K stage), then tile t's PV MFMAs follow.  K is staged
    // two tiles ahead, V one tile ahead.
    const int t_last = __builtin_amdgcn_readfirstlane(min(qw0 / kBN, ntiles - 1));  // wave-uniform
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    if (ntiles > 1) {
        load_k(kBN);
        store_k(1);
    }
    __syncthreads();
    f32x16 sacc[2];
    qk(0, sacc);
    for (int t = 0; t < ntiles; ++t) {
        const int n0 = t * kBN;
        const int buf = t & 1;
        if (t + 2 < ntiles) load_k(n0 + 2 * kBN);  // into registers; stored after this tile
        if (t + 1 < ntiles) load_v(n0 + kBN);
        if (t <= t_last) {
            f16x8 pb[2][2];
            bool moved;
            float m_old = m_ref;
            if (t < t_last) {
                f32x16 snext[2];
                qk(buf ^ 1, snext);
                moved = softmax(sacc, n0, std::false_type{}, pb);
                sacc[0] = snext[0];
                sacc[1] = snext[1];
            } else {
                moved = softmax(sacc, n0, std::true_type{}, pb);
            }
            if constexpr (kWithO) {
                if (__ballot(moved)) {  // wave-uniform, rare
                    const float alpha = __builtin_amdgcn_exp2f(m_old - m_ref);
#pragma unroll
                    for (int d = 0; d < DB; ++d)
#pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
                }
                pv_mma(buf, pb);
            }
        }
        // K(t)'s stage was consumed by the previous iteration's QK and V(t-1)'s
        // stage by the previous PV, so both are free: one barrier per tile.
        if (t + 2 < ntiles) store_k(buf);
        if (t + 1 < ntiles) store_v(buf ^ 1);
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
    const int nwork = nqb * Hq * B;
    const int grid = (nwork + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((fa_fwd_kernel<D, kWithO, WAVES>), dim3(grid), dim3(64 * WAVES), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), B, T_ctx, Hq, Hkv, nqb, sm_scale * kLog2e,
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
